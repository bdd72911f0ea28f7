// Decode (small batch) expert FFN and the fused decode layer: dequant GEMVs
// over the packed NVFP4 layout, W4A4.
//
// For each (token t, slot i), e = ids[t, i] (the release post "capy-flash
// v0.7.1": gate/up weights and down projections, section "What shipped";
// W4A4 path, section "Why it matters"):
//   g = W^_gate[e] x^_t, u = W^_up[e] x^_t, h = SiLU(g) * u
//   h^ = NVFP4(h) per (t, i) row, o[t, i] = W^_down[e] h^
//
// Arithmetic.  With A = E2M1 codes, s = E4M3 block scales and ts = tensor
// scales, a dot product is ts_w ts_x sum_b s_w,b sum_{k in b} A_w,k (A_x,k s_x,b).
// The activation factor A_x s_x is exact in f16 (at most 6 significant bits,
// range 2^-10 .. 2688) and so is the raw weight code A_w; v_dot2_f32_f16
// accumulates a block's 16 products exactly (they share s_x), the block sum
// is scaled by s_w in fp32 and summed over blocks in fp32; tensor scales
// multiply once at the end.
//
// Kernels.
//   gate/up   block = (pair p, 64-lane tile j, K-split s); each lane owns one
//             gate or up weight row, the activation is an LDS broadcast, so no
//             cross-lane reduction; waves split the block's K range and are
//             summed through LDS in a fixed order.  Writes raw partial dot
//             sums per K-split (no scales).  In the fused layer it first ranks
//             the router logits itself (every block the same, deterministic).
//   down      block = (pair p, 64-row tile j).  Issues its weight loads, then
//             finishes h from the gate/up partials (sum over splits, scales,
//             SiLU), quantizes it to NVFP4 (bit-exact quantizer) into LDS and
//             runs the down GEMV.  In the fused layer the last block to finish
//             a 64-column slice of every pair also does the weighted combine of
//             that slice (per-slice arrival counters, left at zero).
// The block of the first pair routed to an expert serves every pair routed
// to it, so each distinct expert's weights are read once per call.
#include "../../include/moe.h"
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int DEC_MAX_WAVES = 8;
constexpr int DEC_CPW = 10;            // chunks (32 elements) per wave held in registers

// ---------------------------------------------------------------- helpers
// Dequantize the NVFP4 activation row (codes, scales) to f16 A*s into LDS.
__device__ __forceinline__ void stage_act_f16(const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales, int K,
                                              half2_t* dst, int tid, int nthreads) {
  for (int b = tid; b < K / 16; b += nthreads) {
    u32x2 c = *reinterpret_cast<const u32x2*>(codes + b * 8);
    _Float16 s = (_Float16)e4m3_to_f32(scales[b]);
    half2_t s2 = {s, s};
    half2_t v[8];
    v[0] = fp4x2_to_f16x2<0>(c.x) * s2; v[1] = fp4x2_to_f16x2<1>(c.x) * s2;
    v[2] = fp4x2_to_f16x2<2>(c.x) * s2; v[3] = fp4x2_to_f16x2<3>(c.x) * s2;
    v[4] = fp4x2_to_f16x2<0>(c.y) * s2; v[5] = fp4x2_to_f16x2<1>(c.y) * s2;
    v[6] = fp4x2_to_f16x2<2>(c.y) * s2; v[7] = fp4x2_to_f16x2<3>(c.y) * s2;
    u32x4* d = reinterpret_cast<u32x4*>(dst + b * 8);
    d[0] = *reinterpret_cast<u32x4*>(&v[0]);
    d[1] = *reinterpret_cast<u32x4*>(&v[4]);
  }
}

// 16 weight codes (one u32x2 half of a lane's chunk) -> 8 f16x2
__device__ __forceinline__ void cvt16(uint32_t lo, uint32_t hi, half2_t (&w)[8]) {
  w[0] = fp4x2_to_f16x2<0>(lo); w[1] = fp4x2_to_f16x2<1>(lo);
  w[2] = fp4x2_to_f16x2<2>(lo); w[3] = fp4x2_to_f16x2<3>(lo);
  w[4] = fp4x2_to_f16x2<0>(hi); w[5] = fp4x2_to_f16x2<1>(hi);
  w[6] = fp4x2_to_f16x2<2>(hi); w[7] = fp4x2_to_f16x2<3>(hi);
}

// acc += s0 * <w[0:16], x[0:16]> + s1 * <w[16:32], x[16:32]> for one chunk.
__device__ __forceinline__ float chunk_dot(const half2_t (&w0)[8], const half2_t (&w1)[8],
                                           float s0, float s1, const half2_t* __restrict__ xs,
                                           float acc) {
  const u32x4* xp = reinterpret_cast<const u32x4*>(xs);
  u32x4 a0 = xp[0], a1 = xp[1], a2 = xp[2], a3 = xp[3];
  half2_t x[16];
  *reinterpret_cast<u32x4*>(&x[0]) = a0;
  *reinterpret_cast<u32x4*>(&x[4]) = a1;
  *reinterpret_cast<u32x4*>(&x[8]) = a2;
  *reinterpret_cast<u32x4*>(&x[12]) = a3;
  float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) b0 = dot2(w0[j], x[j], b0);
#pragma unroll
  for (int j = 0; j < 8; ++j) b1 = dot2(w1[j], x[8 + j], b1);
  acc = fmaf(s0, b0, acc);
  return fmaf(s1, b1, acc);
}

template <int CPW>
__device__ __forceinline__ void load_chunks(const uint8_t* __restrict__ tile, int K, int c0, int nc,
                                            int lane, u32x4 (&cw)[CPW], uint32_t (&sw)[CPW]) {
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    if (i < nc) {
      const int c = c0 + i;
      cw[i] = *reinterpret_cast<const u32x4*>(tile + (size_t)c * 1024 + lane * 16);
      sw[i] = *reinterpret_cast<const uint16_t*>(tile + tile_scale_offset(K) + (size_t)(c >> 2) * 512 + lane * 8 + (c & 3) * 2);
    }
  }
}

// acc[q] += dot of this lane's row slice with activation row q (LDS, f16 A*s)
template <int CPW, int MAXP>
__device__ __forceinline__ void dot_chunks(const u32x4 (&cw)[CPW], const uint32_t (&sw)[CPW], int c0,
                                           int nc, int n, const half2_t* __restrict__ act,
                                           int act_stride, float (&acc)[MAXP]) {
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    if (i < nc) {
      half2_t w0[8], w1[8];
      cvt16(cw[i].x, cw[i].y, w0);
      cvt16(cw[i].z, cw[i].w, w1);
      const float s0 = e4m3_to_f32(sw[i] & 0xFF), s1 = e4m3_to_f32(sw[i] >> 8);
#pragma unroll
      for (int q = 0; q < MAXP; ++q)
        if (q < n) acc[q] = chunk_dot(w0, w1, s0, s1, act + (size_t)q * act_stride + (c0 + i) * 16, acc[q]);
    }
  }
}

// Pairs of expert e from qstart on, at most MAXP; returns the count, writes
// them to list (thread 0) and the next unserved pair to *qnext.
template <int MAXP>
__device__ __forceinline__ int next_pairs(const int32_t* ids, int npairs, int e, int qstart,
                                          int* list, int* qnext, int tid) {
  int n = 0;
  *qnext = npairs;
  for (int q = qstart; q < npairs; ++q) {
    if (ids[q] != e) continue;
    if (n == MAXP) { *qnext = q; break; }
    if (tid == 0) list[n] = q;
    ++n;
  }
  return n;
}

// K-splits of the gate/up contraction: about 40 chunks (1280 elements) per block.
__host__ __device__ inline int dec_ksplit(int H) {
  const int nchunk = H / 32;
  const int ks = nchunk / 40;
  if (ks >= 4 && nchunk % 4 == 0) return 4;
  if (ks >= 2 && nchunk % 2 == 0) return 2;
  return 1;
}

__host__ __device__ inline int dec_waves(int nchunk_block) {
  int nw = (nchunk_block + DEC_CPW - 1) / DEC_CPW;
  return nw < 1 ? 1 : (nw > DEC_MAX_WAVES ? DEC_MAX_WAVES : nw);
}

struct DecodeWs {
  float* gu;          // [KS][T*k][2][I] raw gate/up partial dot sums
  int32_t* counters;  // [H/64] combine arrival counters (fused layer only)
};

// ---------------------------------------------------------------- gate/up
// TOPK: rank the router logits in-block first (fused layer), writing ids and
// w once (block 0,0,0); otherwise read ids.
template <int MAXP, int CPW, bool TOPK>
__global__ __launch_bounds__(64 * DEC_MAX_WAVES) void gate_up_decode_kernel(
    FfnArgs a, DecodeWs ws, const float* __restrict__ logits, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nw = blockDim.x >> 6;
  half2_t* xs = reinterpret_cast<half2_t*>(smem);                         // [MAXP][H/2]
  float* red = reinterpret_cast<float*>(smem + (size_t)MAXP * a.H * 2);   // [nw][MAXP][64]
  __shared__ int list[MAXP];
  __shared__ int sids[MOE_DECODE_MAX_T * MOE_MAX_K];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int npairs = a.T * a.k, p = blockIdx.x, j = blockIdx.y, split = blockIdx.z;
  const int KS = gridDim.z;
  const int32_t* ids;
  if (TOPK) {
    for (int t = wv; t < a.T; t += nw) {
      int id;
      float wt;
      topk_wave(logits + (size_t)t * a.E, a.E, a.k, lane, &id, &wt);
      if (lane < a.k) {
        sids[t * a.k + lane] = id;
        if (p == 0 && j == 0 && split == 0) {
          ids_out[t * a.k + lane] = id;
          w_out[t * a.k + lane] = wt;
        }
      }
    }
    __syncthreads();
    ids = sids;
  } else {
    ids = a.ids;
  }
  const int e = ids[p];
  for (int q = 0; q < p; ++q)
    if (ids[q] == e) return;                                  // another block owns e
  const size_t part_stride = (size_t)npairs * 2 * a.I;
  float* gu = ws.gu + (size_t)split * part_stride;
  if ((unsigned)e >= (unsigned)a.E) {                         // not an expert: partials 0
    for (int q = p; q < npairs; ++q)
      if (ids[q] == e && tid < 64) gu[(size_t)q * 2 * a.I + (tid >> 5) * a.I + 32 * j + (tid & 31)] = 0.0f;
    return;
  }
  const uint8_t* tile = a.gate_up + (size_t)e * gate_up_expert_bytes(a.H, a.I) + (size_t)j * tile_bytes(a.H);
  const int nchunk_b = a.H / 32 / KS;
  const int cpw = (nchunk_b + nw - 1) / nw;
  const int c0 = split * nchunk_b + wv * cpw;
  const int nc = max(0, min(cpw, nchunk_b - wv * cpw));
  u32x4 cw[CPW];
  uint32_t sw[CPW];
  load_chunks<CPW>(tile, a.H, c0, nc, lane, cw, sw);          // all weight loads in flight
  int qstart = p;
  while (true) {
    int qnext;
    const int n = next_pairs<MAXP>(ids, npairs, e, qstart, list, &qnext, tid);
    __syncthreads();
    for (int i = 0; i < n; ++i) {
      const int t = list[i] / a.k;
      stage_act_f16(a.x_codes + (size_t)t * (a.H / 2), a.x_scales + (size_t)t * (a.H / 16), a.H,
                    xs + (size_t)i * (a.H / 2), tid, blockDim.x);
    }
    __syncthreads();
    float acc[MAXP];
#pragma unroll
    for (int i = 0; i < MAXP; ++i) acc[i] = 0.0f;
    dot_chunks<CPW, MAXP>(cw, sw, c0, nc, n, xs, a.H / 2, acc);
#pragma unroll
    for (int i = 0; i < MAXP; ++i) red[(wv * MAXP + i) * 64 + lane] = acc[i];
    __syncthreads();
    if (wv == 0) {
      for (int i = 0; i < n; ++i) {
        float v = 0.0f;
        for (int w = 0; w < nw; ++w) v += red[(w * MAXP + i) * 64 + lane];
        // lane < 32: gate row 32j + lane; lane >= 32: up row 32j + lane - 32
        gu[(size_t)list[i] * 2 * a.I + (lane >> 5) * a.I + 32 * j + (lane & 31)] = v;
      }
    }
    if (qnext >= npairs) break;
    qstart = qnext;
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down
template <int MAXP, int CPW, bool COMBINE>
__global__ __launch_bounds__(64 * DEC_MAX_WAVES) void down_decode_kernel(
    FfnArgs a, DecodeWs ws, const float* __restrict__ w_comb, const uint16_t* __restrict__ residual,
    uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nw = blockDim.x >> 6;
  half2_t* hs = reinterpret_cast<half2_t*>(smem);                          // [MAXP][I/2]
  float* hrow = reinterpret_cast<float*>(smem + (size_t)MAXP * a.I * 2);   // [nw][I]
  float* red = hrow + (size_t)nw * a.I;                                    // [nw][MAXP][64]
  __shared__ int list[MAXP];
  __shared__ float hts[MAXP];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int npairs = a.T * a.k, p = blockIdx.x, j = blockIdx.y;
  const int KS = dec_ksplit(a.H);
  const int e = a.ids[p];
  for (int q = 0; q < p; ++q)
    if (a.ids[q] == e) return;
  int served = 0;
  if ((unsigned)e >= (unsigned)a.E) {                         // not an expert: o = 0
    for (int q = p; q < npairs; ++q)
      if (a.ids[q] == e) {
        if (tid < 64) a.out[(size_t)q * a.H + 64 * j + tid] = 0.0f;
        ++served;
      }
  } else {
    const uint8_t* tile = a.down + (size_t)e * down_expert_bytes(a.H, a.I) + (size_t)j * tile_bytes(a.I);
    const int nchunk = a.I / 32;
    const int cpw = (nchunk + nw - 1) / nw;
    const int c0 = wv * cpw;
    const int nc = max(0, min(cpw, nchunk - c0));
    u32x4 cw[CPW];
    uint32_t sw[CPW];
    load_chunks<CPW>(tile, a.I, c0, nc, lane, cw, sw);
    const int nblk = a.I / 16;
    const size_t part_stride = (size_t)npairs * 2 * a.I;
    int qstart = p;
    while (true) {
      int qnext;
      const int n = next_pairs<MAXP>(a.ids, npairs, e, qstart, list, &qnext, tid);
      __syncthreads();
      // h of pair i (wave i % nw): finish the dot products, SiLU-gate, then
      // NVFP4 with the row's own tensor scale
      for (int i = wv; i < n; i += nw) {
        const int q = list[i], t = q / a.k;
        const float sg = a.x_ts[t] * a.ts_gate[e], su = a.x_ts[t] * a.ts_up[e];
        float* hr = hrow + (size_t)wv * a.I;
        float amax = 0.0f;
        // all partial loads of a 640-column batch first, then the arithmetic
        constexpr int HB = 10;                                // columns per lane per batch
        for (int c0 = 0; c0 < a.I; c0 += 64 * HB) {
          float gp[HB][4], up[HB][4];
#pragma unroll
          for (int r = 0; r < HB; ++r) {
            const int c = c0 + lane + 64 * r;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              if (s < KS && c < a.I) {
                const float* part = ws.gu + (size_t)s * part_stride + (size_t)q * 2 * a.I;
                gp[r][s] = part[c];
                up[r][s] = part[a.I + c];
              }
            }
          }
#pragma unroll
          for (int r = 0; r < HB; ++r) {
            const int c = c0 + lane + 64 * r;
            if (c < a.I) {
              float g = gp[r][0], u = up[r][0];
#pragma unroll
              for (int s = 1; s < 4; ++s)
                if (s < KS) { g += gp[r][s]; u += up[r][s]; }
              g *= sg;
              u *= su;
              const float h = silu_mul(g, u);
              hr[c] = h;
              amax = fmaxf(amax, fabsf(h));
              if (j == 0 && a.dbg_h) a.dbg_h[(size_t)q * a.I + c] = h;
            }
          }
        }
        amax = dpp_wave_max(amax);
        const float ts = tensor_scale_from_amax(amax);
        wave_lds_sync();                                      // hr written by other lanes
        for (int b = lane; b < nblk; b += 64) {
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = hr[b * 16 + r];
          uint32_t pk[2];
          const uint32_t sb = quantize_block16(v, ts, pk);
          if (j == 0) {
            if (a.dbg_h_codes) *reinterpret_cast<u32x2*>(a.dbg_h_codes + (size_t)q * (a.I / 2) + b * 8) = u32x2{pk[0], pk[1]};
            if (a.dbg_h_scales) a.dbg_h_scales[(size_t)q * nblk + b] = (uint8_t)sb;
          }
          _Float16 s = (_Float16)e4m3_to_f32(sb);
          half2_t s2 = {s, s};
          half2_t w[8];
          cvt16(pk[0], pk[1], w);
          half2_t* d = hs + (size_t)i * (a.I / 2) + b * 8;
#pragma unroll
          for (int r = 0; r < 8; ++r) d[r] = w[r] * s2;
        }
        if (lane == 0) {
          hts[i] = ts;
          if (j == 0 && a.dbg_h_ts) a.dbg_h_ts[q] = ts;
        }
      }
      __syncthreads();
      float acc[MAXP];
#pragma unroll
      for (int i = 0; i < MAXP; ++i) acc[i] = 0.0f;
      dot_chunks<CPW, MAXP>(cw, sw, c0, nc, n, hs, a.I / 2, acc);
#pragma unroll
      for (int i = 0; i < MAXP; ++i) red[(wv * MAXP + i) * 64 + lane] = acc[i];
      __syncthreads();
      if (wv == 0) {
        for (int i = 0; i < n; ++i) {
          float v = 0.0f;
          for (int w = 0; w < nw; ++w) v += red[(w * MAXP + i) * 64 + lane];
          a.out[(size_t)list[i] * a.H + 64 * j + lane] = v * (hts[i] * a.ts_down[e]);
        }
      }
      served += n;
      if (qnext >= npairs) break;
      qstart = qnext;
      __syncthreads();
    }
  }
  if (COMBINE) {
    // the block that completes this 64-column slice for all pairs combines it
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int old = atomicAdd(ws.counters + j, served);
      last = (old + served == npairs);
    }
    __syncthreads();
    if (last) {
      __threadfence();
      for (int idx = tid; idx < a.T * 64; idx += blockDim.x) {
        const int t = idx / 64, c = 64 * j + (idx & 63);
        float acc = 0.0f;
        for (int i = 0; i < a.k; ++i)
          acc = fmaf(w_comb[t * a.k + i], __builtin_nontemporal_load(a.out + ((size_t)t * a.k + i) * a.H + c), acc);
        if (residual) acc += bf16_to_f32(residual[(size_t)t * a.H + c]);
        y[(size_t)t * a.H + c] = (uint16_t)f32_to_bf16_rne(acc);
      }
      if (tid == 0) ws.counters[j] = 0;                       // ready for the next call
    }
  }
}

// ---------------------------------------------------------------- router + x quant
// Fused layer, kernel 1: blocks 0..E-1 compute one router logit row each
// (all its weight loads issued first), blocks E.. quantize one token each.
__global__ __launch_bounds__(64) void router_quant_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ bias, int T, int E,
                                                          int H, float* __restrict__ logits,
                                                          uint8_t* __restrict__ xc,
                                                          uint8_t* __restrict__ xsc,
                                                          float* __restrict__ xts) {
  const int lane = threadIdx.x;
  const int blk = blockIdx.x;
  if (blk >= E) {
    const int t = blk - E;
    quantize_row_bf16_wave(x + (size_t)t * H, H, xc + (size_t)t * (H / 2), xsc + (size_t)t * (H / 16),
                           xts + t, lane);
    return;
  }
  constexpr int MAXF4 = 16;                                   // H <= 4096
  const int n4 = H / 256;
  float4_t wv[MAXF4];
  const float4_t* wr = reinterpret_cast<const float4_t*>(W + (size_t)blk * H);
#pragma unroll
  for (int i = 0; i < MAXF4; ++i)
    if (i < n4) wv[i] = wr[lane + 64 * i];
  const float be = bias ? bias[blk] : 0.0f;
  for (int t = 0; t < T; ++t) {
    const u32x2* xr = reinterpret_cast<const u32x2*>(x + (size_t)t * H);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXF4; ++i) {
      if (i < n4) {
        const u32x2 xb = xr[lane + 64 * i];
        acc = fmaf(wv[i].x, bf16_to_f32(xb.x & 0xFFFF), acc);
        acc = fmaf(wv[i].y, bf16_to_f32(xb.x >> 16), acc);
        acc = fmaf(wv[i].z, bf16_to_f32(xb.y & 0xFFFF), acc);
        acc = fmaf(wv[i].w, bf16_to_f32(xb.y >> 16), acc);
      }
    }
    const float v = dpp_wave_sum(acc);
    if (lane == 0) logits[(size_t)t * E + blk] = v + be;
  }
}

// ---------------------------------------------------------------- launchers
static size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(int E, int H, int I, int k, int T) {
  (void)E;
  return al256((size_t)dec_ksplit(H) * T * k * 2 * I * sizeof(float));
}

template <int MAXP, bool FUSED>
static void launch_decode_pair(const FfnArgs& a, DecodeWs ws, const float* logits, int32_t* ids_out,
                               float* w_out, const uint16_t* residual, uint16_t* y, hipStream_t s) {
  const int npairs = a.T * a.k;
  const int KS = dec_ksplit(a.H);
  const int nw1 = dec_waves(a.H / 32 / KS), nw2 = dec_waves(a.I / 32);
  const size_t lds1 = (size_t)MAXP * a.H * 2 + (size_t)nw1 * MAXP * 64 * 4;
  const size_t lds2 = (size_t)MAXP * a.I * 2 + (size_t)nw2 * a.I * 4 + (size_t)nw2 * MAXP * 64 * 4;
  const dim3 g1(npairs, a.I / 32, KS), g2(npairs, a.H / 64);
  gate_up_decode_kernel<MAXP, DEC_CPW, FUSED><<<g1, 64 * nw1, lds1, s>>>(a, ws, logits, ids_out, w_out);
  down_decode_kernel<MAXP, DEC_CPW, FUSED><<<g2, 64 * nw2, lds2, s>>>(a, ws, w_out, residual, y);
}

hipError_t launch_ffn_decode(const FfnArgs& a, void* ws, hipStream_t s) {
  DecodeWs w{reinterpret_cast<float*>(ws), nullptr};
  if (a.T == 1) launch_decode_pair<1, false>(a, w, nullptr, nullptr, nullptr, nullptr, nullptr, s);
  else launch_decode_pair<8, false>(a, w, nullptr, nullptr, nullptr, nullptr, nullptr, s);
  return hipGetLastError();
}

// Fused layer workspace: combine counters (first, so their offset does not
// depend on T), logits, x^ (codes, scales, ts), gate/up partials, o.  The
// counters must start at zero; every call leaves them at zero.
struct LayerWs {
  int32_t* counters; float* logits; int32_t* ids; float* w; uint8_t* xc; uint8_t* xs; float* xts;
  float* gu; float* out;
};

static LayerWs carve_layer(void* ws, int E, int H, int I, int k, int T, size_t* total) {
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  size_t off = 0;
  auto take = [&](size_t b) { uint8_t* q = p ? p + off : nullptr; off += al256(b); return q; };
  LayerWs w;
  w.counters = (int32_t*)take((size_t)(H / 64) * 4);
  w.logits = (float*)take((size_t)T * E * 4);
  w.ids = (int32_t*)take((size_t)T * k * 4);
  w.w = (float*)take((size_t)T * k * 4);
  w.xc = take((size_t)T * H / 2);
  w.xs = take((size_t)T * H / 16);
  w.xts = (float*)take((size_t)T * 4);
  w.gu = (float*)take(decode_workspace_bytes(E, H, I, k, T));
  w.out = (float*)take((size_t)T * k * H * 4);
  if (total) *total = off;
  return w;
}

size_t layer_decode_workspace_bytes(int E, int H, int I, int k, int T) {
  size_t total = 0;
  carve_layer(nullptr, E, H, I, k, T, &total);
  return total;
}

hipError_t launch_layer_decode(const LayerArgs& L, void* ws, hipStream_t s) {
  LayerWs w = carve_layer(ws, L.E, L.H, L.I, L.k, L.T, nullptr);
  router_quant_kernel<<<L.E + L.T, 64, 0, s>>>(L.x, L.W_r, L.bias, L.T, L.E, L.H, w.logits, w.xc, w.xs, w.xts);
  FfnArgs a{};
  a.E = L.E; a.H = L.H; a.I = L.I; a.k = L.k; a.T = L.T; a.fmt = FMT_NVFP4;
  a.gate_up = L.gate_up; a.down = L.down;
  a.ts_gate = L.ts_gate; a.ts_up = L.ts_up; a.ts_down = L.ts_down;
  a.x_codes = w.xc; a.x_scales = w.xs; a.x_ts = w.xts;
  int32_t* ids_out = L.ids_out ? L.ids_out : w.ids;
  float* w_out = L.w_out ? L.w_out : w.w;
  a.ids = ids_out;
  a.out = w.out;
  DecodeWs dw{w.gu, w.counters};
  const uint16_t* res = L.residual ? L.x : nullptr;
  if (L.T == 1)
    launch_decode_pair<1, true>(a, dw, w.logits, ids_out, w_out, res, L.y, s);
  else
    launch_decode_pair<8, true>(a, dw, w.logits, ids_out, w_out, res, L.y, s);
  return hipGetLastError();
}

}  // namespace moe
