// Decode expert FFN (small batch): fused dequant GEMVs over the packed NVFP4
// layout, W4A4.
//
// For each (token t, slot i), e = ids[t, i] (the release post "capy-flash
// v0.7.1": gate/up weights and down projections, section "What shipped";
// W4A4 path, section "Why it matters"):
//   g = W^_gate[e] x^_t, u = W^_up[e] x^_t, h = SiLU(g) * u      (kernel 1)
//   h^ = NVFP4(h) per (t, i) row, o[t, i] = W^_down[e] h^         (kernel 2)
//
// Arithmetic.  With A = E2M1 codes, s = E4M3 block scales and ts = tensor
// scales, a dot product is ts_w ts_x sum_b s_w,b sum_{k in b} A_w,k (A_x,k s_x,b).
// The activation factor A_x s_x is exact in f16 (at most 6 significant bits,
// range 2^-10 .. 2688) and so is the raw weight code A_w; v_dot2_f32_f16
// accumulates the 16 products of a block exactly (they share s_x), the block
// sum is scaled by s_w in fp32 and accumulated over blocks in fp32, and the
// tensor scales multiply once at the end.
//
// Work split: a block owns one distinct expert and one 64-lane weight tile
// (gate/up: 32 gate rows + the same 32 up rows; down: 64 rows); each lane owns
// one weight row, so the activation is a wave-uniform LDS broadcast and no
// cross-lane reduction is needed.  Waves of a block split the contraction
// axis and are reduced through LDS in a fixed order (deterministic).  Every
// distinct expert's weights are read once per call: the block of the first
// (t, i) pair routed to an expert serves all pairs routed to it.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int GU_WAVES = 4;
constexpr int DN_WAVES = 2;

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

// ---------------------------------------------------------------- gate/up
template <int MAXP>
__global__ __launch_bounds__(64 * GU_WAVES) void gate_up_decode_kernel(FfnArgs a, float* __restrict__ h_ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  half2_t* xs = reinterpret_cast<half2_t*>(smem);                         // [MAXP][H/2]
  float* red = reinterpret_cast<float*>(smem + (size_t)MAXP * a.H * 2);   // [GU_WAVES][MAXP][64]
  __shared__ int list[MAXP];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int npairs = a.T * a.k, p = blockIdx.x, j = blockIdx.y;
  const int e = a.ids[p];
  for (int q = 0; q < p; ++q)
    if (a.ids[q] == e) return;                                // another block owns e
  if ((unsigned)e >= (unsigned)a.E) {                         // not an expert: h = 0
    for (int q = p; q < npairs; ++q)
      if (a.ids[q] == e && tid < 32) {
        h_ws[(size_t)q * a.I + 32 * j + tid] = 0.0f;
        if (a.dbg_h) a.dbg_h[(size_t)q * a.I + 32 * j + tid] = 0.0f;
      }
    return;
  }
  const uint8_t* tile = a.gate_up + (size_t)e * gate_up_expert_bytes(a.H, a.I) + (size_t)j * tile_bytes(a.H);
  const int nchunk = a.H / 32;
  const int cpw = nchunk / GU_WAVES;                            // chunks per wave
  const int c0 = wv * cpw;
  int qstart = p;
  while (true) {
    // next batch of up to MAXP pairs of expert e, starting at qstart
    int n = 0;
    int qnext = npairs;
    for (int q = qstart; q < npairs; ++q) {
      if (a.ids[q] != e) continue;
      if (n == MAXP) { qnext = q; break; }
      if (tid == 0) list[n] = q;
      ++n;
    }
    __syncthreads();
    for (int i = 0; i < n; ++i) {
      const int t = list[i] / a.k;
      stage_act_f16(a.x_codes + (size_t)t * (a.H / 2), a.x_scales + (size_t)t * (a.H / 16), a.H,
                    xs + (size_t)i * (a.H / 2), tid, 64 * GU_WAVES);
    }
    __syncthreads();
    float acc[MAXP];
#pragma unroll
    for (int i = 0; i < MAXP; ++i) acc[i] = 0.0f;
    for (int c = c0; c < c0 + cpw; ++c) {
      u32x4 cw = *reinterpret_cast<const u32x4*>(tile + (size_t)c * 1024 + lane * 16);
      uint32_t sw = *reinterpret_cast<const uint16_t*>(tile + tile_scale_offset(a.H) + (size_t)(c >> 2) * 512 + lane * 8 + (c & 3) * 2);
      half2_t w0[8], w1[8];
      cvt16(cw.x, cw.y, w0);
      cvt16(cw.z, cw.w, w1);
      const float s0 = e4m3_to_f32(sw & 0xFF), s1 = e4m3_to_f32(sw >> 8);
#pragma unroll
      for (int i = 0; i < MAXP; ++i)
        if (i < n) acc[i] = chunk_dot(w0, w1, s0, s1, xs + (size_t)i * (a.H / 2) + c * 16, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < MAXP; ++i) red[(wv * MAXP + i) * 64 + lane] = acc[i];
    __syncthreads();
    if (wv == 0) {
      for (int i = 0; i < n; ++i) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < GU_WAVES; ++w) v += red[(w * MAXP + i) * 64 + lane];
        const float other = __shfl(v, (lane + 32) & 63, 64);       // up partner of a gate lane
        const int q = list[i], t = q / a.k;
        if (lane < 32) {
          const float g = v * (a.x_ts[t] * a.ts_gate[e]);
          const float u = other * (a.x_ts[t] * a.ts_up[e]);
          const float h = g / (1.0f + expf(-g)) * u;
          const int nrow = 32 * j + lane;
          h_ws[(size_t)q * a.I + nrow] = h;
          if (a.dbg_h) a.dbg_h[(size_t)q * a.I + nrow] = h;
        }
      }
    }
    if (qnext >= npairs) break;
    qstart = qnext;
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down
// Quantize-on-load: each block recomputes NVFP4(h) of its pairs' rows (a row
// is only I values); the tile-0 block also writes the optional debug copies.
template <int MAXP>
__global__ __launch_bounds__(64 * DN_WAVES) void down_decode_kernel(FfnArgs a, const float* __restrict__ h_ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  half2_t* hs = reinterpret_cast<half2_t*>(smem);                          // [MAXP][I/2]
  float* red = reinterpret_cast<float*>(smem + (size_t)MAXP * a.I * 2);    // [DN_WAVES][MAXP][64]
  __shared__ int list[MAXP];
  __shared__ float hts[MAXP];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int npairs = a.T * a.k, p = blockIdx.x, j = blockIdx.y;
  const int e = a.ids[p];
  for (int q = 0; q < p; ++q)
    if (a.ids[q] == e) return;
  if ((unsigned)e >= (unsigned)a.E) {                         // not an expert: o = 0
    for (int q = p; q < npairs; ++q)
      if (a.ids[q] == e && tid < 64) a.out[(size_t)q * a.H + 64 * j + tid] = 0.0f;
    return;
  }
  const uint8_t* tile = a.down + (size_t)e * down_expert_bytes(a.H, a.I) + (size_t)j * tile_bytes(a.I);
  const int nchunk = a.I / 32;
  const int cpw = nchunk / DN_WAVES;
  const int c0 = wv * cpw;
  const int nblk = a.I / 16;
  int qstart = p;
  while (true) {
    int n = 0;
    int qnext = npairs;
    for (int q = qstart; q < npairs; ++q) {
      if (a.ids[q] != e) continue;
      if (n == MAXP) { qnext = q; break; }
      if (tid == 0) list[n] = q;
      ++n;
    }
    __syncthreads();
    // quantize h rows: wave i%DN_WAVES handles pair i
    for (int i = wv; i < n; i += DN_WAVES) {
      const int q = list[i];
      const float* hr = h_ws + (size_t)q * a.I;
      float amax = 0.0f;
      for (int c = lane; c < a.I; c += 64) amax = fmaxf(amax, fabsf(hr[c]));
      amax = wave_max(amax);
      const float ts = tensor_scale_from_amax(amax);
      for (int b = lane; b < nblk; b += 64) {
        float v[16];
        const float4_t* src = reinterpret_cast<const float4_t*>(hr + b * 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float4_t f = src[r];
          v[4 * r] = f.x; v[4 * r + 1] = f.y; v[4 * r + 2] = f.z; v[4 * r + 3] = f.w;
        }
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
    for (int c = c0; c < c0 + cpw; ++c) {
      u32x4 cw = *reinterpret_cast<const u32x4*>(tile + (size_t)c * 1024 + lane * 16);
      uint32_t sw = *reinterpret_cast<const uint16_t*>(tile + tile_scale_offset(a.I) + (size_t)(c >> 2) * 512 + lane * 8 + (c & 3) * 2);
      half2_t w0[8], w1[8];
      cvt16(cw.x, cw.y, w0);
      cvt16(cw.z, cw.w, w1);
      const float s0 = e4m3_to_f32(sw & 0xFF), s1 = e4m3_to_f32(sw >> 8);
#pragma unroll
      for (int i = 0; i < MAXP; ++i)
        if (i < n) acc[i] = chunk_dot(w0, w1, s0, s1, hs + (size_t)i * (a.I / 2) + c * 16, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < MAXP; ++i) red[(wv * MAXP + i) * 64 + lane] = acc[i];
    __syncthreads();
    if (wv == 0) {
      for (int i = 0; i < n; ++i) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < DN_WAVES; ++w) v += red[(w * MAXP + i) * 64 + lane];
        const int q = list[i];
        a.out[(size_t)q * a.H + 64 * j + lane] = v * (hts[i] * a.ts_down[e]);
      }
    }
    if (qnext >= npairs) break;
    qstart = qnext;
    __syncthreads();
  }
}

size_t decode_workspace_bytes(int E, int H, int I, int k, int T) {
  (void)E; (void)H;
  return (size_t)T * k * I * sizeof(float);
}

hipError_t launch_ffn_decode(const FfnArgs& a, void* ws, hipStream_t s) {
  float* h = reinterpret_cast<float*>(ws);
  const int npairs = a.T * a.k;
  if (a.T == 1) {
    size_t lds1 = (size_t)1 * a.H * 2 + (size_t)GU_WAVES * 1 * 64 * 4;
    gate_up_decode_kernel<1><<<dim3(npairs, a.I / 32), 64 * GU_WAVES, lds1, s>>>(a, h);
    size_t lds2 = (size_t)1 * a.I * 2 + (size_t)DN_WAVES * 1 * 64 * 4;
    down_decode_kernel<1><<<dim3(npairs, a.H / 64), 64 * DN_WAVES, lds2, s>>>(a, h);
  } else {
    size_t lds1 = (size_t)8 * a.H * 2 + (size_t)GU_WAVES * 8 * 64 * 4;
    gate_up_decode_kernel<8><<<dim3(npairs, a.I / 32), 64 * GU_WAVES, lds1, s>>>(a, h);
    size_t lds2 = (size_t)8 * a.I * 2 + (size_t)DN_WAVES * 8 * 64 * 4;
    down_decode_kernel<8><<<dim3(npairs, a.H / 64), 64 * DN_WAVES, lds2, s>>>(a, h);
  }
  return hipGetLastError();
}

}  // namespace moe
