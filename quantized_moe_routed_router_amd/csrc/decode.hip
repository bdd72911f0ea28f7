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
//             summed through LDS in a fixed order.  Writes partial dot sums
//             per K-split with the tensor scales applied.  In the fused layer
//             it first ranks the router logits itself (every block the same,
//             deterministic).
//   h^        block = one pair: sums the K-splits, SiLU-gates, and quantizes
//             h to NVFP4 (bit-exact quantizer) once, for every down block.
//   down      block = 16 output columns of every pair (few pairs) or one
//             (pair, 64-row tile) (many pairs).  Issues its weight loads,
//             stages h^ into LDS as f16 and runs the down GEMV.  In the fused
//             layer the column-slice kernel also does the weighted combine of
//             its columns; with many pairs a separate combine kernel follows.
// The block of the first pair routed to an expert serves every pair routed
// to it, so each distinct expert's weights are read once per call (the
// column-slice down kernel reads an expert once per pair; duplicates only
// occur with several tokens and hit in cache).
#include "../../include/moe.h"
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int DEC_MAX_WAVES = 8;
static_assert(MOE_MAX_K <= TOPK_MAX_K, "top-k scratch holds MOE_MAX_K winners");
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

// The first XREG blocks per thread of a run of `total` 16-element activation
// blocks (rows contiguous), loaded into registers before the weight loads
// (straight-line: slots past the end re-read the last block) and written to
// LDS as f16 A*s after them, so the staging does not wait for the weights.
constexpr int XREG = 2;
struct ActRegs {
  u32x2 c[XREG];
  uint32_t s[XREG];
};
__device__ __forceinline__ void act_load(ActRegs& r, const uint8_t* __restrict__ codes,
                                         const uint8_t* __restrict__ scales, int total, int tid,
                                         int nthreads) {
#pragma unroll
  for (int i = 0; i < XREG; ++i) {
    const int b = min(tid + i * nthreads, total - 1);
    r.c[i] = *reinterpret_cast<const u32x2*>(codes + (size_t)b * 8);
    r.s[i] = scales[b];
  }
}
__device__ __forceinline__ void act_store(const ActRegs& r, const uint8_t* __restrict__ codes,
                                          const uint8_t* __restrict__ scales, int total,
                                          half2_t* dst, int tid, int nthreads) {
#pragma unroll
  for (int i = 0; i < XREG; ++i) {
    const int b = tid + i * nthreads;
    if (b < total) {
      const _Float16 s = (_Float16)e4m3_to_f32(r.s[i]);
      const half2_t s2 = {s, s};
      half2_t v[8];
      v[0] = fp4x2_to_f16x2<0>(r.c[i].x) * s2; v[1] = fp4x2_to_f16x2<1>(r.c[i].x) * s2;
      v[2] = fp4x2_to_f16x2<2>(r.c[i].x) * s2; v[3] = fp4x2_to_f16x2<3>(r.c[i].x) * s2;
      v[4] = fp4x2_to_f16x2<0>(r.c[i].y) * s2; v[5] = fp4x2_to_f16x2<1>(r.c[i].y) * s2;
      v[6] = fp4x2_to_f16x2<2>(r.c[i].y) * s2; v[7] = fp4x2_to_f16x2<3>(r.c[i].y) * s2;
      u32x4* d = reinterpret_cast<u32x4*>(dst + (size_t)b * 8);
      d[0] = *reinterpret_cast<u32x4*>(&v[0]);
      d[1] = *reinterpret_cast<u32x4*>(&v[4]);
    }
  }
  // blocks beyond the register slots: the plain loop
  if (total > XREG * nthreads)
    stage_act_f16(codes, scales, total * 16, dst, tid + XREG * nthreads, nthreads);
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
  // four independent dot2 chains per chunk (short dependency chains)
  float b0 = 0.0f, b1 = 0.0f, b2 = 0.0f, b3 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    b0 = dot2(w0[j], x[j], b0);
    b1 = dot2(w0[4 + j], x[4 + j], b1);
    b2 = dot2(w1[j], x[8 + j], b2);
    b3 = dot2(w1[4 + j], x[12 + j], b3);
  }
  acc = fmaf(s0, b0 + b1, acc);
  return fmaf(s1, b2 + b3, acc);
}

// The CPW chunks c0 .. c0+nc-1 of a lane's row.  Straight-line: slots past
// nc re-read a chunk of the same tile (a cache hit, never used), so the
// compiler can count these loads exactly and later waits on earlier loads
// do not also wait for them.
template <int CPW>
__device__ __forceinline__ void load_chunks(const uint8_t* __restrict__ tile, int K, int c0, int nc,
                                            int lane, u32x4 (&cw)[CPW], uint32_t (&sw)[CPW]) {
  const int clast = K / 32 - 1;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = min(i < nc ? c0 + i : c0, clast);
    cw[i] = *reinterpret_cast<const u32x4*>(tile + (size_t)c * 1024 + lane * 16);
    sw[i] = *reinterpret_cast<const uint16_t*>(tile + tile_scale_offset(K) + (size_t)(c >> 2) * 512 + lane * 8 + (c & 3) * 2);
  }
}

// acc[q] += dot of this lane's row slice with activation row slot[q] (LDS,
// f16 A*s); slot[] is wave-uniform.
template <int CPW, int MAXP>
__device__ __forceinline__ void dot_chunks(const u32x4 (&cw)[CPW], const uint32_t (&sw)[CPW], int c0,
                                           int nc, int n, const half2_t* __restrict__ act,
                                           int act_stride, const int (&slot)[MAXP], float (&acc)[MAXP]) {
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    if (i < nc) {
      half2_t w0[8], w1[8];
      cvt16(cw[i].x, cw[i].y, w0);
      cvt16(cw[i].z, cw[i].w, w1);
      const float s0 = e4m3_to_f32(sw[i] & 0xFF), s1 = e4m3_to_f32(sw[i] >> 8);
#pragma unroll
      for (int q = 0; q < MAXP; ++q)
        if (q < n) acc[q] = chunk_dot(w0, w1, s0, s1, act + (size_t)slot[q] * act_stride + (c0 + i) * 16, acc[q]);
    }
  }
}

// One activation row, no branches: chunks past nc take scale 0 (their loads
// were clamped to valid chunks), so every wait on a chunk's load is the
// in-order wait for that chunk alone.
template <int CPW>
__device__ __forceinline__ float dot_chunks_row(const u32x4 (&cw)[CPW], const uint32_t (&sw)[CPW], int c0,
                                                int nc, int clast, const half2_t* __restrict__ act) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    half2_t w0[8], w1[8];
    cvt16(cw[i].x, cw[i].y, w0);
    cvt16(cw[i].z, cw[i].w, w1);
    const bool ok = i < nc;
    const float s0 = ok ? e4m3_to_f32(sw[i] & 0xFF) : 0.0f;
    const float s1 = ok ? e4m3_to_f32(sw[i] >> 8) : 0.0f;
    acc = chunk_dot(w0, w1, s0, s1, act + (size_t)min(c0 + i, clast) * 16, acc);
  }
  return acc;
}

// ---- gate/up weights in either format, held in registers per wave
// NVFP4 (FMT 0): CPW chunks of 32 elements (16 code bytes + 2 scale bytes per
// lane).  Codebook (FMT 1): CB_GPW groups of 128 elements (three 16-byte
// index words of 3-bit indices + eight fp16 entries per lane); a weight is
// its group's entry, with no block or tensor scale.
constexpr int CB_GPW = 3;
template <int FMT, int CPW> struct GuRegs;
template <int CPW> struct GuRegs<0, CPW> {
  u32x4 cw[CPW];
  uint32_t sw[CPW];
};
template <int CPW> struct GuRegs<1, CPW> {
  u32x4 p[CB_GPW][3];
  u32x4 c[CB_GPW];
};
// K elements per work unit of a wave (a chunk or a group)
template <int FMT> __host__ __device__ constexpr int gu_unit() { return FMT == 1 ? 128 : 32; }

// Groups g0 .. g0+ng-1 of a codebook tile, straight-line (slots past ng
// re-read group g0, a cache hit, never used).
__device__ __forceinline__ void load_groups(const uint8_t* __restrict__ tile, int K, int g0, int ng,
                                            int lane, u32x4 (&p)[CB_GPW][3], u32x4 (&c)[CB_GPW]) {
  const int glast = K / 128 - 1;
#pragma unroll
  for (int i = 0; i < CB_GPW; ++i) {
    const int g = min(i < ng ? g0 + i : g0, glast);
    const uint8_t* grp = tile + (size_t)g * cb_group_bytes();
    const u32x4* pl = reinterpret_cast<const u32x4*>(grp + lane * 48);
    p[i][0] = pl[0];
    p[i][1] = pl[1];
    p[i][2] = pl[2];
    c[i] = *reinterpret_cast<const u32x4*>(grp + 64 * 48 + lane * 16);
  }
}

template <int FMT, int CPW>
__device__ __forceinline__ void gu_load(GuRegs<FMT, CPW>& R, const uint8_t* __restrict__ tile, int K, int u0,
                                        int nu, int lane) {
  if constexpr (FMT == 1) load_groups(tile, K, u0, nu, lane, R.p, R.c);
  else load_chunks<CPW>(tile, K, u0, nu, lane, R.cw, R.sw);
}

// sum over one codebook group of entry * activation (f16 products exact in
// fp32, fp32 accumulation), four independent chains
__device__ __forceinline__ float group_dot(const u32x4 (&p)[3], u32x4 c, const half2_t* __restrict__ xs) {
  float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    half2_t w[16];
    dequant32_cb(p[0][d], p[1][d], p[2][d], c, w);
    const u32x4* xp = reinterpret_cast<const u32x4*>(xs + 16 * d);
    half2_t x[16];
#pragma unroll
    for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x4*>(&x[4 * r]) = xp[r];
#pragma unroll
    for (int j = 0; j < 16; ++j) b[d] = dot2(w[j], x[j], b[d]);
  }
  return (b[0] + b[1]) + (b[2] + b[3]);
}

// One activation row: units past nu count 0 (their loads were clamped).
template <int FMT, int CPW>
__device__ __forceinline__ float gu_dot_row(const GuRegs<FMT, CPW>& R, int u0, int nu, int K,
                                            const half2_t* __restrict__ act) {
  if constexpr (FMT == 1) {
    const int glast = K / 128 - 1;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CB_GPW; ++i) {
      const float gsum = group_dot(R.p[i], R.c[i], act + (size_t)min(u0 + i, glast) * 64);
      acc += i < nu ? gsum : 0.0f;
    }
    return acc;
  } else {
    return dot_chunks_row<CPW>(R.cw, R.sw, u0, nu, K / 32 - 1, act);
  }
}

// acc[q] += dot with activation row slot[q] (wave-uniform slots).
template <int FMT, int CPW, int MAXP>
__device__ __forceinline__ void gu_dot(const GuRegs<FMT, CPW>& R, int u0, int nu, int n,
                                       const half2_t* __restrict__ act, int act_stride,
                                       const int (&slot)[MAXP], float (&acc)[MAXP]) {
  if constexpr (FMT == 1) {
#pragma unroll
    for (int i = 0; i < CB_GPW; ++i) {
      if (i < nu) {
#pragma unroll
        for (int q = 0; q < MAXP; ++q)
          if (q < n) acc[q] += group_dot(R.p[i], R.c[i], act + (size_t)slot[q] * act_stride + (size_t)(u0 + i) * 64);
      }
    }
  } else {
    dot_chunks<CPW, MAXP>(R.cw, R.sw, u0, nu, n, act, act_stride, slot, acc);
  }
}

// All pair ids of the call in registers (lane l holds pair l + 64 i, PC
// chunks of 64 pairs: 1 for one token, 8 up to 16 tokens, 32 up to 64), so
// the owner test and the pair lists come from ballots, not dependent loads.
template <int PC>
struct PairIds {
  int v[PC];
};

template <int PC>
__device__ __forceinline__ PairIds<PC> load_pair_ids(const int32_t* ids, int npairs, int lane) {
  PairIds<PC> p;
#pragma unroll
  for (int i = 0; i < PC; ++i) {                 // every load issued before the first use
    const int q = lane + 64 * i;
    const int v = ids[q < npairs ? q : npairs - 1];
    p.v[i] = q < npairs ? v : 0;
  }
  return p;
}

// Expert of pair p (wave-uniform).
template <int PC>
__device__ __forceinline__ int pair_expert(const PairIds<PC>& P, int p) {
  int sel = 0;
#pragma unroll
  for (int i = 0; i < PC; ++i)
    if (i == (p >> 6)) sel = P.v[i];
  return __builtin_amdgcn_readlane(sel, p & 63);
}

// Ballot masks of the pairs routed to expert e (wave-uniform).
template <int PC>
__device__ __forceinline__ void pair_masks(const PairIds<PC>& P, int npairs, int e, int lane,
                                           uint64_t (&m)[PC]) {
#pragma unroll
  for (int i = 0; i < PC; ++i) m[i] = __ballot(lane + 64 * i < npairs && P.v[i] == e);
}

template <int PC>
__device__ __forceinline__ int first_pair(const uint64_t (&m)[PC]) {
#pragma unroll
  for (int i = 0; i < PC; ++i)
    if (m[i]) return 64 * i + __ffsll((unsigned long long)m[i]) - 1;
  return -1;
}

// Up to MAXP pairs from the masks at or after qstart, written to list by
// thread 0; returns the count and the next unserved pair (or npairs).
template <int MAXP, int PC>
__device__ __forceinline__ int masked_pairs(const uint64_t (&m)[PC], int npairs, int qstart,
                                            int* list, int* qnext, int tid) {
  int n = 0;
  *qnext = npairs;
#pragma unroll
  for (int i = 0; i < PC; ++i) {
    uint64_t mm = m[i];
    const int lo = qstart - 64 * i;
    if (lo >= 64) mm = 0;
    else if (lo > 0) mm &= ~((1ull << lo) - 1ull);
    while (mm) {
      const int q = 64 * i + __ffsll((unsigned long long)mm) - 1;
      if (n == MAXP) { if (*qnext == npairs) *qnext = q; mm = 0; break; }
      if (tid == 0) list[n] = q;
      ++n;
      mm &= mm - 1;
    }
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

// One token: a single split when the row fits one block's waves (then the
// block holds whole gate and up rows and can form h itself).
__host__ __device__ inline int dec_ks(int H, int T) {
  return (T == 1 && H / 32 <= DEC_MAX_WAVES * DEC_CPW) ? 1 : dec_ksplit(H);
}

__host__ __device__ inline int dec_waves(int nchunk_block) {
  int nw = (nchunk_block + DEC_CPW - 1) / DEC_CPW;
  return nw < 1 ? 1 : (nw > DEC_MAX_WAVES ? DEC_MAX_WAVES : nw);
}

struct DecodeWs {
  float* gu;          // [KS][T*k][2][I] gate/up partial dot sums, tensor scales applied;
                      // h mode: h [T*k][I], then max |h| per 32-row tile [T*k][I/32]
  uint8_t* hc;        // [T*k][I/2]  h^ codes
  uint8_t* hsc;       // [T*k][I/16] h^ block scales (E4M3)
  float* hts;         // [T*k]       h^ tensor scales
};

// ---------------------------------------------------------------- gate/up
// TOPK: rank the router logits in-block first (fused layer), writing ids and
// w once (block 0,0,0); otherwise read ids.
template <int MAXP, int CPW, bool TOPK, int PC, int FMT>
__global__ __launch_bounds__(64 * DEC_MAX_WAVES) void gate_up_decode_kernel(
    FfnArgs a, DecodeWs ws, const float* __restrict__ logits, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, int hmode) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nw = blockDim.x >> 6;
  half2_t* xs = reinterpret_cast<half2_t*>(smem);                         // [MAXP][H/2]
  float* red = reinterpret_cast<float*>(smem + (size_t)MAXP * a.H * 2);   // [nw][MAXP][64]
  __shared__ int list[MAXP];
  __shared__ int sids[TOPK ? MOE_MAX_K : 1];             // ranked ids (one token)
  __shared__ int tscr[TOPK ? DEC_MAX_WAVES : 1][TOPK_SCR_INTS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int npairs = a.T * a.k, p = blockIdx.x, j = blockIdx.y, split = blockIdx.z;
  const int KS = gridDim.z;
  // x^ of every token staged once (slot t) when the call has few tokens;
  // otherwise per batch of pairs (slot = batch index)
  const bool by_token = a.T <= MAXP;
  const int32_t* ids;
  if (TOPK) {
    // waves 0..T-1 rank the logits; the other waves stage x^ meanwhile
    const int nrank = min(a.T, nw);
    for (int t = wv; t < a.T; t += nw) {
      int id;
      float wt;
      topk_wave_any(logits + (size_t)t * a.E, a.E, a.k, lane, tscr[wv], &id, &wt);
      if (lane < a.k) {
        sids[t * a.k + lane] = id;
        if (p == 0 && j == 0 && split == 0) {
          ids_out[t * a.k + lane] = id;
          w_out[t * a.k + lane] = wt;
        }
      }
    }
    if (by_token && nrank < nw && wv >= nrank) {
      for (int t = 0; t < a.T; ++t)
        stage_act_f16(a.x_codes + (size_t)t * (a.H / 2), a.x_scales + (size_t)t * (a.H / 16), a.H,
                      xs + (size_t)t * (a.H / 2), tid - 64 * nrank, blockDim.x - 64 * nrank);
    }
    __syncthreads();
    ids = sids;
  } else {
    ids = a.ids;
  }
  const PairIds<PC> P = load_pair_ids<PC>(ids, npairs, lane);
  // one token: its x^ is loaded before the weights and staged while they
  // are in flight; several tokens: only the tokens routed to this block's
  // expert are staged, after the weight loads are issued
  const int xtot = a.T * (a.H / 16);
  ActRegs xr;
  if (!TOPK && MAXP == 1) act_load(xr, a.x_codes, a.x_scales, xtot, tid, blockDim.x);
  const int e = pair_expert(P, p);
  uint64_t pm[PC];
  pair_masks(P, npairs, e, lane, pm);
  if (first_pair(pm) != p) return;                            // another block owns e
  const size_t part_stride = (size_t)npairs * 2 * a.I;
  float* gu = ws.gu + (size_t)split * part_stride;
  if ((unsigned)e >= (unsigned)a.E) {                         // not an expert: partials 0
    for (int q = p; q < npairs; ++q) {
      if (!((pm[q >> 6] >> (q & 63)) & 1) || tid >= 64) continue;
      if (hmode) {                                            // h 0, tile max 0
        if (tid < 32) {
          ws.gu[(size_t)q * a.I + 32 * j + tid] = 0.0f;
          if (a.dbg_h) a.dbg_h[(size_t)q * a.I + 32 * j + tid] = 0.0f;
        }
        if (tid == 0) ws.gu[(size_t)npairs * a.I + (size_t)q * (a.I / 32) + j] = 0.0f;
        if (a.h_ts) {                                         // static mode: h^ = 0
          if (tid < 16) {
            ws.hc[(size_t)q * (a.I / 2) + 16 * j + tid] = 0;
            if (a.dbg_h_codes) a.dbg_h_codes[(size_t)q * (a.I / 2) + 16 * j + tid] = 0;
          }
          if (tid < 2) {
            ws.hsc[(size_t)q * (a.I / 16) + 2 * j + tid] = 0;
            if (a.dbg_h_scales) a.dbg_h_scales[(size_t)q * (a.I / 16) + 2 * j + tid] = 0;
          }
          if (tid == 0 && j == 0) {
            ws.hts[q] = 0.0f;
            if (a.dbg_h_ts) a.dbg_h_ts[q] = 0.0f;
          }
        }
      } else {
        gu[(size_t)q * 2 * a.I + (tid >> 5) * a.I + 32 * j + (tid & 31)] = 0.0f;
      }
    }
    return;
  }
  const uint8_t* tile = FMT == 1
      ? a.gate_up + (size_t)e * cb_gate_up_expert_bytes(a.H, a.I) + (size_t)j * cb_tile_bytes(a.H)
      : a.gate_up + (size_t)e * gate_up_expert_bytes(a.H, a.I) + (size_t)j * tile_bytes(a.H);
  const int nunit_b = a.H / gu_unit<FMT>() / KS;                // chunks or groups of this block
  const int upw = (nunit_b + nw - 1) / nw;
  const int c0 = split * nunit_b + wv * upw;
  const int nc = max(0, min(upw, nunit_b - wv * upw));
  GuRegs<FMT, CPW> R;
  gu_load<FMT, CPW>(R, tile, a.H, c0, nc, lane);              // all weight loads in flight
  if (by_token) {
    if (!TOPK && MAXP == 1) {
      act_store(xr, a.x_codes, a.x_scales, xtot, xs, tid, blockDim.x);
    } else if (MAXP > 1 || min(a.T, nw) >= nw) {
      // stage now, only the tokens routed to this expert (each token at
      // most once: its k experts are distinct)
#pragma unroll
      for (int i = 0; i < PC; ++i) {
        uint64_t mm = pm[i];
        while (mm) {
          const int t = (64 * i + __ffsll((unsigned long long)mm) - 1) / a.k;
          mm &= mm - 1;
          stage_act_f16(a.x_codes + (size_t)t * (a.H / 2), a.x_scales + (size_t)t * (a.H / 16), a.H,
                        xs + (size_t)t * (a.H / 2), tid, blockDim.x);
        }
      }
    }
  }
  if constexpr (MAXP == 1) {
    // one token (MAXP 1 is the one-token launch): every pair on this
    // expert has the same x, so the dots run once, straight-line, and the
    // partial goes to each such pair; tensor scales load per lane beside
    // the weights
    const float tsw = FMT == 1 ? 1.0f : (lane < 32 ? a.ts_gate : a.ts_up)[e];
    const float xts = a.x_ts[lane < a.T ? lane : a.T - 1];
    __syncthreads();                                           // x^ staged
    const float acc = gu_dot_row<FMT, CPW>(R, c0, nc, a.H, xs);
    red[wv * 64 + lane] = acc;
    __syncthreads();
    if (wv == 0) {
      float v = 0.0f;
      for (int w = 0; w < nw; ++w) v += red[w * 64 + lane];
      v *= __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(xts))) * tsw;
      if (hmode) {
        // h mode (one split): this block holds whole gate rows (lanes 0-31)
        // and up rows (lanes 32-63) 32j..32j+31, so it forms h = SiLU(g) u
        // and the tile's max |h| for the down step's quantizer
        const float u = __shfl_xor(v, 32, 64);
        const float h = silu_mul(v, u);
        const float hm = dpp_wave_max(lane < 32 ? fabsf(h) : 0.0f);
        float* hmax = ws.gu + (size_t)npairs * a.I;
        // static h scale: this tile's two 16-row blocks are quantized here
        // (block max over each 16-lane row, one element per lane, the odd
        // lane's code folded into the even lane's byte), so the down kernel
        // reads h^ instead of quantizing h itself
        uint32_t c4 = 0, sb = 0, cpair = 0;
        float hts_s = 0.0f;
        if (a.h_ts) {
          hts_s = a.h_ts[e];
          float ab = fabsf(h);
          ab = fmaxf(ab, __int_as_float(dpp_mov<0xB1>(0, __float_as_int(ab))));
          ab = fmaxf(ab, __int_as_float(dpp_mov<0x4E>(0, __float_as_int(ab))));
          ab = fmaxf(ab, __int_as_float(dpp_mov<0x141>(0, __float_as_int(ab))));   // row_half_mirror
          ab = fmaxf(ab, __int_as_float(dpp_mov<0x140>(0, __float_as_int(ab))));   // row_mirror
          sb = quantize_one(h, ab, hts_s, c4);
          cpair = c4 | (__shfl_xor(c4, 1, 64) << 4);
        }
#pragma unroll
        for (int i = 0; i < PC; ++i) {
          uint64_t mm = pm[i];
          while (mm) {
            const int q = 64 * i + __ffsll((unsigned long long)mm) - 1;
            mm &= mm - 1;
            if (lane < 32) {
              ws.gu[(size_t)q * a.I + 32 * j + lane] = h;
              if (a.dbg_h) a.dbg_h[(size_t)q * a.I + 32 * j + lane] = h;
            }
            if (lane == 0) hmax[(size_t)q * (a.I / 32) + j] = hm;
            if (a.h_ts) {
              if (lane < 32 && (lane & 1) == 0) {
                ws.hc[(size_t)q * (a.I / 2) + 16 * j + lane / 2] = (uint8_t)cpair;
                if (a.dbg_h_codes) a.dbg_h_codes[(size_t)q * (a.I / 2) + 16 * j + lane / 2] = (uint8_t)cpair;
              }
              if (lane == 0 || lane == 16) {
                ws.hsc[(size_t)q * (a.I / 16) + 2 * j + lane / 16] = (uint8_t)sb;
                if (a.dbg_h_scales) a.dbg_h_scales[(size_t)q * (a.I / 16) + 2 * j + lane / 16] = (uint8_t)sb;
              }
              if (lane == 0 && j == 0) {
                ws.hts[q] = hts_s;
                if (a.dbg_h_ts) a.dbg_h_ts[q] = hts_s;
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < PC; ++i) {
          uint64_t mm = pm[i];
          while (mm) {
            const int q = 64 * i + __ffsll((unsigned long long)mm) - 1;
            mm &= mm - 1;
            gu[(size_t)q * 2 * a.I + (lane >> 5) * a.I + 32 * j + (lane & 31)] = v;
          }
        }
      }
    }
  } else {
    int qstart = p;
    while (true) {
      int qnext;
      const int n = masked_pairs<MAXP, PC>(pm, npairs, qstart, list, &qnext, tid);
      __syncthreads();
      if (!by_token) {
        for (int i = 0; i < n; ++i) {
          const int t = list[i] / a.k;
          stage_act_f16(a.x_codes + (size_t)t * (a.H / 2), a.x_scales + (size_t)t * (a.H / 16), a.H,
                        xs + (size_t)i * (a.H / 2), tid, blockDim.x);
        }
        __syncthreads();
      }
      int slot[MAXP];
  #pragma unroll
      for (int i = 0; i < MAXP; ++i) slot[i] = (i < n) ? (by_token ? list[i] / a.k : i) : 0;
      float acc[MAXP];
  #pragma unroll
      for (int i = 0; i < MAXP; ++i) acc[i] = 0.0f;
      gu_dot<FMT, CPW, MAXP>(R, c0, nc, n, xs, a.H / 2, slot, acc);
  #pragma unroll
      for (int i = 0; i < MAXP; ++i) red[(wv * MAXP + i) * 64 + lane] = acc[i];
      __syncthreads();
      if (wv == 0) {
        for (int i = 0; i < n; ++i) {
          float v = 0.0f;
          for (int w = 0; w < nw; ++w) v += red[(w * MAXP + i) * 64 + lane];
          // lane < 32: gate row 32j + lane; lane >= 32: up row 32j + lane - 32;
          // the partial carries its tensor scales (x row, weight matrix)
          const int q = list[i];
          const float sc = a.x_ts[q / a.k] * (FMT == 1 ? 1.0f : (lane < 32 ? a.ts_gate[e] : a.ts_up[e]));
          gu[(size_t)q * 2 * a.I + (lane >> 5) * a.I + 32 * j + (lane & 31)] = v * sc;
        }
      }
      if (qnext >= npairs) break;
      qstart = qnext;
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- h^
// h = SiLU(g) * u of every pair from the gate/up partials (summed over the
// K-splits in split order), then NVFP4 with the row's own tensor scale.
// Block = one pair; four lanes per 16-element block (four elements each):
// the block max is a quad reduction, the row amax a wave max plus a fixed
// pass over the waves' maxima in LDS, and each lane quantizes its quarter
// (the same steps as the whole-block quantizer).  h^ is written once here
// and read by every down block.
__global__ __launch_bounds__(1024) void h_quant_decode_kernel(FfnArgs a, DecodeWs ws) {
  __shared__ float wmax[16];
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int nq = a.I / 4;                                  // quarters in the row
  const int KS = dec_ks(a.H, a.T);
  const size_t part_stride = (size_t)a.T * a.k * 2 * a.I;
  const int qi = tid < nq ? tid : nq - 1;                   // extra lanes redo the last quarter
  float g[4], u[4];
  for (int sp0 = 0; sp0 < KS; sp0 += 2) {                   // two splits' loads in flight at once
    float4_t g4[2], u4[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int spc = min(sp0 + s2, KS - 1);
      const float* gp = ws.gu + (size_t)spc * part_stride + (size_t)q * 2 * a.I + qi * 4;
      g4[s2] = *reinterpret_cast<const float4_t*>(gp);
      u4[s2] = *reinterpret_cast<const float4_t*>(gp + a.I);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      if (sp0 + s2 < KS) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          g[c] = (sp0 + s2 == 0) ? g4[s2][c] : g[c] + g4[s2][c];
          u[c] = (sp0 + s2 == 0) ? u4[s2][c] : u[c] + u4[s2][c];
        }
      }
    }
  }
  float hv[4];
  float m4 = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    hv[c] = silu_mul(g[c], u[c]);
    m4 = fmaxf(m4, fabsf(hv[c]));
  }
  // block max over the quad (lanes 4b .. 4b+3 hold block b)
  float bmax = fmaxf(m4, __int_as_float(dpp_mov<0xB1>(0, __float_as_int(m4))));
  bmax = fmaxf(bmax, __int_as_float(dpp_mov<0x4E>(0, __float_as_int(bmax))));
  const float m = dpp_wave_max(tid < nq ? m4 : 0.0f);
  if (lane == 0) wmax[wv] = m;
  __syncthreads();
  float amax = wmax[0];
  for (int w = 1; w < nw; ++w) amax = fmaxf(amax, wmax[w]);
  // static mode: the pair's expert's calibrated scale (0 for an invalid id,
  // whose h is 0)
  int eq = 0;
  if (a.h_ts) eq = a.ids[q];
  const float ts = a.h_ts ? ((unsigned)eq < (unsigned)a.E ? a.h_ts[eq] : 0.0f) : tensor_scale_from_amax(amax);
  if (tid < nq) {
    uint32_t bits;
    const uint32_t sb = quantize_quarter4(hv, bmax, ts, bits);
    const int b = qi >> 2, part = qi & 3;
    *reinterpret_cast<uint16_t*>(ws.hc + (size_t)q * (a.I / 2) + qi * 2) = (uint16_t)bits;
    if (part == 0) ws.hsc[(size_t)q * (a.I / 16) + b] = (uint8_t)sb;
    if (a.dbg_h) *reinterpret_cast<float4_t*>(a.dbg_h + (size_t)q * a.I + qi * 4) = float4_t{hv[0], hv[1], hv[2], hv[3]};
    if (a.dbg_h_codes) *reinterpret_cast<uint16_t*>(a.dbg_h_codes + (size_t)q * (a.I / 2) + qi * 2) = (uint16_t)bits;
    if (a.dbg_h_scales && part == 0) a.dbg_h_scales[(size_t)q * (a.I / 16) + b] = (uint8_t)sb;
  }
  if (tid == 0) {
    ws.hts[q] = ts;
    if (a.dbg_h_ts) a.dbg_h_ts[q] = ts;
  }
}

// ---------------------------------------------------------------- down
template <int MAXP, int CPW, int PC>
__global__ __launch_bounds__(64 * DEC_MAX_WAVES) void down_decode_kernel(FfnArgs a, DecodeWs ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nw = blockDim.x >> 6;
  half2_t* hs = reinterpret_cast<half2_t*>(smem);                          // [MAXP][I/2]
  float* red = reinterpret_cast<float*>(smem + (size_t)MAXP * a.I * 2);    // [nw][MAXP][64]
  __shared__ int list[MAXP];
  __shared__ float hts[MAXP];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int npairs = a.T * a.k, p = blockIdx.x, j = blockIdx.y;
  const PairIds<PC> P = load_pair_ids<PC>(a.ids, npairs, lane);
  const int e = pair_expert(P, p);
  uint64_t pm[PC];
  pair_masks(P, npairs, e, lane, pm);
  if (first_pair(pm) != p) return;                            // another block owns e
  if ((unsigned)e >= (unsigned)a.E) {                         // not an expert: o = 0
    for (int q = p; q < npairs; ++q)
      if (((pm[q >> 6] >> (q & 63)) & 1) && tid < 64) a.out[(size_t)q * a.H + 64 * j + tid] = 0.0f;
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
    int qstart = p;
    while (true) {
      int qnext;
      const int n = masked_pairs<MAXP, PC>(pm, npairs, qstart, list, &qnext, tid);
      __syncthreads();
      // h^ of the batch's pairs (quantized once by the h^ kernel) as f16 A*s
      for (int i = 0; i < n; ++i) {
        const int q = list[i];
        stage_act_f16(ws.hc + (size_t)q * (a.I / 2), ws.hsc + (size_t)q * nblk, a.I,
                      hs + (size_t)i * (a.I / 2), tid, blockDim.x);
        if (tid == 0) hts[i] = ws.hts[q];
      }
      __syncthreads();
      int slot[MAXP];
#pragma unroll
      for (int i = 0; i < MAXP; ++i) slot[i] = i;
      float acc[MAXP];
#pragma unroll
      for (int i = 0; i < MAXP; ++i) acc[i] = 0.0f;
      dot_chunks<CPW, MAXP>(cw, sw, c0, nc, n, hs, a.I / 2, slot, acc);
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
      if (qnext >= npairs) break;
      qstart = qnext;
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- down + combine
// Down step for few pairs: a block owns 16 output columns n0..n0+15 of the
// pairs of blockIdx.y's group of tokens (all T tokens when T*k <= SL_MAXP,
// else one token, so k <= SL_MAXP) and wave q serves the group's pair q.
// Per-token blocks read an expert's rows once per token that routes to it
// (a few per cent more than once per distinct expert at eight tokens, most of
// it from L2) and in exchange need neither o in HBM nor a combine kernel.  Lane (r = lane & 15,
// quarter qt = lane >> 4) reads row n0 + r of the pair's 64-row down tile at
// chunks qt, qt+4, ...; the quarters are summed with lane shuffles.
// Order of work: the pair ids, the combine inputs and this thread's block of
// h^ are loaded first; the weight loads follow as soon as the ids are in;
// h^ goes to LDS as f16 A*s while the weights are in flight.  All loads are
// straight-line (clamped indices instead of branches), so each wait covers
// exactly the loads it needs.  With COMBINE the block also does the weighted
// combine of its 16 columns, so no cross-block step is needed.  A pair whose
// id is outside [0, E) gets o = 0.
constexpr int SL_MAXP = 16;              // pairs (= waves) per block
constexpr int SL_CPQ = 5;                // chunks per quarter held in registers (I <= 640)

constexpr int SL_HQR = 3;                // h quarters per lane in h mode (I <= 768)
// Per-token slice blocks in the fused layer up to this many tokens.  Layer
// step at H 2560, I 640, E 512, k 10 (graph-replayed, 8 layers cycled), against
// the per-expert down GEMVs plus the combine kernel: 40.0 -> 36.2 us at 2
// tokens, 53.2 -> 50.1 at 4, 77.6 -> 75.4 at 8, 98.8 -> 100.8 at 12 and
// 126.9 -> 128.1 at 16 (duplicate expert reads grow with the tokens).
constexpr int SL_TOKEN_MAX_T = 8;

// HQ (h mode, one token): wave q quantizes pair q's h row itself, from h
// and the 32-row tile maxima the gate/up step wrote (the row amax is their
// max), with the h^ quantizer's steps: four lanes per 16-element block
// (quad max), each lane coding its quarter.  Every block repeats this for
// all pairs; no separate h^ pass.
template <bool COMBINE, bool HQ>
__global__ __launch_bounds__(64 * SL_MAXP) void down_slice_kernel(FfnArgs a, DecodeWs ws,
                                                                  const float* __restrict__ w_comb,
                                                                  const uint16_t* __restrict__ residual,
                                                                  uint16_t* __restrict__ y,
                                                                  const float* __restrict__ res_scale) {
  extern __shared__ __align__(16) unsigned char smem[];
  // this block's tokens tok0 .. tok0+ntok-1, pairs q0 .. q0+npairs-1
  const int ntok = gridDim.y == 1 ? a.T : 1;
  const int tok0 = blockIdx.y * ntok, q0 = tok0 * a.k;
  const int npairs = ntok * a.k;
  half2_t* hs = reinterpret_cast<half2_t*>(smem);                              // [npairs][I/2]
  float* obuf = reinterpret_cast<float*>(smem + (size_t)npairs * a.I * 2);     // [npairs][16]
  __shared__ float hts[SL_MAXP];
  __shared__ float wcs[SL_MAXP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int q = __builtin_amdgcn_readfirstlane(tid >> 6);    // this wave's pair
  const int n0 = blockIdx.x * 16;
  const int r = lane & 15, qt = lane >> 4;
  const int jt = n0 >> 6, lit = (n0 & 63) + r;               // down tile, lane within it
  const int nchunk = a.I / 32, nblk = a.I / 16;
  const int nitems = npairs * nblk;
  // ---- loads that do not depend on the routing, ids first
  const int qid = a.ids[q0 + (lane < npairs ? lane : npairs - 1)];
  const float htl = HQ ? 0.0f : ws.hts[q0 + (lane < npairs ? lane : npairs - 1)];
  float wc = 0.0f;
  uint16_t res = 0;
  if (COMBINE) {
    wc = w_comb[q0 + (tid < npairs ? tid : npairs - 1)];
    const int cidx = tid < ntok * 16 ? tid : ntok * 16 - 1;
    // no residual: read y's own column instead (unused), keeping the load unconditional
    const uint16_t* rp = residual ? residual : y;
    res = rp[(size_t)(tok0 + (cidx >> 4)) * a.H + n0 + (cidx & 15)];
    if (res_scale) res = (uint16_t)bf16_scaled(res, res_scale[tok0 + (cidx >> 4)]);
  }
  const int item = tid < nitems ? tid : nitems - 1;
  const int jq = item / nblk, jb = item % nblk;
  u32x2 hcw = {0u, 0u};
  uint32_t hsw = 0;
  float4_t hq[HQ ? SL_HQR : 1];
  float hmx = 0.0f;
  const int nqr = a.I / 4, ntile = a.I / 32;
  if (!HQ) {
    hcw = *reinterpret_cast<const u32x2*>(ws.hc + (size_t)(q0 + jq) * (a.I / 2) + jb * 8);
    hsw = ws.hsc[(size_t)(q0 + jq) * nblk + jb];
  } else {
    // h mode: h rows and the 32-row tile maxima behind all T*k h rows
    const float* hrow = ws.gu + (size_t)(q0 + q) * a.I;
#pragma unroll
    for (int m = 0; m < SL_HQR; ++m)
      hq[m] = *reinterpret_cast<const float4_t*>(hrow + (size_t)min(lane + 64 * m, nqr - 1) * 4);
    hmx = ws.gu[(size_t)a.T * a.k * a.I + (size_t)(q0 + q) * ntile + min(lane, ntile - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);        // these loads stay ahead of the weight loads
  // ---- this pair's expert and its weight loads
  const int e = __builtin_amdgcn_readlane(qid, q);
  const bool valid = (unsigned)e < (unsigned)a.E;
  const uint8_t* tile = a.down + (size_t)(valid ? e : 0) * down_expert_bytes(a.H, a.I) + (size_t)jt * tile_bytes(a.I);
  u32x4 cw[SL_CPQ];
  uint32_t sw[SL_CPQ];
#pragma unroll
  for (int m = 0; m < SL_CPQ; ++m) {
    const int c = min(qt + 4 * m, nchunk - 1);
    cw[m] = *reinterpret_cast<const u32x4*>(tile + (size_t)c * 1024 + lit * 16);
    sw[m] = *reinterpret_cast<const uint16_t*>(tile + tile_scale_offset(a.I) + (size_t)(c >> 2) * 512 + lit * 8 + (c & 3) * 2);
  }
  // this pair's tensor scale as a per-lane load (lane l: pair l's expert)
  const float tsd_l = a.ts_down[(unsigned)qid < (unsigned)a.E ? qid : 0];
  __builtin_amdgcn_sched_barrier(0);        // keep the weight loads ahead of the staging

  // ---- h^ into LDS as f16 A*s
  if (!HQ) {
    if (tid < nitems) {
      const _Float16 sc = (_Float16)e4m3_to_f32(hsw);
      const half2_t s2 = {sc, sc};
      half2_t wq[8];
      cvt16(hcw.x, hcw.y, wq);
      half2_t* d = hs + (size_t)jq * (a.I / 2) + jb * 8;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) d[rr] = wq[rr] * s2;
    }
    if (tid < npairs) hts[tid] = htl;
  } else {
    const float amax = dpp_wave_max(lane < ntile ? hmx : 0.0f);
    const float ts = tensor_scale_from_amax(amax);
    const bool dbg = blockIdx.x == 0;
#pragma unroll
    for (int m = 0; m < SL_HQR; ++m) {
      const int qi = lane + 64 * m;
      const float v[4] = {hq[m][0], hq[m][1], hq[m][2], hq[m][3]};
      const float m4 = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
      float b4 = fmaxf(m4, __int_as_float(dpp_mov<0xB1>(0, __float_as_int(m4))));
      b4 = fmaxf(b4, __int_as_float(dpp_mov<0x4E>(0, __float_as_int(b4))));
      if (qi < nqr) {
        uint32_t bits;
        const uint32_t sb = quantize_quarter4(v, b4, ts, bits);
        const _Float16 sc = (_Float16)e4m3_to_f32(sb);
        const half2_t s2 = {sc, sc};
        half2_t* d = hs + (size_t)q * (a.I / 2) + qi * 2;
        d[0] = fp4x2_to_f16x2<0>(bits) * s2;
        d[1] = fp4x2_to_f16x2<1>(bits) * s2;
        if (dbg && a.dbg_h_codes)
          *reinterpret_cast<uint16_t*>(a.dbg_h_codes + (size_t)(q0 + q) * (a.I / 2) + qi * 2) = (uint16_t)bits;
        if (dbg && a.dbg_h_scales && (qi & 3) == 0) a.dbg_h_scales[(size_t)(q0 + q) * nblk + (qi >> 2)] = (uint8_t)sb;
      }
    }
    if (lane == 0) {
      hts[q] = ts;
      if (dbg && a.dbg_h_ts) a.dbg_h_ts[q0 + q] = ts;
    }
  }
  if (COMBINE && tid < npairs) wcs[tid] = wc;
  __syncthreads();

  // ---- down dot of pair q over this block's 16 rows
  // no branches: chunks past the row take scale 0 (their loads were clamped)
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < SL_CPQ; ++m) {
    const int c = qt + 4 * m;
    const bool ok = c < nchunk;
    half2_t w0[8], w1[8];
    cvt16(cw[m].x, cw[m].y, w0);
    cvt16(cw[m].z, cw[m].w, w1);
    acc = chunk_dot(w0, w1, ok ? e4m3_to_f32(sw[m] & 0xFF) : 0.0f, ok ? e4m3_to_f32(sw[m] >> 8) : 0.0f,
                    hs + (size_t)q * (a.I / 2) + min(c, nchunk - 1) * 16, acc);
  }
  const float tsd = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tsd_l), q));
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  if (lane < 16) {
    const float ov = valid ? acc * (hts[q] * tsd) : 0.0f;
    obuf[q * 16 + r] = ov;
    if (!COMBINE) a.out[(size_t)(q0 + q) * a.H + n0 + r] = ov;   // with the combine o stays in LDS
  }
  if (!COMBINE) return;
  __syncthreads();

  // ---- combine these 16 columns: fp32 in slot order, one bf16 rounding
  if (tid < ntok * 16) {
    const int t = tid >> 4, c = tid & 15;
    float accy = 0.0f;
    for (int i = 0; i < a.k; ++i) accy = fmaf(wcs[t * a.k + i], obuf[(t * a.k + i) * 16 + c], accy);
    if (residual) accy += bf16_to_f32(res);
    y[(size_t)(tok0 + t) * a.H + n0 + c] = (uint16_t)f32_to_bf16_rne(accy);
  }
}

// ---------------------------------------------------------------- router + x quant
// Fused layer, kernel 1 (256 threads): E blocks compute one router logit row
// each (the same routine as the standalone router) and T blocks quantize one
// token row each.
// in_rms > 0 (the stack's rescaled input, one token): every block takes the
// token's scale s = in_rms / rms(x) (the shared fixed-order routine, so all
// blocks agree bit for bit; router blocks while their weight row loads are
// in flight), the router rows use bf16(x s), the quantizer block quantizes it
// and stores s for the down step's residual.
__global__ __launch_bounds__(256) void router_quant_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ W,
                                                           const float* __restrict__ bias, int T, int E,
                                                           int H, float* __restrict__ logits,
                                                           uint8_t* __restrict__ xc,
                                                           uint8_t* __restrict__ xsc,
                                                           float* __restrict__ xts, float in_rms,
                                                           float* __restrict__ xscale) {
  __shared__ float red[64];
  __shared__ float rsc[MOE_LAYER_MAX_T];
  const int tid = threadIdx.x;
  // the T quantizer blocks take the first block indices: dispatched first,
  // their chain (row loads, block reductions, codes) ends no later than the
  // router rows' (one token: decode step 20.81 -> 20.51 us against last)
  const int blk = (int)blockIdx.x >= T ? (int)blockIdx.x - T : E + (int)blockIdx.x;
  const bool rescale = in_rms > 0.0f;
  if (blk >= E) {
    const int t = blk - E;
    float sc = 1.0f;
    if (rescale) {
      rows_rms_scales(x + (size_t)t * H, 1, H, in_rms, tid, red, rsc);
      sc = rsc[0];
      if (tid == 0) xscale[t] = sc;
    }
    quantize_row_bf16_block(x + (size_t)t * H, H, xc + (size_t)t * (H / 2), xsc + (size_t)t * (H / 16),
                            xts + t, tid, 256, red, rescale, sc);
    return;
  }
  router_row_block(x, W, bias, T, E, H, blk, logits, tid, red, in_rms, rsc);
}

// ---------------------------------------------------------------- launchers
static size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

// Decode workspace: gate/up partials, then h^ (codes, block scales, tensor scales).
static DecodeWs carve_decode(void* ws, int H, int I, int npairs, size_t* total) {
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  size_t off = 0;
  auto take = [&](size_t b) { uint8_t* q = p ? p + off : nullptr; off += al256(b); return q; };
  DecodeWs w;
  w.gu = (float*)take((size_t)dec_ksplit(H) * npairs * 2 * I * sizeof(float));
  w.hc = take((size_t)npairs * I / 2);
  w.hsc = take((size_t)npairs * I / 16);
  w.hts = (float*)take((size_t)npairs * sizeof(float));
  if (total) *total = off;
  return w;
}

size_t decode_workspace_bytes(int E, int H, int I, int k, int T) {
  (void)E;
  size_t total = 0;
  carve_decode(nullptr, H, I, T * k, &total);
  return total;
}

// The down step: the 16-column slice kernel when the pairs fit one block
// (then the combine runs inside it), else one block per (pair, 64-row tile)
// followed by the combine kernel when a combine is asked for.
static size_t slice_lds_bytes(int npairs, int I) {
  return (size_t)npairs * I * 2 + (size_t)npairs * 16 * 4;
}
static bool slice_fits(int npairs, int H, int I) {
  return npairs <= SL_MAXP && I <= 32 * 4 * SL_CPQ && I / 16 <= 64 && H % 16 == 0 &&
         slice_lds_bytes(npairs, I) <= 56 * 1024;
}
// h mode: one token, one gate/up split, the slice kernel quantizing h itself
static bool decode_h_mode(int T, int npairs, int H, int I) {
  return T == 1 && dec_ks(H, T) == 1 && slice_fits(npairs, H, I) && I / 4 <= 64 * SL_HQR &&
         I / 32 <= 64;
}

// Whether the decode kernels take these shapes in gate/up format fmt: the
// codebook format needs whole 128-element groups per K-split and at most
// CB_GPW groups per wave.
bool decode_fmt_ok(int H, int T, int fmt) {
  if (fmt != FMT_CB3G128) return true;
  const int KS = dec_ks(H, T);
  if ((H / 128) % KS) return false;
  const int nw = dec_waves(H / 32 / KS);
  return (H / 128 / KS + nw - 1) / nw <= CB_GPW;
}

template <int MAXP, int PC, bool FUSED, int FMT>
static void launch_decode_pair(const FfnArgs& a, DecodeWs ws, const float* logits, int32_t* ids_out,
                               float* w_out, const uint16_t* residual, uint16_t* y, hipStream_t s,
                               const float* res_scale = nullptr) {
  const int npairs = a.T * a.k;
  const int KS = dec_ks(a.H, a.T);
  const int nw1 = dec_waves(a.H / 32 / KS);
  const int hm = decode_h_mode(a.T, npairs, a.H, a.I) ? 1 : 0;
  const size_t lds1 = (size_t)MAXP * a.H * 2 + (size_t)nw1 * MAXP * 64 * 4;
  // The fused layer ranks the logits inside every gate/up block when there
  // is one token (no extra launch on the critical path); with several
  // tokens every block would rank all of them, so one wave per token ranks
  // them once in the top-k kernel first.
  if constexpr (FUSED && MAXP > 1) {
    (void)launch_topk(logits, a.T, a.E, a.k, ids_out, w_out, s);
    gate_up_decode_kernel<MAXP, DEC_CPW, false, PC, FMT><<<dim3(npairs, a.I / 32, KS), 64 * nw1, lds1, s>>>(a, ws, logits, ids_out, w_out, hm);
  } else {
    gate_up_decode_kernel<MAXP, DEC_CPW, FUSED, PC, FMT><<<dim3(npairs, a.I / 32, KS), 64 * nw1, lds1, s>>>(a, ws, logits, ids_out, w_out, hm);
  }
  if (hm) {
    const size_t lds = slice_lds_bytes(npairs, a.I);
    if (a.h_ts) {                              // static h scale: h^ written by gate/up
      if (FUSED) down_slice_kernel<true, false><<<a.H / 16, 64 * npairs, lds, s>>>(a, ws, w_out, residual, y, res_scale);
      else down_slice_kernel<false, false><<<a.H / 16, 64 * npairs, lds, s>>>(a, ws, nullptr, nullptr, nullptr, nullptr);
    } else {
      if (FUSED) down_slice_kernel<true, true><<<a.H / 16, 64 * npairs, lds, s>>>(a, ws, w_out, residual, y, res_scale);
      else down_slice_kernel<false, true><<<a.H / 16, 64 * npairs, lds, s>>>(a, ws, nullptr, nullptr, nullptr, nullptr);
    }
    return;
  }
  h_quant_decode_kernel<<<npairs, 64 * ((a.I / 4 + 63) / 64), 0, s>>>(a, ws);
  if (slice_fits(npairs, a.H, a.I)) {
    const size_t lds = slice_lds_bytes(npairs, a.I);
    if (FUSED) down_slice_kernel<true, false><<<a.H / 16, 64 * npairs, lds, s>>>(a, ws, w_out, residual, y, res_scale);
    else down_slice_kernel<false, false><<<a.H / 16, 64 * npairs, lds, s>>>(a, ws, nullptr, nullptr, nullptr, nullptr);
  } else if (FUSED && a.T <= SL_TOKEN_MAX_T && slice_fits(a.k, a.H, a.I)) {
    // the fused layer at a few tokens: one slice block per (16 columns,
    // token), the combine in the block (no o round trip, no combine kernel)
    const size_t lds = slice_lds_bytes(a.k, a.I);
    down_slice_kernel<true, false><<<dim3(a.H / 16, a.T), 64 * a.k, lds, s>>>(a, ws, w_out, residual, y, res_scale);
  } else {
    const int nw2 = dec_waves(a.I / 32);
    const size_t lds2 = (size_t)MAXP * a.I * 2 + (size_t)nw2 * MAXP * 64 * 4;
    down_decode_kernel<MAXP, DEC_CPW, PC><<<dim3(npairs, a.H / 64), 64 * nw2, lds2, s>>>(a, ws);
    if (FUSED) (void)launch_combine(a.out, w_out, residual, a.T, a.k, a.H, y, s, res_scale);
  }
}

template <int FMT>
static void launch_ffn_decode_fmt(const FfnArgs& a, DecodeWs w, hipStream_t s) {
  if (a.T == 1) launch_decode_pair<1, 1, false, FMT>(a, w, nullptr, nullptr, nullptr, nullptr, nullptr, s);
  else if (a.T * a.k <= 512) launch_decode_pair<4, 8, false, FMT>(a, w, nullptr, nullptr, nullptr, nullptr, nullptr, s);
  else launch_decode_pair<4, 32, false, FMT>(a, w, nullptr, nullptr, nullptr, nullptr, nullptr, s);
}

hipError_t launch_ffn_decode(const FfnArgs& a, void* ws, hipStream_t s) {
  DecodeWs w = carve_decode(ws, a.H, a.I, a.T * a.k, nullptr);
  if (a.fmt == FMT_CB3G128) launch_ffn_decode_fmt<1>(a, w, s);
  else launch_ffn_decode_fmt<0>(a, w, s);
  return hipGetLastError();
}

// Fused layer workspace: logits, ids, w, x^ (codes, scales, ts), the decode
// workspace (gate/up partials, h^), o.
struct LayerWs {
  float* logits; int32_t* ids; float* w; uint8_t* xc; uint8_t* xs; float* xts;
  float* gu; float* out; float* xscale; uint16_t* xr;
};

static LayerWs carve_layer(void* ws, int E, int H, int I, int k, int T, size_t* total) {
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  size_t off = 0;
  auto take = [&](size_t b) { uint8_t* q = p ? p + off : nullptr; off += al256(b); return q; };
  LayerWs w;
  w.logits = (float*)take((size_t)T * E * 4);
  w.ids = (int32_t*)take((size_t)T * k * 4);
  w.w = (float*)take((size_t)T * k * 4);
  w.xc = take((size_t)T * H / 2);
  w.xs = take((size_t)T * H / 16);
  w.xts = (float*)take((size_t)T * 4);
  w.gu = (float*)take(decode_workspace_bytes(E, H, I, k, T));
  w.out = (float*)take((size_t)T * k * H * 4);
  w.xscale = (float*)take((size_t)T * 4);
  w.xr = (uint16_t*)take((size_t)T * H * 2);            // rescaled input rows (T > 1)
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
  if (L.in_rms > 0.0f && L.T > 1) {
    // several tokens: every router block would take every token's scale, so
    // the rows are rescaled once by the standalone kernel (the same routine,
    // the same bits) and the layer runs on them
    hipError_t e = launch_rms_norm(L.x, L.T, L.H, L.in_rms, w.xr, s);
    if (e != hipSuccess) return e;
    LayerArgs L2 = L;
    L2.x = w.xr;
    L2.in_rms = 0.0f;
    return launch_layer_decode(L2, ws, s);
  }
  router_quant_kernel<<<L.E + L.T, 256, 0, s>>>(L.x, L.W_r, L.bias, L.T, L.E, L.H, w.logits, w.xc, w.xs, w.xts,
                                                L.in_rms, w.xscale);
  FfnArgs a{};
  a.E = L.E; a.H = L.H; a.I = L.I; a.k = L.k; a.T = L.T; a.fmt = L.fmt;
  a.gate_up = L.gate_up; a.down = L.down;
  a.ts_gate = L.ts_gate; a.ts_up = L.ts_up; a.ts_down = L.ts_down; a.h_ts = L.h_ts;
  a.x_codes = w.xc; a.x_scales = w.xs; a.x_ts = w.xts;
  int32_t* ids_out = L.ids_out ? L.ids_out : w.ids;
  float* w_out = L.w_out ? L.w_out : w.w;
  a.ids = ids_out;
  a.out = w.out;
  DecodeWs dw = carve_decode(w.gu, L.H, L.I, L.T * L.k, nullptr);
  const uint16_t* res = L.residual ? L.x : nullptr;
  const float* rsc = L.residual && L.in_rms > 0.0f ? w.xscale : nullptr;
  if (L.fmt == FMT_CB3G128) {
    if (L.T == 1) launch_decode_pair<1, 1, true, 1>(a, dw, w.logits, ids_out, w_out, res, L.y, s, rsc);
    else launch_decode_pair<4, 8, true, 1>(a, dw, w.logits, ids_out, w_out, res, L.y, s, rsc);
  } else {
    if (L.T == 1) launch_decode_pair<1, 1, true, 0>(a, dw, w.logits, ids_out, w_out, res, L.y, s, rsc);
    else launch_decode_pair<4, 8, true, 0>(a, dw, w.logits, ids_out, w_out, res, L.y, s, rsc);
  }
  return hipGetLastError();
}

}  // namespace moe
