// Softmax top-k router: fp32 logits of the bf16 hidden state against fp32
// router weights (+ optional per-expert bias), then per token the k largest
// logits (ties to the lower expert id) and their softmax renormalised over the
// selected k.  Each token runs only some of the experts (blog "Capy Flash
// ...", section "Where the experts live"); the picked experts come in rank
// order (forum repost, paragraph "Where it stands").
#include "../../include/moe.h"
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// ---------------------------------------------------------------- small T: GEMV
// One 256-thread block per router row (router_row_block in common.hpp; the
// fused decode layer uses the same routine, so both give identical logits).
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int H,
                                                          float* __restrict__ logits) {
  __shared__ float red[64];
  router_row_block(x, W, bias, T, E, H, blockIdx.x, logits, threadIdx.x, red);
}

// ---------------------------------------------------------------- large T: GEMM
// 64 tokens x 64 experts per 256-thread block, K step 32, fp32 FMA from LDS
// tiles; each thread owns a 4x4 patch.
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int H,
                                                          float* __restrict__ logits) {
  __shared__ float As[32][65];
  __shared__ float Bs[32][65];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
  const int tr = tid / 16, tc = tid % 16;               // 16 x 16 threads, 4x4 each
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += 32) {
    // A: 64 tokens x 32 k (bf16) -> As[k][t]; B: 64 experts x 32 k -> Bs[k][e]
    for (int i = tid; i < 64 * 32; i += 256) {
      int r = i / 32, c = i % 32;
      int t = t0 + r, e = e0 + r;
      As[c][r] = t < T ? bf16_to_f32(x[(size_t)t * H + k0 + c]) : 0.0f;
      Bs[c][r] = e < E ? W[(size_t)e * H + k0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][tr * 4 + i]; b[i] = Bs[kk][tc * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int t = t0 + tr * 4 + i, e = e0 + tc * 4 + j;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.0f);
    }
}

// ---------------------------------------------------------------- large T: matrix cores
// logits = x W_r^T with W_r split exactly into three bf16 parts while it is
// staged into LDS (hi = bf16(W), mid = bf16(W - hi), lo = bf16(W - hi - mid):
// 3 x 8 significant bits cover fp32's 24).  x is bf16, so every product of x
// with a part is exact in fp32, and the three v_mfma_f32_32x32x16_bf16 passes
// (smallest part first) accumulate in fp32 like an fp32 GEMM.  Block = 128
// tokens x RM_BN = 64 experts, 256 threads (2 x 2 waves of 64 x 32), K step
// 64; the next step's global loads are in flight during the current step's
// MFMAs.  64 experts per block rather than 128: twice the blocks and 46 KB of
// LDS, so two or three blocks share a CU and hide each other's load waits
// (router and top-k at 2,560 / 4,096 / 8,192 tokens 102 / 102 / 109 ->
// 57 / 60 / 85 us).  Needs H % 64 == 0.
constexpr int RG_BM = 128, RG_BN = 128, RG_BK = 64, RG_LDK = RG_BK + 8;
constexpr int RM_BN = 64;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> their three bf16 parts, each part's pair packed in one
// dword (first value in the low half): hi = bf16(w), mid = bf16(w - hi),
// lo = bf16(w - hi - mid), rounded to nearest even by the hardware pair
// conversion; the differences are exact in fp32, so hi + mid + lo = w.
__device__ __forceinline__ void split3_pk(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  auto cvt = [](float2_t f) {
    const bf16x2_t v = __builtin_convertvector(f, bf16x2_t);
    return *reinterpret_cast<const uint32_t*>(&v);
  };
  auto widen = [](uint32_t q) { return float2_t{__uint_as_float(q << 16), __uint_as_float(q & 0xFFFF0000u)}; };
  const float2_t w = {a, b};
  hi = cvt(w);
  const float2_t r1 = w - widen(hi);
  mid = cvt(r1);
  const float2_t r2 = r1 - widen(mid);
  lo = cvt(r2);
}

// (token tile, expert tile) of this block for the token-tile x expert-tile
// GEMM grids: blocks are dealt to the eight XCDs round-robin in dispatch
// order, so each XCD's consecutive blocks take every expert tile of one token
// tile before the next token tile: the token rows (the large operand, read
// once per expert tile) then come from that XCD's L2 after the first read
// instead of from HBM once per expert tile.  A bijection on the grid; grids
// whose token-tile count is not a multiple of eight keep the plain order.
__device__ __forceinline__ void router_tile_of_block(int& tt, int& et) {
  const int ntok = gridDim.x, nexp = gridDim.y;
  const int b = blockIdx.x + ntok * blockIdx.y;
  if (ntok % 8 == 0) {
    const int xcd = b & 7, i = b >> 3;
    tt = (i / nexp) * 8 + xcd;
    et = i % nexp;
  } else {
    tt = blockIdx.x;
    et = blockIdx.y;
  }
}

__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int H,
                                                          float* __restrict__ logits) {
  constexpr int BN = RM_BN;
  constexpr int NJ = BN / 64;                      // 32-expert MFMA tiles per wave
  constexpr int WTPR = 256 / BN;                   // W staging threads per expert row
  constexpr int WV = RG_BK / WTPR;                 // W values each stages per step (32 or 16)
  __shared__ __align__(16) uint16_t As[RG_BM][RG_LDK];
  __shared__ __align__(16) uint16_t Bs[3][BN][RG_LDK];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;             // wave patch: tokens wm*64, experts wn*BN/2
  int tt, et;
  router_tile_of_block(tt, et);
  const int t0 = tt * RG_BM, e0 = et * BN;
  // staging roles: x tile row r, K half hf (32 elements); W row rw, part
  // qw of WV elements
  const int r = tid >> 1, hf = tid & 1;
  const int rw = tid / WTPR, qw = tid % WTPR;
  const bool tv = t0 + r < T, ev = e0 + rw < E;
  const uint16_t* xr = x + (size_t)(tv ? t0 + r : 0) * H + 32 * hf;    // clamped: always valid
  const float* wr = W + (size_t)(ev ? e0 + rw : 0) * H + WV * qw;
  u32x4 xa[4];
  float4_t wa[WV / 4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const u32x4*>(xr + 8 * i);
#pragma unroll
  for (int i = 0; i < WV / 4; ++i) wa[i] = *reinterpret_cast<const float4_t*>(wr + 4 * i);

  float16_t acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  for (int k0 = 0; k0 < H; k0 += RG_BK) {
    // ---- stage: x as is, W split into three bf16 parts
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&As[r][32 * hf + 8 * i]) = tv ? xa[i] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < WV / 4; i += 2) {
      uint32_t p[3][4];
      for (int wd = 0; wd < 4; ++wd) {
        auto wf = [&](int c) { return ev ? wa[i + (c >> 2)][c & 3] : 0.0f; };
        split3_pk(wf(2 * wd), wf(2 * wd + 1), p[0][wd], p[1][wd], p[2][wd]);
      }
#pragma unroll
      for (int q = 0; q < 3; ++q)
        *reinterpret_cast<u32x4*>(&Bs[q][rw][WV * qw + 4 * i]) = u32x4{p[q][0], p[q][1], p[q][2], p[q][3]};
    }
    __syncthreads();
    // ---- next step's loads in flight during this step's MFMAs
    if (k0 + RG_BK < H) {
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const u32x4*>(xr + k0 + RG_BK + 8 * i);
#pragma unroll
      for (int i = 0; i < WV / 4; ++i) wa[i] = *reinterpret_cast<const float4_t*>(wr + k0 + RG_BK + 4 * i);
    }
#pragma unroll
    for (int kk = 0; kk < RG_BK; kk += 16) {
      bf16x8_t af[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[wm * 64 + i * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int q = 2; q >= 0; --q) {                 // lo, mid, hi
        bf16x8_t bq[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          bq[j] = *reinterpret_cast<const bf16x8_t*>(
              &Bs[q][wn * (BN / 2) + j * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bq[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // ---- epilogue: acc[i][j][q] is row wm*64 + i*32 + (q%4) + 8(q/4) + 4(lane/32),
  // column wn*BN/2 + j*32 + lane%32 of the tile
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = e0 + wn * (BN / 2) + j * 32 + (lane & 31);
    if (e >= E) continue;
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = t0 + wm * 64 + i * 32 + (q & 3) + 8 * (q >> 2) + 4 * (lane >> 5);
        if (t < T) logits[(size_t)t * E + e] = acc[i][j][q] + b;
      }
  }
}

// Large T (>= RM256_MIN_T): the same GEMM on 256-token x 128-expert tiles, 512
// threads (4 x 2 waves of 64 x 64).  Splitting W into its three bf16 parts is
// VALU work per block; twice the tokens per W tile halve it per token (router
// 0.70 -> ~0.5 ms at 65,536 tokens; below 16k tokens the halved block count
// costs more).

__global__ __launch_bounds__(512) void router_mfma256_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int H,
                                                          float* __restrict__ logits) {
  __shared__ __align__(16) uint16_t As[2 * RG_BM][RG_LDK];
  __shared__ __align__(16) uint16_t Bs[3][RG_BN][RG_LDK];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  int tt, et;
  router_tile_of_block(tt, et);
  const int t0 = tt * (2 * RG_BM), e0 = et * RG_BN;
  // staging roles: x row r (of 256), K half hf (32 elements); W row rb (of
  // 128), K quarter qb (16 elements)
  const int r = tid >> 1, hf = tid & 1, rb = tid >> 2, qb = tid & 3;
  const bool tv = t0 + r < T, ev = e0 + rb < E;
  const uint16_t* xr = x + (size_t)(tv ? t0 + r : 0) * H + 32 * hf;    // clamped: always valid
  const float* wr = W + (size_t)(ev ? e0 + rb : 0) * H + 16 * qb;
  u32x4 xa[4];
  float4_t wa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const u32x4*>(xr + 8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) wa[i] = *reinterpret_cast<const float4_t*>(wr + 4 * i);

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  for (int k0 = 0; k0 < H; k0 += RG_BK) {
    // ---- stage: x as is, W split into three bf16 parts
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&As[r][32 * hf + 8 * i]) = tv ? xa[i] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      uint32_t p[3][4];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        auto wf = [&](int c) { return ev ? wa[i + (c >> 2)][c & 3] : 0.0f; };
        split3_pk(wf(2 * wd), wf(2 * wd + 1), p[0][wd], p[1][wd], p[2][wd]);
      }
#pragma unroll
      for (int q = 0; q < 3; ++q)
        *reinterpret_cast<u32x4*>(&Bs[q][rb][16 * qb + 4 * i]) = u32x4{p[q][0], p[q][1], p[q][2], p[q][3]};
    }
    __syncthreads();
    // ---- next step's loads in flight during this step's MFMAs
    if (k0 + RG_BK < H) {
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const u32x4*>(xr + k0 + RG_BK + 8 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i) wa[i] = *reinterpret_cast<const float4_t*>(wr + k0 + RG_BK + 4 * i);
    }
#pragma unroll
    for (int kk = 0; kk < RG_BK; kk += 16) {
      bf16x8_t af[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[wm * 64 + i * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int q = 2; q >= 0; --q) {                 // lo, mid, hi
        bf16x8_t bq[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bq[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[q][wn * 64 + j * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bq[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // ---- epilogue: acc[i][j][q] is row wm*64 + i*32 + (q%4) + 8(q/4) + 4(lane/32),
  // column wn*64 + j*32 + lane%32 of the tile
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + wn * 64 + j * 32 + (lane & 31);
    if (e >= E) continue;
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = t0 + wm * 64 + i * 32 + (q & 3) + 8 * (q >> 2) + 4 * (lane >> 5);
        if (t < T) logits[(size_t)t * E + e] = acc[i][j][q] + b;
      }
  }
}

// Mid token counts (tens to about a thousand tokens): the 128 x 64 tiles above
// leave most of the chip idle (8 blocks at 128 tokens) and walk H in a serial
// chain of staged steps.  Here one block of eight waves owns a 32-token x
// 32-expert tile and each wave one eighth of H: x (bf16) and W (fp32, split
// into the same three bf16 parts in registers) go straight from memory into
// the MFMA operands (lane l: row l%32, eight k values at 8*(l/32) of each
// 16-wide group), NB groups of loads in flight while the previous NB are
// multiplied; the eight partial tiles are summed in LDS in wave order
// (deterministic) and the bias added once.
constexpr int RS_WAVES = 8, RS_NB = 4;
constexpr int RS16_MAX_T = 128;         // 16 x 16 tiles up to here (below)
constexpr int RS_MAX_T = 1280;          // above: the 128 x 64 tiles (router and top-k at 1,024 / 2,048
                                        // tokens: 46 / 83 us here, 53 / 54 us there)
constexpr int RM256_MIN_T = 16384;      // 256-token tiles from here (fewer blocks below it)

__global__ __launch_bounds__(64 * RS_WAVES) void router_splitk_kernel(const uint16_t* __restrict__ x,
                                                                      const float* __restrict__ W,
                                                                      const float* __restrict__ bias,
                                                                      int T, int E, int H,
                                                                      float* __restrict__ logits) {
  __shared__ float red[RS_WAVES][32][33];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int r = lane & 31, hf = lane >> 5;
  // padding rows read row 0 of the tile (valid); their outputs are not stored
  const uint16_t* xr = x + (size_t)(t0 + r < T ? t0 + r : t0) * H + 8 * hf;
  const float* wr = W + (size_t)(e0 + r < E ? e0 + r : e0) * H + 8 * hf;
  const int G = H / 16;                                   // 16-wide k groups
  const int g0 = wv * G / RS_WAVES, g1 = (wv + 1) * G / RS_WAVES;

  struct Batch { u32x4 xa[RS_NB]; float4_t wa[RS_NB][2]; };
  auto load = [&](Batch& b, int gb) {
#pragma unroll
    for (int i = 0; i < RS_NB; ++i) {
      const int g = gb + i < g1 ? gb + i : g1 - 1;         // clamped: always in the slice
      b.xa[i] = *reinterpret_cast<const u32x4*>(xr + 16 * g);
      b.wa[i][0] = *reinterpret_cast<const float4_t*>(wr + 16 * g);
      b.wa[i][1] = *reinterpret_cast<const float4_t*>(wr + 16 * g + 4);
    }
  };
  float16_t acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
  auto mul = [&](const Batch& b, int gb) {
#pragma unroll
    for (int i = 0; i < RS_NB; ++i) {
      if (gb + i >= g1) break;
      uint32_t p[3][4];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        auto wf = [&](int c) { return b.wa[i][c >> 2][c & 3]; };
        split3_pk(wf(2 * wd), wf(2 * wd + 1), p[0][wd], p[1][wd], p[2][wd]);
      }
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&b.xa[i]);
#pragma unroll
      for (int q = 2; q >= 0; --q) {                     // lo, mid, hi
        const u32x4 pq = {p[q][0], p[q][1], p[q][2], p[q][3]};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, *reinterpret_cast<const bf16x8_t*>(&pq), acc, 0, 0, 0);
      }
    }
  };
  Batch b0, b1;
  load(b0, g0);
  load(b1, g0 + RS_NB);
  for (int gb = g0; gb < g1; gb += 2 * RS_NB) {
    mul(b0, gb);
    load(b0, gb + 2 * RS_NB);
    mul(b1, gb + RS_NB);
    load(b1, gb + 3 * RS_NB);
  }
  // acc[q]: token row (q%4) + 8(q/4) + 4*hf, expert column r
#pragma unroll
  for (int q = 0; q < 16; ++q) red[wv][(q & 3) + 8 * (q >> 2) + 4 * hf][r] = acc[q];
  __syncthreads();
  for (int o = threadIdx.x; o < 32 * 32; o += 64 * RS_WAVES) {
    const int row = o >> 5, col = o & 31;
    const int t = t0 + row, e = e0 + col;
    if (t >= T || e >= E) continue;
    float s = red[0][row][col];
#pragma unroll
    for (int w = 1; w < RS_WAVES; ++w) s += red[w][row][col];
    logits[(size_t)t * E + e] = s + (bias ? bias[e] : 0.0f);
  }
}

// Few tokens (up to a few hundred): the 32 x 32 tiles above leave most CUs
// idle (64 blocks at 128 tokens).  Same scheme on 16-token x 16-expert tiles
// with v_mfma_f32_16x16x32_bf16: lane l gives row l%16 and eight k values at
// 8*(l/16) of each 32-wide group and gets rows 4*(l/16)..+3 of column l%16.
// Needs H % 256 == 0 (every wave's slice of H non-empty).
typedef float float4v_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64 * RS_WAVES) void router_splitk16_kernel(const uint16_t* __restrict__ x,
                                                                        const float* __restrict__ W,
                                                                        const float* __restrict__ bias,
                                                                        int T, int E, int H,
                                                                        float* __restrict__ logits) {
  __shared__ float red[RS_WAVES][16][17];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
  const int r = lane & 15, qd = lane >> 4;
  // padding rows read row 0 of the tile (valid); their outputs are not stored
  const uint16_t* xr = x + (size_t)(t0 + r < T ? t0 + r : t0) * H + 8 * qd;
  const float* wr = W + (size_t)(e0 + r < E ? e0 + r : e0) * H + 8 * qd;
  const int G = H / 32;                                   // 32-wide k groups
  const int g0 = wv * G / RS_WAVES, g1 = (wv + 1) * G / RS_WAVES;

  struct Batch { u32x4 xa[RS_NB]; float4_t wa[RS_NB][2]; };
  auto load = [&](Batch& b, int gb) {
#pragma unroll
    for (int i = 0; i < RS_NB; ++i) {
      const int g = gb + i < g1 ? gb + i : g1 - 1;         // clamped: always in the slice
      b.xa[i] = *reinterpret_cast<const u32x4*>(xr + 32 * g);
      b.wa[i][0] = *reinterpret_cast<const float4_t*>(wr + 32 * g);
      b.wa[i][1] = *reinterpret_cast<const float4_t*>(wr + 32 * g + 4);
    }
  };
  float4v_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto mul = [&](const Batch& b, int gb) {
#pragma unroll
    for (int i = 0; i < RS_NB; ++i) {
      if (gb + i >= g1) break;
      uint32_t p[3][4];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        auto wf = [&](int c) { return b.wa[i][c >> 2][c & 3]; };
        split3_pk(wf(2 * wd), wf(2 * wd + 1), p[0][wd], p[1][wd], p[2][wd]);
      }
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&b.xa[i]);
#pragma unroll
      for (int q = 2; q >= 0; --q) {                     // lo, mid, hi
        const u32x4 pq = {p[q][0], p[q][1], p[q][2], p[q][3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, *reinterpret_cast<const bf16x8_t*>(&pq), acc, 0, 0, 0);
      }
    }
  };
  Batch b0, b1;
  load(b0, g0);
  load(b1, g0 + RS_NB);
  for (int gb = g0; gb < g1; gb += 2 * RS_NB) {
    mul(b0, gb);
    load(b0, gb + 2 * RS_NB);
    mul(b1, gb + RS_NB);
    load(b1, gb + 3 * RS_NB);
  }
  // acc[j]: token row 4*qd + j, expert column r
#pragma unroll
  for (int j = 0; j < 4; ++j) red[wv][4 * qd + j][r] = acc[j];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
    const int t = t0 + row, e = e0 + col;
    if (t < T && e < E) {
      float s = red[0][row][col];
#pragma unroll
      for (int w = 1; w < RS_WAVES; ++w) s += red[w][row][col];
      logits[(size_t)t * E + e] = s + (bias ? bias[e] : 0.0f);
    }
  }
}

// ---------------------------------------------------------------- top-k
// One wave per token (topk_wave: a lower bound from the lane maxima, then
// the few candidates above it ranked; exact ties go to the lower id), then
// the winners' softmax renormalised over the k.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  __shared__ int scr[4][TOPK_SCR_INTS];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                  // wave-uniform; no block barrier below
  int id;
  float wt;
  topk_wave_any(logits + (size_t)t * E, E, k, lane, scr[threadIdx.x >> 6], &id, &wt);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
  }
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const float* W_r, const float* bias, int T, int E,
                         int H, int k, int32_t* ids, float* w, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= 16 && H % 4 == 0 && H <= 4096) {
    router_gemv_kernel<<<E, 256, 0, s>>>(x, W_r, bias, T, E, H, logits);
  } else if (T <= RS16_MAX_T && H % 256 == 0) {
    router_splitk16_kernel<<<dim3((T + 15) / 16, (E + 15) / 16), 64 * RS_WAVES, 0, s>>>(x, W_r, bias, T, E, H, logits);
  } else if (T <= RS_MAX_T && H % 128 == 0) {
    router_splitk_kernel<<<dim3((T + 31) / 32, (E + 31) / 32), 64 * RS_WAVES, 0, s>>>(x, W_r, bias, T, E, H, logits);
  } else if (H % RG_BK == 0 && T >= RM256_MIN_T) {
    router_mfma256_kernel<<<dim3((T + 2 * RG_BM - 1) / (2 * RG_BM), (E + RG_BN - 1) / RG_BN), 512, 0, s>>>(x, W_r, bias, T, E, H, logits);
  } else if (H % RG_BK == 0) {
    router_mfma_kernel<<<dim3((T + RG_BM - 1) / RG_BM, (E + RM_BN - 1) / RM_BN), 256, 0, s>>>(x, W_r, bias, T, E, H,
                                                                                            logits);
  } else {
    router_gemm_kernel<<<dim3((E + 63) / 64, (T + 63) / 64), 256, 0, s>>>(x, W_r, bias, T, E, H, logits);
  }
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
