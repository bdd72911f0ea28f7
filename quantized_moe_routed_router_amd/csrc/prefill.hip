// Prefill expert FFN: grouped GEMMs on matrix cores over the token-by-expert
// permutation, W4A4 NVFP4 (or 3-bit fp16-codebook gate/up weights).
//
// The pages: routed experts with gate/up weights and down projections, and
// 3-bit q3_g128_fp16 codebook weights as the alternative format (release post
// "capy-flash v0.7.1", section "What shipped"); NVFP4 activations and weights
// on the GPU's W4A4 path (section "Why it matters").
//
// Pipeline (one call, no host round trip):
//   permute   stable counting sort of the (t, slot) pairs by expert, plus the
//             per-expert count of BM-row tiles (prefix in tile_prefix) and one
//             record per tile {expert, first row, end row} (tile_map); the
//             same for the 32-row second list (tile_prefix2, tile_map2)
//   gate/up   per (expert, row tile, column tile): rows are the expert's
//             pairs (x^ rows gathered through perm), cols 64-row packed weight
//             tiles (32 gate rows + the same 32 up rows), multiplied with
//             v_mfma_f32_32x32x16_f16 in fp32 on operands dequantized to f16
//             (E2M1 x E4M3 is exact in f16, so is a codebook entry).  Few rows
//             per expert: 32-row tiles, one wave per tile pair, operands
//             straight to registers (K split at a handful of rows); else
//             256 x 256 (or 128 x 128) block tiles staged through LDS, where
//             the experts under 128 rows keep 32-row tiles (a second list, run
//             by trailing blocks of the same launch).
//             Epilogue: h = SiLU(g ts_x ts_g) * (u ts_x ts_u), fp32, sorted order.
//   h quant   NVFP4 of each h row (one tensor scale per (t, slot) row)
//   down      same GEMM on h^ rows; epilogue scales by ts_h ts_down and
//             scatters o rows back to (t, slot) through perm.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int BM = 128, BN = 128, BK = 64, LDSK = BK + 8;   // +8 halves: bank spread
constexpr int PF_THREADS = 256;
// Up to SPLIT_MAX_N (token, slot) rows (SPLIT_MAX_N_NVFP4 for NVFP4 gate/up)
// ksplit waves of one block (ksplit <= SPLIT_K_MAX) share each 32-row gate/up
// item, each taking 1/ksplit of K, and sum their accumulators in LDS: few
// expert tiles exist there, and a wave walking all of K alone is VALU-
// (codebook) or latency- (NVFP4, at a handful of rows) bound.  Measured layer
// step: codebook 97 -> 51 us at 1 token; NVFP4 71 -> 44 us at 1 token and
// 67 -> 65 us at 4, slower from 8 tokens (the split waves' registers).
constexpr int SPLIT_MAX_N = 256, SPLIT_MAX_N_NVFP4 = 40, SPLIT_K_MAX = 4;

struct PrefillWs {
  int32_t* perm_ws;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  int32_t* tile_prefix;
  int32_t* tile_map;     // per tile {expert, first row, end row of the expert, 0}
  int32_t* tile_prefix2; // the 256-row tiling's second list: 32-row tiles of the
  int32_t* tile_map2;    // experts with fewer than BB_SPLIT_ROWS rows
  float* h;
  uint8_t* hq_codes;
  uint8_t* hq_scales;
  float* hq_ts;
};

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

static PrefillWs carve(void* ws, int E, int I, int k, int T, size_t* total) {
  const size_t N = (size_t)T * k;
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) { uint8_t* q = p ? p + off : nullptr; off += align256(bytes); return q; };
  PrefillWs w;
  w.perm_ws = (int32_t*)take(permute_workspace_bytes(T, k, E));
  w.counts = (int32_t*)take((size_t)E * 4);
  w.offsets = (int32_t*)take((size_t)(E + 1) * 4);
  w.perm = (int32_t*)take(N * 4);
  w.inv = (int32_t*)take(N * 4);
  w.tile_prefix = (int32_t*)take((size_t)(E + 1) * 4);
  w.tile_map = (int32_t*)take(((N + 31) / 32 + (size_t)E) * 16);   // enough for 32-, 128- and 256-row tiles
  w.tile_prefix2 = (int32_t*)take((size_t)(E + 1) * 4);
  w.tile_map2 = (int32_t*)take(((N + 31) / 32 + (size_t)E) * 16);
  w.h = (float*)take(N * I * 4);
  w.hq_codes = take(N * I / 2);
  w.hq_scales = take(N * I / 16);
  w.hq_ts = (float*)take(N * 4);
  if (total) *total = off;
  return w;
}

size_t prefill_workspace_bytes(int E, int H, int I, int k, int T) {
  (void)H;
  size_t total = 0;
  carve(nullptr, E, I, k, T, &total);
  return total;
}


// 32 NVFP4 elements (16 code bytes, 2 E4M3 scales) -> 32 f16 values e2m1*s
__device__ __forceinline__ void dequant32_nvfp4(u32x4 cw, uint32_t sw, half2_t (&o)[16]) {
  const half2_t s = e4m3x2_to_f16x2(sw);
  const half2_t a = {s.x, s.x}, b = {s.y, s.y};
  o[0] = fp4x2_to_f16x2<0>(cw.x) * a; o[1] = fp4x2_to_f16x2<1>(cw.x) * a;
  o[2] = fp4x2_to_f16x2<2>(cw.x) * a; o[3] = fp4x2_to_f16x2<3>(cw.x) * a;
  o[4] = fp4x2_to_f16x2<0>(cw.y) * a; o[5] = fp4x2_to_f16x2<1>(cw.y) * a;
  o[6] = fp4x2_to_f16x2<2>(cw.y) * a; o[7] = fp4x2_to_f16x2<3>(cw.y) * a;
  o[8] = fp4x2_to_f16x2<0>(cw.z) * b; o[9] = fp4x2_to_f16x2<1>(cw.z) * b;
  o[10] = fp4x2_to_f16x2<2>(cw.z) * b; o[11] = fp4x2_to_f16x2<3>(cw.z) * b;
  o[12] = fp4x2_to_f16x2<0>(cw.w) * b; o[13] = fp4x2_to_f16x2<1>(cw.w) * b;
  o[14] = fp4x2_to_f16x2<2>(cw.w) * b; o[15] = fp4x2_to_f16x2<3>(cw.w) * b;
}

__device__ __forceinline__ half8_t cat8(half2_t a, half2_t b, half2_t c, half2_t d) {
  const half4_t lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const half4_t hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight E2M1 codes (one dword: element 2j in byte j's low nibble) times the
// block scale s (both halves) -> eight f16 values, exact.  The hardware's
// scaled conversion applies only the exponent of its scale operand (a device
// probe over all code bytes and E4M3 scales), so the scale is an f16 multiply.
__device__ __forceinline__ half8_t dq8(uint32_t w, half2_t s) {
  return cat8(fp4x2_to_f16x2<0>(w) * s, fp4x2_to_f16x2<1>(w) * s, fp4x2_to_f16x2<2>(w) * s,
              fp4x2_to_f16x2<3>(w) * s);
}

__device__ __forceinline__ void store32(_Float16* dst, const half2_t (&o)[16]) {
  u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = *reinterpret_cast<const u32x4*>(&o[4 * i]);
}

__device__ __forceinline__ void zero32(_Float16* dst) {
  u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = u32x4{0, 0, 0, 0};
}

// MODE 0: gate/up NVFP4, 1: gate/up codebook, 2: down
template <int MODE>
__global__ __launch_bounds__(PF_THREADS) void grouped_gemm_kernel(FfnArgs a, PrefillWs w, int n_ntiles) {
  __shared__ __align__(16) _Float16 As[BM][LDSK];
  __shared__ __align__(16) _Float16 Bs[BN][LDSK];
  __shared__ int row_pos[BM];          // sorted position of each tile row, -1 if padding
  __shared__ float row_scale[BM];      // ts of the row's activation (x or h)

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int gm = blockIdx.x / n_ntiles, nt = blockIdx.x % n_ntiles;
  const int total_tiles = w.tile_prefix[a.E];
  if (gm >= total_tiles) return;
  const int4 tr = reinterpret_cast<const int4*>(w.tile_map)[gm];   // {expert, first row, end row}
  const int e = tr.x, row0 = tr.y, row_end = tr.z;

  const bool down = MODE == 2;
  const int K = down ? a.I : a.H;               // contraction length
  const size_t w_tile_bytes = (MODE == 1) ? cb_tile_bytes(K) : tile_bytes(K);
  const size_t w_expert_bytes = down ? down_expert_bytes(a.H, a.I)
                                     : (MODE == 1 ? cb_gate_up_expert_bytes(a.H, a.I) : gate_up_expert_bytes(a.H, a.I));
  const uint8_t* wbase = (down ? a.down : a.gate_up) + (size_t)e * w_expert_bytes + (size_t)(nt * 2) * w_tile_bytes;

  if (tid < BM) {
    const int pos = row0 + tid;
    int rp = -1;
    float sc = 0.0f;
    if (pos < row_end) {
      rp = pos;
      sc = down ? w.hq_ts[pos] : a.x_ts[w.perm[pos] / a.k];
    }
    row_pos[tid] = rp;
    row_scale[tid] = sc;
  }
  __syncthreads();

  // A-load role: row ar, half ah (32 elements); B-load role: tile jj, chunk c, lane bl
  const int ar = tid >> 1, ah = tid & 1;
  const int arow_pos = row_pos[ar];
  const uint8_t* acodes = nullptr;
  const uint8_t* ascales = nullptr;
  if (arow_pos >= 0) {
    if (down) {
      acodes = w.hq_codes + (size_t)arow_pos * (a.I / 2);
      ascales = w.hq_scales + (size_t)arow_pos * (a.I / 16);
    } else {
      const int t = w.perm[arow_pos] / a.k;
      acodes = a.x_codes + (size_t)t * (a.H / 2);
      ascales = a.x_scales + (size_t)t * (a.H / 16);
    }
  }
  const int bj = tid >> 7, bc = (tid >> 6) & 1, bl = tid & 63;
  const uint8_t* btile = wbase + (size_t)bj * w_tile_bytes;

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += BK) {
    // ---- A: activation rows (NVFP4), gathered through perm
    {
      half2_t o[16];
      _Float16* dst = &As[ar][32 * ah];
      if (acodes) {
        const int kk = k0 + 32 * ah;
        u32x4 cw = *reinterpret_cast<const u32x4*>(acodes + kk / 2);
        uint32_t sw = *reinterpret_cast<const uint16_t*>(ascales + kk / 16);
        dequant32_nvfp4(cw, sw, o);
        store32(dst, o);
      } else {
        zero32(dst);
      }
    }
    // ---- B: packed weight tile (two 64-row tiles), chunk k0/32 + bc
    {
      half2_t o[16];
      const int ck = k0 / 32 + bc;
      if (MODE == 1) {
        const uint8_t* grp = btile + (size_t)(ck >> 2) * cb_group_bytes();
        const uint32_t* iw = reinterpret_cast<const uint32_t*>(grp + bl * 48);
        const int d = ck & 3;
        u32x4 cb = *reinterpret_cast<const u32x4*>(grp + 64 * 48 + bl * 16);
        dequant32_cb(iw[d], iw[4 + d], iw[8 + d], cb, o);
      } else {
        u32x4 cw = *reinterpret_cast<const u32x4*>(btile + (size_t)ck * 1024 + bl * 16);
        uint32_t sw = *reinterpret_cast<const uint16_t*>(btile + tile_scale_offset(K) + (size_t)(ck >> 2) * 512 + bl * 8 + (ck & 3) * 2);
        dequant32_nvfp4(cw, sw, o);
      }
      store32(&Bs[bj * 64 + bl][32 * bc], o);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      half8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(&As[wm * 64 + i * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(&Bs[wn * 64 + j * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue.  acc[i][j][r]: row wm*64 + i*32 + (r%4) + 8*(r/4) + 4*(lane/32),
  // col wn*64 + j*32 + lane%32 of the 128x128 tile.
  if (!down) {
    const float tsg = (MODE == 0) ? a.ts_gate[e] : 1.0f;
    const float tsu = (MODE == 0) ? a.ts_up[e] : 1.0f;
    const int n = (nt * 2 + wn) * 32 + (lane & 31);           // h column (gate/up row)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * 64 + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
        const int pos = row_pos[rl];
        if (pos < 0) continue;
        const float sx = row_scale[rl];
        const float g = acc[i][0][r] * (sx * tsg);
        const float u = acc[i][1][r] * (sx * tsu);
        w.h[(size_t)pos * a.I + n] = silu_mul(g, u);
      }
  } else {
    const float tsd = a.ts_down[e];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = nt * BN + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * 64 + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
          const int pos = row_pos[rl];
          if (pos < 0) continue;
          const int pair = w.perm[pos];
          a.out[(size_t)pair * a.H + n] = acc[i][j][r] * (row_scale[rl] * tsd);
        }
      }
  }
}

// ---------------------------------------------------------------- 256 x 256 tiles
// The main prefill GEMM: one 256 x 256 output tile per block of 8 waves
// (2 x 4), each wave a 128 x 64 patch (4 x 2 tiles of v_mfma_f32_32x32x16_f16,
// 128 accumulator registers), two waves per SIMD so one wave's dequantization
// runs while the other's MFMAs execute.  LDS holds two K-step buffers of A
// (256 activation rows) and B (256 weight rows) dequantized to f16 (147,456 B
// of the 160 KiB).  Step s: the MFMAs on buffer s%2 with the registers fetched
// for step s+1 dequantized into buffer (s+1)%2 alongside, step s+3's global
// loads issued (two register sets), one barrier.  A buffer is rewritten only
// after every wave has passed the barrier that ends the step reading it.
// Staging: wave w dequantizes tile rows 32w .. 32w+31 of A (lane l: row
// 32w + l%32, chunk l/32 of the step) and chunk w%2 of the step of packed
// weight tile w/2 for B (lane = weight row: one 1 KiB-contiguous load; the
// codebook mode: a thread pair per weight row, one chunk each).
// k order: in K step s, lane l of a 32-row fragment holds chunk 2s + l/32 of
// its row (32 elements) and MFMA kk of the step takes the chunk's elements
// 8kk .. 8kk+7, for A and B alike, so every product is summed once.  Loads are
// straight-line: a padding row reads a valid row with scale 0.
constexpr int BB = 256, BBK = 64, BLDK = BBK + 8, BTHREADS = 512;
constexpr int MB = 32, MWAVES = 4;    // the 32-row kernel's tile rows and waves per block
constexpr int OPND_F16 = BB * BLDK * 2;          // one operand's K step in LDS: 256 rows x 72 halves
constexpr int EPI_BYTES = 8 * 64 * 36 * 4;       // the epilogue's eight 64 x 36-float wave regions

template <int MODE, int KS>
__device__ __forceinline__ void mid_tile_body(const FfnArgs& a, const PrefillWs& w, int n_ptiles, int blk, int wv,
                                              int lane);

// Whether the 256-row gate/up epilogue codes h^ (a static h scale per expert
// and no debug copies of h or h^ requested).
__host__ __device__ inline bool h_coded_in_gemm(const FfnArgs& a) {
  return a.h_ts && !a.dbg_h && !a.dbg_h_codes && !a.dbg_h_scales && !a.dbg_h_ts;
}

// Blocks from n_big on run the 32-row tiles of the second tile list (small
// tiles: small_prefix / small_map, np_small packed weight tiles per tile), two
// groups of four waves per block, looping with the trailing blocks' count as
// stride, so they fill the CUs the 256-row tiles' last round leaves idle
// instead of waiting for a launch of their own.
template <int MODE>
__global__ __launch_bounds__(BTHREADS) void grouped_gemm_big_kernel(FfnArgs a, PrefillWs w, int n_ntiles,
                                                                  const int32_t* small_prefix,
                                                                  const int32_t* small_map, int np_small,
                                                                  int n_big) {
  constexpr int STAGE = 2 * OPND_F16;              // A at 0, B at OPND_F16
  static_assert(2 * STAGE >= EPI_BYTES, "the epilogue reuses the stage buffers");
  __shared__ __align__(16) uint8_t lds[2 * STAGE];
  __shared__ int row_pos[BB];
  __shared__ int row_pair[BB];         // (t, slot) pair of the row: where down writes o
  __shared__ float row_scale[BB];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;                    // wave patch: rows wm*128, cols wn*64
  if ((int)blockIdx.x >= n_big) {
    PrefillWs w2 = w;
    w2.tile_prefix = const_cast<int32_t*>(small_prefix);
    w2.tile_map = const_cast<int32_t*>(small_map);
    const int n_items = small_prefix[a.E] * np_small, stride = (int)gridDim.x - n_big;
    for (int b = (int)blockIdx.x - n_big; b * 2 * MWAVES < n_items; b += stride)
      mid_tile_body<MODE, 1>(a, w2, np_small, 2 * b + (wv >> 2), wv & 3, lane);
    return;
  }
  const int total_tiles = w.tile_prefix[a.E];
  const int active = total_tiles * n_ntiles;
  if ((int)blockIdx.x >= active) return;
  // XCD-aware order: blocks are dealt to the 8 XCDs round-robin, so block b
  // runs on XCD b % 8; mapping each XCD's blocks to one contiguous range of
  // tiles keeps the column tiles of a row tile (same gathered activation
  // rows) and the row tiles of an expert (same weights) in one L2.  A
  // bijection on [0, active).
  int lb;
  {
    const int q = active >> 3, r = active & 7, xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    lb = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
  }
  const int gm = lb / n_ntiles, nt = lb % n_ntiles;
  const int4 tr = reinterpret_cast<const int4*>(w.tile_map)[gm];   // {expert, first row, end row}
  const int e = tr.x, row0 = tr.y, row_end = tr.z;
  // the expert's tensor scales (gate and up, or down), read ahead of the K
  // loop so the epilogue never waits for them
  const float ts0 = MODE == 0 ? a.ts_gate[e] : MODE == 2 ? a.ts_down[e] : 1.0f;
  const float ts1 = MODE == 0 ? a.ts_up[e] : 1.0f;
  // gate/up with a static h scale and no debug copies: the epilogue writes
  // h^ itself (its 128 columns are whole 16-element blocks) instead of h
  const bool code_h = MODE != 2 && h_coded_in_gemm(a);
  const float hts = code_h ? a.h_ts[e] : 0.0f;

  constexpr bool down = MODE == 2;
  const int K = down ? a.I : a.H;
  const int S = K / BBK;                                   // even, >= 4
  const size_t w_tile_bytes = (MODE == 1) ? cb_tile_bytes(K) : tile_bytes(K);
  const size_t w_expert_bytes = down ? down_expert_bytes(a.H, a.I)
                                     : (MODE == 1 ? cb_gate_up_expert_bytes(a.H, a.I) : gate_up_expert_bytes(a.H, a.I));
  const uint8_t* wbase = (down ? a.down : a.gate_up) + (size_t)e * w_expert_bytes + (size_t)(nt * 4) * w_tile_bytes;

  const int h = lane >> 5, r = lane & 31;
  const int sra = 32 * wv + r;                             // this thread's A row of the tile (chunk h)
  // its B row of the tile and chunk parity: NVFP4, packed weight tile wv/2,
  // lane = row (one 1 KiB-contiguous load per wave); codebook, a thread pair
  // per row (a row's index words and entries of a group are 48 + 16 B)
  const int bsr = MODE == 1 ? tid >> 1 : (wv >> 1) * 64 + lane;
  const int bh = MODE == 1 ? tid & 1 : wv & 1;
  const int bl = bsr & 63;
  const uint8_t* btile = wbase + (size_t)(MODE == 1 ? bsr >> 6 : wv >> 1) * w_tile_bytes;

  // one K step's global data for this thread
  struct Regs {
    u32x4 acw, bcw;
    uint32_t asw, bsw, p0, p1, p2;
  };
  auto load_B = [&](Regs& R, int st) {
    const int ck = 2 * st + bh;
    if (MODE == 1) {
      // group ck/4: [64 rows][3 index words x 4 dwords], then [64 rows][8 fp16]
      const uint8_t* grp = btile + (size_t)(ck >> 2) * cb_group_bytes();
      const uint32_t* iw = reinterpret_cast<const uint32_t*>(grp + bl * 48);
      const int d = ck & 3;
      R.p0 = iw[d]; R.p1 = iw[4 + d]; R.p2 = iw[8 + d];
      R.bcw = *reinterpret_cast<const u32x4*>(grp + 64 * 48 + bl * 16);
    } else {
      R.bcw = *reinterpret_cast<const u32x4*>(btile + (size_t)ck * 1024 + lane * 16);
      R.bsw = *reinterpret_cast<const uint16_t*>(btile + tile_scale_offset(K) + (size_t)(ck >> 2) * 512 + lane * 8 +
                                                 (ck & 3) * 2);
    }
  };
  // this thread's A row: down reads the tile's own sorted rows of h^ (no
  // gather), gate/up the x^ row of the row's token (known after the row
  // metadata below)
  bool avalid = false;
  const uint8_t* acodes = nullptr;
  const uint8_t* ascales = nullptr;
  if (down) {
    avalid = row0 + sra < row_end;
    const int rp = avalid ? row0 + sra : row0;           // row0 < row_end: a valid row
    acodes = w.hq_codes + (size_t)rp * (a.I / 2);
    ascales = w.hq_scales + (size_t)rp * (a.I / 16);
  }
  auto load_A = [&](Regs& R, int st) {
    const int ck = 2 * st + h;
    R.acw = *reinterpret_cast<const u32x4*>(acodes + ck * 16);
    R.asw = *reinterpret_cast<const uint16_t*>(ascales + ck * 2);
  };
  // the first two steps' weights depend only on the tile, and down's rows
  // too: in flight before the row metadata and its barrier
  Regs R0, R1;
  load_B(R0, 0);
  load_B(R1, 1);
  if (down) {
    load_A(R0, 0);
    load_A(R1, 1);
  }

  if (tid < BB) {
    const int pos = row0 + tid;
    int rp = -1, pr = 0;
    float rs = 0.0f;
    if (pos < row_end) {
      rp = pos;
      pr = w.perm[pos];
      rs = down ? w.hq_ts[pos] : a.x_ts[pr / a.k];
    }
    row_pos[tid] = rp;
    row_pair[tid] = pr;
    row_scale[tid] = rs;
  }
  __syncthreads();

  if (!down) {
    avalid = row_pos[sra] >= 0;
    const int t = row_pair[sra] / a.k;                  // padding rows: pair 0, a valid token
    acodes = a.x_codes + (size_t)t * (a.H / 2);
    ascales = a.x_scales + (size_t)t * (a.H / 16);
  }
  auto load_step = [&](Regs& R, int st) {
    load_A(R, st);
    load_B(R, st);
  };

  // where this thread's staged elements 8kk .. 8kk+7 go (bytes in a stage)
  const int a_wr = (sra * BLDK + 32 * h) * 2;
  const int b_wr = MODE == 1 ? OPND_F16 + (bsr * BLDK + 32 * bh) * 2
                              : OPND_F16 + (((wv >> 1) * 64 + lane) * BLDK + 32 * bh) * 2;
  // part kk of the staging of R into buffer dst: elements 8kk .. 8kk+7 of
  // this thread's A and B chunks (sa, sb: their block scales; cbt: the B
  // row's codebook, MODE 1)
  auto put = [&](const Regs& R, uint8_t* dst, int kk, half2_t sa, half2_t sb, const CbTable& cbt) {
    const half2_t s = kk < 2 ? half2_t{sa.x, sa.x} : half2_t{sa.y, sa.y};
    const uint32_t aw = kk == 0 ? R.acw.x : kk == 1 ? R.acw.y : kk == 2 ? R.acw.z : R.acw.w;
    *reinterpret_cast<half8_t*>(dst + a_wr + 16 * kk) = dq8(aw, s);
    half8_t bv;
    if constexpr (MODE == 1) {
      half2_t ob[4];
      if (kk == 0) cb_decode8<0>(R.p0, R.p1, R.p2, cbt, ob);
      else if (kk == 1) cb_decode8<1>(R.p0, R.p1, R.p2, cbt, ob);
      else if (kk == 2) cb_decode8<2>(R.p0, R.p1, R.p2, cbt, ob);
      else cb_decode8<3>(R.p0, R.p1, R.p2, cbt, ob);
      bv = cat8(ob[0], ob[1], ob[2], ob[3]);
    } else {
      const half2_t t = kk < 2 ? half2_t{sb.x, sb.x} : half2_t{sb.y, sb.y};
      const uint32_t bw = kk == 0 ? R.bcw.x : kk == 1 ? R.bcw.y : kk == 2 ? R.bcw.z : R.bcw.w;
      bv = dq8(bw, t);
    }
    *reinterpret_cast<half8_t*>(dst + b_wr + 16 * kk) = bv;
  };
  auto scales_of = [&](const Regs& R, half2_t& sa, half2_t& sb, CbTable& cbt) {
    sa = e4m3x2_to_f16x2(avalid ? R.asw : 0u);          // padding rows: scale 0 stages zeros
    if constexpr (MODE == 1) cbt = cb_table(R.bcw);
    else sb = e4m3x2_to_f16x2(R.bsw);
  };

  float16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // the MFMAs of the step in buffer src; with nxt, the next step's registers
  // are staged into buffer dst alongside, a quarter per K slice
  auto compute = [&](const uint8_t* src, const Regs* nxt, uint8_t* dst) {
    half2_t sa{}, sb{};
    CbTable cbt{};
    if (nxt) scales_of(*nxt, sa, sb, cbt);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      half8_t af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(src + ((wm * 128 + i * 32 + r) * BLDK + 32 * h + 8 * kk) * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(src + OPND_F16 +
                                                  ((wn * 64 + j * 32 + r) * BLDK + 32 * h + 8 * kk) * 2);
      if (nxt) put(*nxt, dst, kk, sa, sb, cbt);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // Two register sets, so a step's loads are issued two steps before it is
  // staged.  At the top of each loop pass (step st even): buffer 0 holds
  // step st, R1 step st+1, R0 step st+2.
  uint8_t* const buf0 = lds;
  uint8_t* const buf1 = lds + STAGE;
  if (!down) {
    load_A(R0, 0);
    load_A(R1, 1);
  }
  {
    half2_t sa, sb{};
    CbTable cbt{};
    scales_of(R0, sa, sb, cbt);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) put(R0, buf0, kk, sa, sb, cbt);
  }
  __syncthreads();
  load_step(R0, 2);
  int st = 0;
  for (; st + 4 < S; st += 2) {
    compute(buf0, &R1, buf1);
    load_step(R1, st + 3);
    __syncthreads();
    compute(buf1, &R0, buf0);
    load_step(R0, st + 4);
    __syncthreads();
  }
  // the last four steps (st = S - 4): buffer 0 = st, R1 = st+1, R0 = st+2
  compute(buf0, &R1, buf1);
  load_step(R1, st + 3);
  __syncthreads();
  compute(buf1, &R0, buf0);
  __syncthreads();
  compute(buf0, &R1, buf1);
  __syncthreads();
  compute(buf1, nullptr, nullptr);
  __syncthreads();                                         // every wave done with both buffers

  // ---- epilogue.  acc[i][j][q]: row wm*128 + i*32 + (q%4) + 8*(q/4) + 4*h,
  // col wn*64 + j*32 + r of the 256x256 tile.  Each wave turns its results
  // around in its own 9 KB of LDS (the stage buffers are free), a 64 x 32
  // quarter at a time, and writes 16 B per lane (eight lanes per 32-column
  // row, eight rows per store instruction); a wave-level LDS sync suffices.
  constexpr int QS = 36;                                   // row stride (floats) of a quarter
  float* q = reinterpret_cast<float*>(lds) + wv * (64 * QS);
  const int c4 = (lane & 7) * 4, rq = lane >> 3;
  if (!down) {
    // packed tile nt*4 + wn: gate cols = MFMA tile 0, up cols = tile 1; the
    // wave's h columns are that tile's 32
    const int n = (nt * 4 + wn) * 32 + c4;
#pragma unroll
    for (int ih = 0; ih < 2; ++ih) {
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
        for (int qq = 0; qq < 16; ++qq) {
          const int lr = i2 * 32 + (qq & 3) + 8 * (qq >> 2) + 4 * h;
          const float sx = row_scale[wm * 128 + ih * 64 + lr];
          const float g = acc[2 * ih + i2][0][qq] * (sx * ts0);
          const float u = acc[2 * ih + i2][1][qq] * (sx * ts1);
          q[lr * QS + r] = silu_mul(g, u);
        }
      wave_lds_sync();
      if (code_h) {
        // lane l: row l of the quarter, its two 16-element blocks (h columns
        // (nt*4 + wn)*32 .. +31), coded as the h quantizer codes them
        const int pos = row_pos[wm * 128 + ih * 64 + lane];
        if (pos >= 0) {
          const int b0 = (nt * 4 + wn) * 2;                // first block of the row's 32 columns
#pragma unroll
          for (int bk = 0; bk < 2; ++bk) {
            float v[16];
#pragma unroll
            for (int c = 0; c < 16; c += 4) {
              const float4_t f = *reinterpret_cast<const float4_t*>(q + lane * QS + 16 * bk + c);
              v[c] = f.x; v[c + 1] = f.y; v[c + 2] = f.z; v[c + 3] = f.w;
            }
            uint32_t pk[2];
            const uint32_t sb = quantize_block16(v, hts, pk);
            *reinterpret_cast<u32x2*>(w.hq_codes + (size_t)pos * (a.I / 2) + (b0 + bk) * 8) = u32x2{pk[0], pk[1]};
            w.hq_scales[(size_t)pos * (a.I / 16) + b0 + bk] = (uint8_t)sb;
          }
          if (nt == 0 && wn == 0) w.hq_ts[pos] = hts;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int row = rq + 8 * m;
          const float4_t v = *reinterpret_cast<const float4_t*>(q + row * QS + c4);
          const int pos = row_pos[wm * 128 + ih * 64 + row];
          if (pos >= 0) *reinterpret_cast<float4_t*>(w.h + (size_t)pos * a.I + n) = v;
        }
      }
      wave_lds_sync();                                     // reads done before the next quarter's writes
    }
  } else {
    // rows of o are scattered: one (t, slot) pair each
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ih = 0; ih < 2; ++ih) {
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
          for (int qq = 0; qq < 16; ++qq)
            q[(i2 * 32 + (qq & 3) + 8 * (qq >> 2) + 4 * h) * QS + r] = acc[2 * ih + i2][j][qq];
        wave_lds_sync();
        const int n = nt * BB + wn * 64 + j * 32 + c4;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int row = rq + 8 * m;
          const int rl = wm * 128 + ih * 64 + row;
          const float4_t v = *reinterpret_cast<const float4_t*>(q + row * QS + c4);
          if (row_pos[rl] >= 0) {
            const float sc = row_scale[rl] * ts0;
            *reinterpret_cast<float4_t*>(a.out + (size_t)row_pair[rl] * a.H + n) = v * sc;
          }
        }
        wave_lds_sync();                                   // reads done before the next quarter's writes
      }
  }
}

// ---------------------------------------------------------------- 32-row tiles
// Mid batches, where an expert holds a few rows: one wave per (32-row expert
// tile, 64-row packed weight tile), operands loaded straight into MFMA
// registers, no LDS and no barrier, so the weight stream (read once per
// expert tile) is the whole cost.  v_mfma_f32_32x32x16_f16 takes from lane l
// row l%32 of A and of B and eight k values.  In K step s (64 values), lanes
// 0-31 hold chunk 2s and lanes 32-63 chunk 2s+1, 16 code bytes each,
// dequantized to 32 f16 per lane, and MFMA m of the step takes values
// 8m..8m+7 of each lane's chunk: A and B share this k order, so the four
// MFMAs cover the step's 64 products exactly once.  Two register sets
// alternate, one step's loads in flight while the other's are consumed.
// Codebook gate/up (MODE 1): the lane reads its chunk's three index words
// and its row's eight fp16 entries instead.  K % 128 == 0 (even step count).
constexpr int MID_MAX_AVG_ROWS = 96;   // 32-row tiles while T*k <= this * E
constexpr int MID_MAX_AVG_ROWS_CB = 64;   // the same for codebook gate/up (VALU-heavier decode:
                                          // it repays the big tiles' reuse sooner)
// In the 256-row tiling, experts below this many rows take 32-row tiles (the
// 32-row kernels stream an expert's weights once per 32 rows, the 256-row
// ones stage a mostly empty tile at full cost).
constexpr int BB_SPLIT_ROWS = 128;
constexpr int SMALL_BLOCKS = 256;     // trailing 32-row-tile blocks of a 256-row launch: the CU count

struct MidRegs {
  u32x4 ac;          // A codes, this lane's chunk of its row
  uint32_t as;       // A block scales (two E4M3 bytes)
  u32x4 bc[2];       // B codes (NVFP4) or codebook entries: packed rows r and 32 + r
  uint32_t bs[2];    // B block scales (NVFP4)
  uint32_t bp[2][3]; // B index words (codebook)
};

// MODE 0: gate/up NVFP4, 1: gate/up codebook, 2: down.  KS: waves per item,
// each on 1/KS of K (gate/up at small N), else 1.  The codebook mode is held
// to 168 VGPRs (three waves per SIMD; a few spilled registers): 4-5 % faster
// at 16 and 1024 tokens than at 252 VGPRs and two waves.
// The body of one block of MWAVES waves (block index blk, wave wv); also run
// by the 256-row kernel's trailing blocks over the second tile list.
template <int MODE, int KS>
__device__ __forceinline__ void mid_tile_body(const FfnArgs& a, const PrefillWs& w, int n_ptiles, int blk, int wv,
                                              int lane) {
  constexpr int ksplit = KS;
  constexpr int IPB = MWAVES / KS;                 // items per block; KS waves per item
  constexpr bool down = MODE == 2;
  const int slot = wv / KS, ks = wv % KS;
  const int total_items = w.tile_prefix[a.E] * n_ptiles;
  if (blk * IPB >= total_items) return;                           // whole block idle
  const int item = blk * IPB + slot;
  const bool valid = item < total_items;
  const int tp = valid ? item : blk * IPB;                        // idle waves shadow slot 0
  const int gm = tp / n_ptiles, p = tp % n_ptiles;
  const int4 tr = reinterpret_cast<const int4*>(w.tile_map)[gm];   // {expert, first row, end row}
  const int e = tr.x, row0 = tr.y, row_end = tr.z;
  const int K = down ? a.I : a.H;
  const int r = lane & 31, hf = lane >> 5;

  // this lane's A row; a padding lane reads the tile's first row (its
  // output rows are never stored)
  const int pos = row0 + r < row_end ? row0 + r : row0;
  const int pair = w.perm[pos];
  const uint8_t* acodes;
  const uint8_t* ascales;
  float own_scale;
  if (down) {
    acodes = w.hq_codes + (size_t)pos * (a.I / 2);
    ascales = w.hq_scales + (size_t)pos * (a.I / 16);
    own_scale = w.hq_ts[pos];
  } else {
    const int t = pair / a.k;
    acodes = a.x_codes + (size_t)t * (a.H / 2);
    ascales = a.x_scales + (size_t)t * (a.H / 16);
    own_scale = a.x_ts[t];
  }
  const uint8_t* tile;
  if (MODE == 1)
    tile = a.gate_up + (size_t)e * cb_gate_up_expert_bytes(a.H, a.I) + (size_t)p * cb_tile_bytes(K);
  else
    tile = (down ? a.down + (size_t)e * down_expert_bytes(a.H, a.I)
                 : a.gate_up + (size_t)e * gate_up_expert_bytes(a.H, a.I)) +
           (size_t)p * tile_bytes(K);
  const uint8_t* bcodes = tile + r * 16;
  const uint8_t* bscales = tile + tile_scale_offset(K) + r * 8;

  auto load = [&](MidRegs& o, int s) {
    const int ck = 2 * s + hf;
    o.ac = *reinterpret_cast<const u32x4*>(acodes + ck * 16);
    o.as = *reinterpret_cast<const uint16_t*>(ascales + ck * 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (MODE == 1) {
        // group ck/4: [64 rows][3 index words x 4 dwords], then [64 rows][8 fp16]
        const uint8_t* grp = tile + (size_t)(ck >> 2) * cb_group_bytes();
        const uint32_t* iw = reinterpret_cast<const uint32_t*>(grp + (j * 32 + r) * 48);
        const int d = ck & 3;
        o.bp[j][0] = iw[d];
        o.bp[j][1] = iw[4 + d];
        o.bp[j][2] = iw[8 + d];
        o.bc[j] = *reinterpret_cast<const u32x4*>(grp + 64 * 48 + (j * 32 + r) * 16);
      } else {
        o.bc[j] = *reinterpret_cast<const u32x4*>(bcodes + (size_t)ck * 1024 + j * 512);
        o.bs[j] = *reinterpret_cast<const uint16_t*>(bscales + (size_t)(ck >> 2) * 512 + j * 256 + (ck & 3) * 2);
      }
    }
  };
  float16_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;
  auto step = [&](const MidRegs& o) {
    half2_t av[16], bv[2][16];
    dequant32_nvfp4(o.ac, o.as, av);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (MODE == 1)
        dequant32_cb(o.bp[j][0], o.bp[j][1], o.bp[j][2], o.bc[j], bv[j]);
      else
        dequant32_nvfp4(o.bc[j], o.bs[j], bv[j]);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const half8_t af = cat8(av[4 * m], av[4 * m + 1], av[4 * m + 2], av[4 * m + 3]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            af, cat8(bv[j][4 * m], bv[j][4 * m + 1], bv[j][4 * m + 2], bv[j][4 * m + 3]), acc[j], 0, 0, 0);
    }
  };

  const int Sk = K / 64 / ksplit, s0 = ks * Sk;    // this wave's K steps (an even count)
  MidRegs o0, o1;
  load(o0, s0);
  load(o1, s0 + 1);
  for (int s = s0; s < s0 + Sk - 2; s += 2) {
    step(o0);
    load(o0, s + 2);
    step(o1);
    load(o1, s + 3);
  }
  step(o0);
  step(o1);

  if (KS > 1) {                                    // sum the K shares in LDS, share order
    __shared__ float red[KS > 1 ? (KS - 1) * IPB : 1][32][64];
    if (ks > 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) red[(ks - 1) * IPB + slot][j * 16 + q][lane] = acc[j][q];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int k2 = 1; k2 < KS; ++k2)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[j][q] += red[(k2 - 1) * IPB + slot][j * 16 + q][lane];
  }
  if (!valid) return;
  // acc[j][q]: tile row (q%4) + 8*(q/4) + 4*hf, column r of sub-tile j
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int rl = (q & 3) + 8 * (q >> 2) + 4 * hf;
    const float sc = __shfl(own_scale, rl);
    const int pr = __shfl(pair, rl);
    if (row0 + rl >= row_end) continue;
    if (!down) {
      const float g = acc[0][q] * (sc * (MODE == 0 ? a.ts_gate[e] : 1.0f));
      const float u = acc[1][q] * (sc * (MODE == 0 ? a.ts_up[e] : 1.0f));
      w.h[(size_t)(row0 + rl) * a.I + p * 32 + r] = silu_mul(g, u);
    } else {
      const float tsd = a.ts_down[e];
#pragma unroll
      for (int j = 0; j < 2; ++j) a.out[(size_t)pr * a.H + p * 64 + j * 32 + r] = acc[j][q] * (sc * tsd);
    }
  }
}

template <int MODE, int KS>
__global__ __launch_bounds__(64 * MWAVES, MODE == 1 ? 3 : 1) void grouped_gemm_mid_kernel(FfnArgs a, PrefillWs w, int n_ptiles) {
  mid_tile_body<MODE, KS>(a, w, n_ptiles, (int)blockIdx.x, (int)(threadIdx.x >> 6), (int)(threadIdx.x & 63));
}

// NVFP4 of each h row (sorted order), one wave per row, one pass: lane l
// holds the row's 16-element blocks l, l+64, ... (all loads first), the row
// amax is a wave max of the block maxima; also the optional debug copies in
// (t, slot) order.  I <= 64 * HQ_MAXB * 16; NB = blocks per lane, the
// fewest that cover the row (one up to I = 1024), so no lane holds or loads
// more than it quantizes.
constexpr int HQ_MAXB = 4;
template <int NB>
__global__ __launch_bounds__(256) void h_quant_kernel(FfnArgs a, PrefillWs w, int N, int coded_min_rows) {
  const int lane = threadIdx.x & 63;
  const int pos = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pos >= N) return;
  if (pos >= w.offsets[a.E]) {                           // pair with an id outside [0, E):
    const int pair = w.perm[pos];                        // its output row is zero, and so
    for (int c = lane; c < a.H; c += 64) a.out[(size_t)pair * a.H + c] = 0.0f;
    if (a.dbg_h)                                         // are its debug h and h^ (as in
      for (int c = lane; c < a.I; c += 64) a.dbg_h[(size_t)pair * a.I + c] = 0.0f;   // the decode path)
    if (a.dbg_h_codes)
      for (int c = lane; c < a.I / 2; c += 64) a.dbg_h_codes[(size_t)pair * (a.I / 2) + c] = 0;
    if (a.dbg_h_scales)
      for (int c = lane; c < a.I / 16; c += 64) a.dbg_h_scales[(size_t)pair * (a.I / 16) + c] = 0;
    if (a.dbg_h_ts && lane == 0) a.dbg_h_ts[pair] = 0.0f;
    return;
  }
  const int I = a.I, nblk = I / 16;
  const float* hr = w.h + (size_t)pos * I;
  const int pair = w.perm[pos];
  // rows of experts with at least coded_min_rows rows were coded by the
  // 256-row GEMM's epilogue (static h scale)
  if (coded_min_rows < INT_MAX && w.counts[a.ids[pair]] >= coded_min_rows) return;
  float v[NB][16];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int b = min(lane + 64 * j, nblk - 1);          // clamped: straight-line loads
    const float4_t* src = reinterpret_cast<const float4_t*>(hr + b * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4_t f = src[r];
      v[j][4 * r] = f.x; v[j][4 * r + 1] = f.y; v[j][4 * r + 2] = f.z; v[j][4 * r + 3] = f.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (lane + 64 * j < nblk) {
#pragma unroll
      for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(v[j][c]));
    }
  amax = dpp_wave_max(amax);
  // static mode: the row's expert's calibrated scale
  const float ts = a.h_ts ? a.h_ts[a.ids[pair]] : tensor_scale_from_amax(amax);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int b = lane + 64 * j;
    if (b >= nblk) continue;
    uint32_t pk[2];
    const uint32_t sb = quantize_block16(v[j], ts, pk);
    *reinterpret_cast<u32x2*>(w.hq_codes + (size_t)pos * (I / 2) + b * 8) = u32x2{pk[0], pk[1]};
    w.hq_scales[(size_t)pos * nblk + b] = (uint8_t)sb;
    if (a.dbg_h) {
#pragma unroll
      for (int c = 0; c < 16; ++c) a.dbg_h[(size_t)pair * I + b * 16 + c] = v[j][c];
    }
    if (a.dbg_h_codes) *reinterpret_cast<u32x2*>(a.dbg_h_codes + (size_t)pair * (I / 2) + b * 8) = u32x2{pk[0], pk[1]};
    if (a.dbg_h_scales) a.dbg_h_scales[(size_t)pair * nblk + b] = (uint8_t)sb;
  }
  if (lane == 0) {
    w.hq_ts[pos] = ts;
    if (a.dbg_h_ts) a.dbg_h_ts[pair] = ts;
  }
}

// coded_min_rows: rows of experts with at least this many rows are already
// coded (the 256-row tiling with a static h scale), else INT_MAX
static void launch_h_quant(const FfnArgs& a, const PrefillWs& w, int N, hipStream_t s,
                           int coded_min_rows = INT_MAX) {
  const int nb = (a.I / 16 + 63) / 64;                   // 1..HQ_MAXB (I <= 4096)
  const unsigned g = (unsigned)((N + 3) / 4);
  if (nb <= 1) h_quant_kernel<1><<<g, 256, 0, s>>>(a, w, N, coded_min_rows);
  else if (nb == 2) h_quant_kernel<2><<<g, 256, 0, s>>>(a, w, N, coded_min_rows);
  else if (nb == 3) h_quant_kernel<3><<<g, 256, 0, s>>>(a, w, N, coded_min_rows);
  else h_quant_kernel<HQ_MAXB><<<g, 256, 0, s>>>(a, w, N, coded_min_rows);
}

static bool big_tiles_fit(const FfnArgs& a) {
  return a.H % BB == 0 && (2 * a.I) % BB == 0 && a.I % (2 * BBK) == 0 && a.I >= 4 * BBK &&
         a.H % (2 * BBK) == 0 && a.H >= 4 * BBK;
}

// Row-tile height the grouped GEMMs use for these shapes: 32 while the
// experts hold few rows on average (the weight stream is the cost and the
// 32-row wave kernel reads it once per expert tile), 256 when the shapes
// allow the big tiles, else 128.
int prefill_tile_rows(int E, int H, int I, int k, int T, int fmt) {
  FfnArgs a{};
  a.E = E; a.H = H; a.I = I; a.k = k; a.T = T; a.fmt = fmt;
  const int lim = fmt == FMT_CB3G128 ? MID_MAX_AVG_ROWS_CB : MID_MAX_AVG_ROWS;
  if ((long long)T * k <= (long long)lim * E) return MB;
  return big_tiles_fit(a) ? BB : BM;
}

hipError_t launch_ffn_prefill(const FfnArgs& a, void* ws, hipStream_t s) {
  const int N = a.T * a.k;
  PrefillWs w = carve(ws, a.E, a.I, a.k, a.T, nullptr);
  const int rows = prefill_tile_rows(a.E, a.H, a.I, a.k, a.T, a.fmt);
  if (rows == MB) {
    hipError_t err = launch_permute(a.ids, a.T, a.k, a.E, w.counts, w.offsets, w.perm, w.inv,
                                    w.perm_ws, w.tile_prefix, w.tile_map, MB, s);
    if (err != hipSuccess) return err;
    const long long max_mtiles = (N + MB - 1) / MB + a.E;
    const int np_gu = a.I / 32, np_dn = a.H / 64;   // 64-row packed tiles per projection
    const int S_gu = a.H / 64;                       // gate/up K steps
    const int split_max = a.fmt == FMT_CB3G128 ? SPLIT_MAX_N : SPLIT_MAX_N_NVFP4;
    const int ksplit = N > split_max ? 1 : S_gu % (2 * SPLIT_K_MAX) == 0 ? SPLIT_K_MAX : S_gu % 4 == 0 ? 2 : 1;
    const unsigned g_gu = (unsigned)((max_mtiles * np_gu * ksplit + MWAVES - 1) / MWAVES);   // KS waves per item
    const bool cb = a.fmt == FMT_CB3G128;
    if (ksplit == 4) {
      if (cb) grouped_gemm_mid_kernel<1, 4><<<g_gu, 64 * MWAVES, 0, s>>>(a, w, np_gu);
      else grouped_gemm_mid_kernel<0, 4><<<g_gu, 64 * MWAVES, 0, s>>>(a, w, np_gu);
    } else if (ksplit == 2) {
      if (cb) grouped_gemm_mid_kernel<1, 2><<<g_gu, 64 * MWAVES, 0, s>>>(a, w, np_gu);
      else grouped_gemm_mid_kernel<0, 2><<<g_gu, 64 * MWAVES, 0, s>>>(a, w, np_gu);
    } else {
      if (cb) grouped_gemm_mid_kernel<1, 1><<<g_gu, 64 * MWAVES, 0, s>>>(a, w, np_gu);
      else grouped_gemm_mid_kernel<0, 1><<<g_gu, 64 * MWAVES, 0, s>>>(a, w, np_gu);
    }
    launch_h_quant(a, w, N, s);
    grouped_gemm_mid_kernel<2, 1><<<(max_mtiles * np_dn + MWAVES - 1) / MWAVES, 64 * MWAVES, 0, s>>>(a, w, np_dn);
    return hipGetLastError();
  }
  if (rows == BB) {
    // experts with fewer than BB_SPLIT_ROWS rows (a skewed routing's long
    // tail) take 32-row tiles in a second list rather than one mostly empty
    // 256-row tile each; both lists index the same permuted rows
    TileSplit sp;
    sp.tile_prefix = w.tile_prefix2;
    sp.tile_map = w.tile_map2;
    sp.BM = MB;
    sp.split_rows = BB_SPLIT_ROWS;
    hipError_t err = launch_permute(a.ids, a.T, a.k, a.E, w.counts, w.offsets, w.perm, w.inv,
                                    w.perm_ws, w.tile_prefix, w.tile_map, BB, s, sp);
    if (err != hipSuccess) return err;
    const int max_mtiles = (N + BB - 1) / BB + a.E;
    const long long max_small = std::min<long long>((N + MB - 1) / MB + a.E,
                                                    (long long)a.E * ((BB_SPLIT_ROWS + MB - 2) / MB));
    const int nt_gu = (2 * a.I) / BB;
    const int np_gu = a.I / 32, np_dn = a.H / 64;     // 64-row packed tiles per projection
    // the second list's 32-row tiles ride in trailing blocks of the same
    // launches (two groups of MWAVES waves per block, at most one block per CU)
    const int n_big_gu = max_mtiles * nt_gu;
    const int g_gu_small = std::min(SMALL_BLOCKS, (int)((max_small * np_gu + 2 * MWAVES - 1) / (2 * MWAVES)));
    if (a.fmt == FMT_CB3G128)
      grouped_gemm_big_kernel<1><<<n_big_gu + g_gu_small, BTHREADS, 0, s>>>(a, w, nt_gu, w.tile_prefix2, w.tile_map2,
                                                                             np_gu, n_big_gu);
    else
      grouped_gemm_big_kernel<0><<<n_big_gu + g_gu_small, BTHREADS, 0, s>>>(a, w, nt_gu, w.tile_prefix2, w.tile_map2,
                                                                             np_gu, n_big_gu);
    launch_h_quant(a, w, N, s, h_coded_in_gemm(a) ? BB_SPLIT_ROWS : INT_MAX);
    const int nt_dn = a.H / BB;
    const int n_big_dn = max_mtiles * nt_dn;
    const int g_dn_small = std::min(SMALL_BLOCKS, (int)((max_small * np_dn + 2 * MWAVES - 1) / (2 * MWAVES)));
    grouped_gemm_big_kernel<2><<<n_big_dn + g_dn_small, BTHREADS, 0, s>>>(a, w, nt_dn, w.tile_prefix2, w.tile_map2,
                                                                           np_dn, n_big_dn);
    return hipGetLastError();
  }
  hipError_t err = launch_permute(a.ids, a.T, a.k, a.E, w.counts, w.offsets, w.perm, w.inv,
                                  w.perm_ws, w.tile_prefix, w.tile_map, BM, s);
  if (err != hipSuccess) return err;
  const int max_mtiles = (N + BM - 1) / BM + a.E;
  const int nt_gu = (2 * a.I) / BN;                  // 64-row packed tiles, two per block
  if (a.fmt == FMT_CB3G128)
    grouped_gemm_kernel<1><<<max_mtiles * nt_gu, PF_THREADS, 0, s>>>(a, w, nt_gu);
  else
    grouped_gemm_kernel<0><<<max_mtiles * nt_gu, PF_THREADS, 0, s>>>(a, w, nt_gu);
  launch_h_quant(a, w, N, s);
  const int nt_dn = a.H / BN;
  grouped_gemm_kernel<2><<<max_mtiles * nt_dn, PF_THREADS, 0, s>>>(a, w, nt_dn);
  return hipGetLastError();
}

}  // namespace moe
