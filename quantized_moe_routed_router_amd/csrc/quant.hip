// NVFP4 quantizers (activations: one tensor scale per row; weights: one per
// matrix) and the packed-layout writers.
//
// Quantizer steps (fp32, round-to-nearest-even, no contraction), applied to
// the layer input x and to expert weights: amax over the scope, ts =
// amax / 2688, per 16-element block an E4M3 scale of max|v| / (6 ts), then
// E2M1 codes of v / (E4M3(scale) * ts).  The release post ("capy-flash
// v0.7.1", sections "What shipped" and "Why it matters") names NVFP4 weights
// and a W4A4 path; the step order is the plain reading of the NVFP4 format.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// ---------------------------------------------------------------- activations
// One 256-thread block per row: every thread loads its 16-element blocks once,
// the row amax goes through DPP + LDS, then each thread quantizes its blocks
// (32 B of bf16 in, 8 B codes + 1 B scale out, coalesced across the block).
// One wave per token row, four rows per block: many rows in flight per CU
// (one 256-thread block per row left most of a 2560-wide row's threads idle
// and few rows in flight).
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x, int T,
                                                        int H, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales,
                                                        float* __restrict__ ts_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  quantize_row_bf16_wave(x + (size_t)row * H, H, codes + (size_t)row * (H / 2),
                         scales + (size_t)row * (H / 16), ts_out + row, threadIdx.x & 63);
}

hipError_t launch_act_quant(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales,
                            float* ts, hipStream_t s) {
  if (T == 0) return hipSuccess;
  act_quant_kernel<<<(T + 3) / 4, 256, 0, s>>>(x, T, H, codes, scales, ts);
  return hipGetLastError();
}

// ---------------------------------------------------------------- weights
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// amax of each matrix, as float bits in ts (non-negative floats order like
// their unsigned bit patterns, so atomicMax on the bits is exact and
// order-independent).
__global__ __launch_bounds__(256) void weight_amax_kernel(const float* __restrict__ W,
                                                          size_t per_mat, float* ts) {
  const int m = blockIdx.y;
  const float4_t* p = reinterpret_cast<const float4_t*>(W + per_mat * m);
  const size_t n4 = per_mat / 4;
  float amax = 0.0f;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    float4_t v = p[i];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = wave_max(amax);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(reinterpret_cast<unsigned int*>(ts + m), __float_as_uint(a));
  }
}

// One thread per 16-element block; amax read from ts (still holding amax).
__global__ __launch_bounds__(256) void weight_quant_kernel(const float* __restrict__ W,
                                                           size_t nblocks_total,
                                                           size_t blocks_per_mat,
                                                           const float* __restrict__ amax_per_mat,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  size_t b = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks_total) return;
  const size_t m = b / blocks_per_mat;
  const float ts = tensor_scale_from_amax(amax_per_mat[m]);
  const float4_t* p = reinterpret_cast<const float4_t*>(W + b * 16);
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4_t q = p[i];
    v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
  }
  uint32_t pk[2];
  uint32_t sb = quantize_block16(v, ts, pk);
  *reinterpret_cast<u32x2*>(codes + b * 8) = u32x2{pk[0], pk[1]};
  scales[b] = (uint8_t)sb;
}

__global__ void weight_ts_finalize_kernel(float* ts, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ts[i] = tensor_scale_from_amax(ts[i]);
}

hipError_t launch_weight_quant(const float* W, int n_mat, int rows, int cols, uint8_t* codes,
                               uint8_t* scales, float* ts, hipStream_t s) {
  if (n_mat == 0 || rows == 0) {
    if (n_mat) fill_u32_kernel<<<(n_mat + 255) / 256, 256, 0, s>>>((uint32_t*)ts, 0u, n_mat);
    return hipGetLastError();
  }
  const size_t per_mat = (size_t)rows * cols;
  fill_u32_kernel<<<(n_mat + 255) / 256, 256, 0, s>>>(reinterpret_cast<uint32_t*>(ts), 0u, n_mat);
  size_t want = (per_mat / 4 + 255) / 256;
  int gx = (int)(want < 256 ? want : 256);
  if (gx < 1) gx = 1;
  weight_amax_kernel<<<dim3(gx, n_mat), 256, 0, s>>>(W, per_mat, ts);
  const size_t bpm = per_mat / 16, nb = bpm * n_mat;
  weight_quant_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, s>>>(W, nb, bpm, ts, codes, scales);
  weight_ts_finalize_kernel<<<(n_mat + 255) / 256, 256, 0, s>>>(ts, n_mat);
  return hipGetLastError();
}

// ---------------------------------------------------------------- packing
// Row of plain matrix behind lane `l` of tile `j`.
//   gate/up: lanes 0..31 -> gate row 32j + l, lanes 32..63 -> up row 32j + l - 32
//   down:    lane l -> row 64j + l
// One thread moves one 16-byte code chunk or one 8-byte scale group.
template <bool UNPACK>
__global__ __launch_bounds__(256) void pack_nvfp4_kernel(
    int n, int N_tiles, int K, bool gate_up,
    uint8_t* g_codes, uint8_t* g_scales,     // gate (or down) plain, [n, rows, K/2], [n, rows, K/16]
    uint8_t* u_codes, uint8_t* u_scales,     // up plain (gate_up only)
    uint8_t* packed,                          // experts e0..e0+n-1 of the layer buffer
    size_t rows_per_mat) {
  const int chunks = K / 32, groups = K / 128;
  const size_t items_per_tile = (size_t)64 * (chunks + groups);
  const size_t total = (size_t)n * N_tiles * items_per_tile;
  size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const size_t tile_lin = idx / items_per_tile;        // expert * N_tiles + tile
  const int item = (int)(idx % items_per_tile);
  const int e = (int)(tile_lin / N_tiles), j = (int)(tile_lin % N_tiles);
  uint8_t* tile = packed + tile_lin * tile_bytes(K);
  int lane, c_or_g;
  bool is_code = item < 64 * chunks;
  if (is_code) { c_or_g = item / 64; lane = item % 64; }
  else { c_or_g = (item - 64 * chunks) / 64; lane = (item - 64 * chunks) % 64; }
  uint8_t *pc, *ps;
  size_t row;
  if (gate_up) {
    row = (size_t)32 * j + (lane & 31);
    pc = lane < 32 ? g_codes : u_codes;
    ps = lane < 32 ? g_scales : u_scales;
  } else {
    row = (size_t)64 * j + lane;
    pc = g_codes; ps = g_scales;
  }
  const size_t mrow = (size_t)e * rows_per_mat + row;
  if (is_code) {
    u32x4* dst = reinterpret_cast<u32x4*>(tile + (size_t)c_or_g * 1024 + lane * 16);
    u32x4* src = reinterpret_cast<u32x4*>(pc + mrow * (K / 2) + c_or_g * 16);
    if (UNPACK) *src = *dst; else *dst = *src;
  } else {
    u32x2* dst = reinterpret_cast<u32x2*>(tile + tile_scale_offset(K) + (size_t)c_or_g * 512 + lane * 8);
    u32x2* src = reinterpret_cast<u32x2*>(ps + mrow * (K / 16) + c_or_g * 8);
    if (UNPACK) *src = *dst; else *dst = *src;
  }
}

hipError_t launch_pack_nvfp4(bool unpack, int H, int I, int e0, int n, uint8_t* gc, uint8_t* gs,
                             uint8_t* uc, uint8_t* us, uint8_t* dc, uint8_t* ds,
                             uint8_t* gate_up, uint8_t* down, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (gc) {
    const int nt = I / 32;
    size_t total = (size_t)n * nt * 64 * (H / 32 + H / 128);
    uint8_t* base = gate_up + (size_t)e0 * gate_up_expert_bytes(H, I);
    if (unpack)
      pack_nvfp4_kernel<true><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(n, nt, H, true, gc, gs, uc, us, base, I);
    else
      pack_nvfp4_kernel<false><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(n, nt, H, true, gc, gs, uc, us, base, I);
  }
  if (dc) {
    const int nt = H / 64;
    size_t total = (size_t)n * nt * 64 * (I / 32 + I / 128);
    uint8_t* base = down + (size_t)e0 * down_expert_bytes(H, I);
    if (unpack)
      pack_nvfp4_kernel<true><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(n, nt, I, false, dc, ds, nullptr, nullptr, base, H);
    else
      pack_nvfp4_kernel<false><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(n, nt, I, false, dc, ds, nullptr, nullptr, base, H);
  }
  return hipGetLastError();
}

// Codebook gate/up: one thread per (expert, tile, group, lane): writes the
// lane's 3 index words (48 B) and its 8 fp16 entries (16 B).
__global__ __launch_bounds__(256) void pack_codebook_kernel(int n, int N_tiles, int K,
                                                            const uint16_t* __restrict__ g_cb,
                                                            const uint8_t* __restrict__ g_idx,
                                                            const uint16_t* __restrict__ u_cb,
                                                            const uint8_t* __restrict__ u_idx,
                                                            uint8_t* __restrict__ packed, int I) {
  const int groups = K / 128;
  size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)n * N_tiles * groups * 64;
  if (idx >= total) return;
  const int lane = (int)(idx % 64);
  size_t r = idx / 64;
  const int g = (int)(r % groups); r /= groups;
  const int j = (int)(r % N_tiles);
  const int e = (int)(r / N_tiles);
  const size_t row = (size_t)e * I + 32 * j + (lane & 31);
  const uint16_t* cb = (lane < 32 ? g_cb : u_cb) + (row * groups + g) * 8;
  const uint8_t* ix = (lane < 32 ? g_idx : u_idx) + row * K + (size_t)g * 128;
  uint8_t* grp = packed + ((size_t)e * N_tiles + j) * cb_tile_bytes(K) + (size_t)g * cb_group_bytes();
  // index words (the codebook tile layout): element c of chunk d has bits 0-1
  // in word c / 16 at bits 8 (c % 4) + 2 ((c % 16) / 4) and bit 2 in word 2
  // at bit 8 (c % 4) + c / 4
  uint32_t words[3][4] = {};
  for (int el = 0; el < 128; ++el) {
    const uint32_t v = ix[el] & 7;
    const int d = el >> 5, c = el & 31, j = c & 3;
    words[c >> 4][d] |= (v & 3u) << (8 * j + 2 * ((c & 15) >> 2));
    words[2][d] |= ((v >> 2) & 1u) << (8 * j + (c >> 2));
  }
  u32x4* dst = reinterpret_cast<u32x4*>(grp + lane * 48);
#pragma unroll
  for (int p = 0; p < 3; ++p) dst[p] = u32x4{words[p][0], words[p][1], words[p][2], words[p][3]};
  const u32x4* cs = reinterpret_cast<const u32x4*>(cb);
  *reinterpret_cast<u32x4*>(grp + 64 * 48 + lane * 16) = *cs;
}

hipError_t launch_pack_codebook(int H, int I, int e0, int n, const uint16_t* gcb, const uint8_t* gidx,
                                const uint16_t* ucb, const uint8_t* uidx, uint8_t* gate_up,
                                hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int nt = I / 32;
  size_t total = (size_t)n * nt * (H / 128) * 64;
  uint8_t* base = gate_up + (size_t)e0 * cb_gate_up_expert_bytes(H, I);
  pack_codebook_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(n, nt, H, gcb, gidx, ucb, uidx, base, I);
  return hipGetLastError();
}

}  // namespace moe
