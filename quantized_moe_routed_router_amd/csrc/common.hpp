// Shared device helpers for the MoE kernels (gfx950 / CDNA4, wave64).
//
// NVFP4 element and scale formats (public definition; the pages name NVFP4
// in the release post "capy-flash v0.7.1", section "What shipped"):
//   E2M1: sign bit 3, magnitudes of codes 0..7 = 0, .5, 1, 1.5, 2, 3, 4, 6.
//   E4M3 (OCP "FN"): bias 7, subnormals m/8 * 2^-6, max 448 (0x7E), 0x7F NaN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr float TS_DIVISOR = 2688.0f;  // 6 * 448: largest E2M1 times largest E4M3
constexpr int FMT_NVFP4 = 0, FMT_CB3G128 = 1;  // gate/up weight formats

// ---------------------------------------------------------------- packed layout
// A "tile" is 64 weight rows (lanes) x the whole contraction length K:
//   codes  [K/32 chunks][64 lanes][16 B]   32 elements per lane-chunk, element
//                                          2j of the chunk in byte j's low nibble
//   scales [K/128 groups][64 lanes][8 B]   8 E4M3 block scales per lane-group
// so one wave-wide 16-byte load of a chunk reads 1 KiB contiguous, and one
// 8-byte load of a group reads 512 B contiguous.  Tile bytes = 36 * K.
// Gate/up tiles hold 32 gate rows (lanes 0..31) and the same 32 up rows
// (lanes 32..63): tile j covers n = 32j .. 32j+31.  Down tiles hold 64
// consecutive rows.  Experts follow each other; tiles follow each other.
__host__ __device__ constexpr size_t tile_bytes(int K) { return (size_t)36 * K; }
__host__ __device__ constexpr size_t tile_scale_offset(int K) { return (size_t)32 * K; }
__host__ __device__ constexpr size_t gate_up_expert_bytes(int H, int I) {
  return (size_t)(I / 32) * tile_bytes(H);
}
__host__ __device__ constexpr size_t down_expert_bytes(int H, int I) {
  return (size_t)(H / 64) * tile_bytes(I);
}
// Codebook gate/up tiles (3-bit indices, fp16 codebook per 128-group):
//   per group g: [64 lanes][3 bit-planes x 16 B] then [64 lanes][8 x fp16]
//   bit-plane p, dword d, bit b = bit p of the index of element 32d + b.
__host__ __device__ constexpr size_t cb_group_bytes() { return 64 * 48 + 64 * 16; }
__host__ __device__ constexpr size_t cb_tile_bytes(int K) { return (size_t)(K / 128) * cb_group_bytes(); }
__host__ __device__ constexpr size_t cb_gate_up_expert_bytes(int H, int I) {
  return (size_t)(I / 32) * cb_tile_bytes(H);
}

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  // non-negative E4M3 code (bit 7 ignored by callers that pass scales 0..0x7E)
  uint32_t e = (b >> 3) & 0xF, m = b & 7;
  float nrm = __uint_as_float(((b & 0x7F) << 20) + (120u << 23));
  float sub = (float)m * 0x1p-9f;
  return e ? nrm : sub;
}

// Round s >= 0 to the nearest E4M3 code (ties to even), saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne_satfinite(float s) {
  if (!(s < 448.0f)) return 0x7E;                 // also catches +inf
  if (s < 0x1p-6f) {                              // subnormal grid, quantum 2^-9
    return (uint32_t)__builtin_rintf(s * 512.0f); // exact scaling; rint = RNE
  }
  uint32_t u = __float_as_uint(s);
  uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);   // RNE at mantissa bit 20
  uint32_t c = (r >> 20) - (120u << 3);
  return c > 0x7Eu ? 0x7Eu : c;
}

// 3-bit magnitude code of a >= 0 on {0,.5,1,1.5,2,3,4,6}: nearest, ties to
// the even code, saturating (the interval boundaries are exact in fp32).
__device__ __forceinline__ uint32_t e2m1_rne_sat(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Quantize one 16-element block given its row's tensor scale ts (fp32 steps,
// no contraction): returns the E4M3 scale code and writes 8 code bytes
// (element 2j in the low nibble of byte j).
__device__ __forceinline__ uint32_t quantize_block16(const float (&v)[16], float ts,
                                                     uint32_t (&packed)[2]) {
#pragma clang fp contract(off)
  float ab = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(v[i]));
  uint32_t sb = 0;
  if (ts != 0.0f) {
    float six_ts = 6.0f * ts;
    sb = e4m3_rne_satfinite(__fdiv_rn(ab, six_ts));
  }
  float d = e4m3_to_f32(sb) * ts;
  packed[0] = packed[1] = 0;
  if (d != 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float q = __fdiv_rn(v[i], d);
      uint32_t c = e2m1_rne_sat(fabsf(q)) | ((__float_as_uint(v[i]) >> 31) << 3);
      packed[i >> 3] |= c << (4 * (i & 7));
    }
  }
  return sb;
}

__device__ __forceinline__ float tensor_scale_from_amax(float amax) {
  return amax == 0.0f ? 0.0f : __fdiv_rn(amax, TS_DIVISOR);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, WAVE));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

// E2M1 pair (one byte, low nibble first) -> f16x2, exact.
template <int SEL>
__device__ __forceinline__ half2_t fp4x2_to_f16x2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL);
}

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

}  // namespace moe
