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
//   per group g: [64 lanes][3 index words x 4 dwords] then [64 lanes][8 x fp16]
//   chunk d = elements 32d .. 32d+31 of the group, in dword d of each index
//   word: word 0 holds bits 0-1 of the index of element 32d + 4m + j (m, j in
//   0..3) at bits 8j + 2m, 8j + 2m + 1; word 1 the same for elements
//   32d + 16 + 4m + j; word 2 bit 2 of element 32d + 4m + j (m in 0..7) at
//   bit 8j + m.  So four consecutive indices come to the bytes of one word by
//   shifts and masks.
__host__ __device__ constexpr size_t cb_group_bytes() { return 64 * 48 + 64 * 16; }
__host__ __device__ constexpr size_t cb_tile_bytes(int K) { return (size_t)(K / 128) * cb_group_bytes(); }
__host__ __device__ constexpr size_t cb_gate_up_expert_bytes(int H, int I) {
  return (size_t)(I / 32) * cb_tile_bytes(H);
}

// ---------------------------------------------------------------- formats
// E4M3 (OCP FN) code in byte 0 of b -> fp32 in one hardware conversion.  An
// in-bounds check of all 256 codes on the device matched the format's
// definition exactly (subnormals, both signs, NaN for 0x7F and 0xFF).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8(b, 0);
}
// E4M3 codes in bytes 0 and 1 of w -> two f16 values, one instruction (every
// E4M3 value is an f16 value; scale operand 1 is exact).
__device__ __forceinline__ half2_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

// Round s >= 0 to the nearest E4M3 code (ties to even), saturating at 448:
// the hardware OCP FP8 (E4M3FN) conversion with scale 1 rounds exactly so
// below 464 and returns NaN (0x7F) above, so s is clamped to 448 first (NaN
// also becomes 448, as it did through the comparison form); the sign bit is
// dropped so -0 gives code 0.  Checked against the bit-level rounding over
// every fp32 s >= 0.
typedef short fp8x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3_rne_satfinite(float s) {
  const fp8x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((fp8x2_t){0, 0}, fminf(s, 448.0f), 0.0f,
                                                              1.0f, false);
  return (uint32_t)r[0] & 0x7Fu;
}

// Signed E2M1 codes of q0 (low nibble) and q1 into byte SEL of old: the
// hardware FP4 conversion with scale 1 rounds |q| to nearest even on
// {0,.5,1,1.5,2,3,4,6}, saturates at 6 and keeps the sign bit (checked over
// every non-NaN fp32 of both signs).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_into(uint32_t old, float q0, float q1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, q0, q1, 1.0f, SEL);
}

// fp32 division v / d rounded to nearest even, in the hardware division's
// own steps (reciprocal, one Newton step, two residual corrections) without
// its operand scaling and fixup, which leave finite operands unchanged when
// d lies in [2^-60, 2^60] (checked by div_fast_ok).  y = recip_refined(d)
// is shared by every quotient with divisor d.  A numerator below 2^-100
// (where the hardware would scale it) gives a quotient below 2^-40 either
// way, which every caller rounds to code 0.
__device__ __forceinline__ bool div_fast_ok(float d) {
  return d >= 0x1p-60f && d <= 0x1p60f;
}
__device__ __forceinline__ float recip_refined(float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  return fmaf(fmaf(-d, y, 1.0f), y, y);
}
__device__ __forceinline__ float div_refined(float v, float d, float y) {
  float q = v * y;
  q = fmaf(fmaf(-d, q, v), y, q);
  return fmaf(fmaf(-d, q, v), y, q);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// bf16_rne(x * s) of a bf16 value (bits), and of both halves of a word.
__device__ __forceinline__ uint32_t bf16_scaled(uint32_t b, float s) {
  return f32_to_bf16_rne(bf16_to_f32(b & 0xFFFF) * s);
}
__device__ __forceinline__ uint32_t bf16x2_scaled(uint32_t w, float s) {
  return bf16_scaled(w & 0xFFFF, s) | (bf16_scaled(w >> 16, s) << 16);
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
    const float six_ts = 6.0f * ts;
    float r;
    if (div_fast_ok(six_ts)) r = div_refined(ab, six_ts, recip_refined(six_ts));
    else r = __fdiv_rn(ab, six_ts);
    sb = e4m3_rne_satfinite(r);
  }
  float d = e4m3_to_f32(sb) * ts;
  packed[0] = packed[1] = 0;
  if (d != 0.0f) {
    float q[16];
    if (div_fast_ok(d)) {
      const float y = recip_refined(d);
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = div_refined(v[i], d, y);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = __fdiv_rn(v[i], d);
    }
    // the code's sign is v's (also for v = -0, whose quotient may be +0)
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = __builtin_copysignf(q[i], v[i]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w = e2m1x2_into<0>(0u, q[8 * h + 0], q[8 * h + 1]);
      w = e2m1x2_into<1>(w, q[8 * h + 2], q[8 * h + 3]);
      w = e2m1x2_into<2>(w, q[8 * h + 4], q[8 * h + 5]);
      packed[h] = e2m1x2_into<3>(w, q[8 * h + 6], q[8 * h + 7]);
    }
  }
  return sb;
}

// The same quantizer for a quarter of a 16-element block held by one lane
// (four lanes per block): ab is the whole block's max |v|, so the block
// scale is the one quantize_block16 computes; returns it and writes the
// quarter's four codes (element 2j in the low nibble) to bits16.
__device__ __forceinline__ uint32_t quantize_quarter4(const float (&v)[4], float ab, float ts,
                                                      uint32_t& bits16) {
#pragma clang fp contract(off)
  uint32_t sb = 0;
  if (ts != 0.0f) {
    const float six_ts = 6.0f * ts;
    float r;
    if (div_fast_ok(six_ts)) r = div_refined(ab, six_ts, recip_refined(six_ts));
    else r = __fdiv_rn(ab, six_ts);
    sb = e4m3_rne_satfinite(r);
  }
  float d = e4m3_to_f32(sb) * ts;
  bits16 = 0;
  if (d != 0.0f) {
    float q[4];
    if (div_fast_ok(d)) {
      const float y = recip_refined(d);
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = div_refined(v[i], d, y);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = __fdiv_rn(v[i], d);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = __builtin_copysignf(q[i], v[i]);
    bits16 = e2m1x2_into<1>(e2m1x2_into<0>(0u, q[0], q[1]), q[2], q[3]);
  }
  return sb;
}

// The same quantizer for one element held by one lane (sixteen lanes per
// block): ab is the block's max |v|; returns the block scale code and writes
// the element's signed E2M1 code to code4.
__device__ __forceinline__ uint32_t quantize_one(float v, float ab, float ts, uint32_t& code4) {
#pragma clang fp contract(off)
  uint32_t sb = 0;
  if (ts != 0.0f) {
    const float six_ts = 6.0f * ts;
    float r;
    if (div_fast_ok(six_ts)) r = div_refined(ab, six_ts, recip_refined(six_ts));
    else r = __fdiv_rn(ab, six_ts);
    sb = e4m3_rne_satfinite(r);
  }
  const float d = e4m3_to_f32(sb) * ts;
  code4 = 0;
  if (d != 0.0f) {
    float q;
    if (div_fast_ok(d)) q = div_refined(v, d, recip_refined(d));
    else q = __fdiv_rn(v, d);
    code4 = e2m1x2_into<0>(0u, __builtin_copysignf(q, v), 0.0f) & 0xFu;
  }
  return sb;
}

__device__ __forceinline__ float tensor_scale_from_amax(float amax) {
  return amax == 0.0f ? 0.0f : __fdiv_rn(amax, TS_DIVISOR);
}

// SwiGLU gate: SiLU(g) * u with SiLU(z) = z / (1 + e^-z), fp32, hardware
// exp and reciprocal (a few ulp; the NVFP4 quantizer downstream is exact on
// whatever h this produces).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------- wave ops
// Make this wave's LDS stores visible to its other lanes' later LDS loads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

// Cross-lane reductions on DPP (gfx9 family): quad permutes and row mirrors
// reduce within 16-lane rows, row broadcasts (15, 31) fold the rows; lane 63
// ends with the full-wave result, read back as a wave-uniform scalar.  Lanes
// a DPP move does not write (masked rows) take `old`, the operation's identity.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_mov(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}

template <typename Op>
__device__ __forceinline__ int dpp_wave_reduce(int v, int ident, Op op) {
  v = op(v, dpp_mov<0xB1>(ident, v));          // quad_perm [1,0,3,2]
  v = op(v, dpp_mov<0x4E>(ident, v));          // quad_perm [2,3,0,1]
  v = op(v, dpp_mov<0x141>(ident, v));         // row_half_mirror
  v = op(v, dpp_mov<0x140>(ident, v));         // row_mirror
  v = op(v, dpp_mov<0x142, 0xA>(ident, v));    // row_bcast:15 into rows 1, 3
  v = op(v, dpp_mov<0x143, 0xC>(ident, v));    // row_bcast:31 into rows 2, 3
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float dpp_wave_max(float v) {
  return __int_as_float(dpp_wave_reduce(__float_as_int(v), __float_as_int(-INFINITY),
      [](int a, int b) { return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b))); }));
}

__device__ __forceinline__ int dpp_wave_min(int v) {
  return dpp_wave_reduce(v, 0x7FFFFFFF, [](int a, int b) { return min(a, b); });
}

__device__ __forceinline__ float dpp_wave_sum(float v) {
  return __int_as_float(dpp_wave_reduce(__float_as_int(v), 0,
      [](int a, int b) { return __float_as_int(__int_as_float(a) + __int_as_float(b)); }));
}

// Top-k of one token's logits by one wave (E <= 64 * PER, k <= TOPK_MAX_K).
// Lane l holds logits l*PER .. l*PER+PER-1 as order-preserving integer keys
// (-0 folded into +0); the order is (key descending, id ascending), so exact
// ties go to the lower expert id.
// Fast path: the k-th largest of the 64 lane maxima is a lower bound of the
// k-th largest logit (the k largest lane maxima are k distinct logits), so
// every winner's key is at or above that lane maximum's top 16 bits, found
// bit by bit from ballot counts.  The few keys at or above it (typically
// k to 2k) are compacted into LDS, each candidate lane counts the candidates
// that beat it (its rank), and the winners land in LDS slots by rank.  When
// more than 64 keys pass the bound (many equal or nearly equal logits) the
// full selection runs instead: each lane sorts its keys, then k rounds take
// the wave maximum of the lanes' heads (DPP) and pop it from the lowest lane
// holding it (lower lane = lower ids).  Keys and ids live in vector
// registers (ext_vector), which keeps the compiler from turning the selects
// into indexed private-array accesses.  The winners' softmax, renormalised
// over the k, is summed on DPP with winner r in lane r either way, so both
// paths give the same weights bit for bit.  Lane r < k returns winner r.
// scr: TOPK_SCR_INTS ints of LDS owned by this wave.
constexpr int TOPK_MAX_K = 32;
constexpr int TOPK_SCR_INTS = 128 + 2 * TOPK_MAX_K;

__device__ __forceinline__ int float_order_key(float f) {
  const int i = __float_as_int(f + 0.0f);             // -0 -> +0
  return i ^ ((i >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float order_key_float(int k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}

template <int PER>
__device__ __forceinline__ void topk_wave(const float* __restrict__ lrow, int E, int k, int lane,
                                          int* scr, int* out_id, float* out_w) {
  typedef int ivec __attribute__((ext_vector_type(PER)));
  constexpr int KMIN = (int)0x80000000;
  constexpr int CBITS = PER >= 16 ? 5 : PER >= 8 ? 4 : PER >= 4 ? 3 : PER >= 2 ? 2 : 1;
  ivec key, id;
  if (E == 64 * PER) {                       // full lanes: plain loads, all in flight at once
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      id[i] = lane * PER + i;
      key[i] = float_order_key(lrow[lane * PER + i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      id[i] = e;
      key[i] = e < E ? float_order_key(lrow[e]) : KMIN;
    }
  }
  // ---- lower bound: top 16 bits of the k-th largest lane maximum
  int m = key[0];
#pragma unroll
  for (int i = 1; i < PER; ++i) m = max(m, key[i]);
  const uint32_t mp = ((uint32_t)m ^ 0x80000000u) >> 16;           // unsigned order, 16-bit prefix
  uint32_t P = 0;
#pragma unroll
  for (int b = 15; b >= 0; --b) {
    const uint32_t c = P | (1u << b);
    if (__popcll(__ballot(mp >= c)) >= (unsigned)k) P = c;
  }
  const int thr = (int)((P << 16) ^ 0x80000000u);
  // ---- candidates (keys >= thr): per-lane count, exclusive prefix over lanes
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) cnt += key[i] >= thr ? 1 : 0;
  int off = 0, n_c = 0;
#pragma unroll
  for (int b = 0; b < CBITS; ++b) {
    const uint64_t bm = __ballot((cnt >> b) & 1);
    off += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u)) << b;
    n_c += __popcll(bm) << b;
  }
  int* wid = scr + 128;                      // winner r's id
  int* wkey = scr + 128 + TOPK_MAX_K;        // winner r's key
  if (n_c <= 64) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (key[i] >= thr) {
        scr[off] = key[i];
        scr[64 + off] = id[i];
        ++off;
      }
    }
    wave_lds_sync();
    const int ck = lane < n_c ? scr[lane] : KMIN;
    const int ci = lane < n_c ? scr[64 + lane] : 0x7FFFFFFF;
    int rank = 0;
    for (int j = 0; j < n_c; ++j) {
      const int kj = __builtin_amdgcn_readlane(ck, j), ij = __builtin_amdgcn_readlane(ci, j);
      rank += (kj > ck || (kj == ck && ij < ci)) ? 1 : 0;
    }
    if (lane < n_c && rank < k) {
      wid[rank] = ci;
      wkey[rank] = ck;
    }
    wave_lds_sync();
  } else {
    // sort descending by (key desc, id asc): odd-even transposition network
#pragma unroll
    for (int pass = 0; pass < PER; ++pass) {
#pragma unroll
      for (int i = pass & 1; i + 1 < PER; i += 2) {
        const int a = key[i], b = key[i + 1], ia = id[i], ib = id[i + 1];
        const bool sw = b > a;                           // equal keys keep id order
        key[i] = sw ? b : a;
        key[i + 1] = sw ? a : b;
        id[i] = sw ? ib : ia;
        id[i + 1] = sw ? ia : ib;
      }
    }
    for (int r = 0; r < k; ++r) {
      const int M = dpp_wave_reduce(key[0], KMIN, [](int a, int b) { return max(a, b); });
      const uint64_t hit = __ballot(key[0] == M);
      const int wl = __ffsll((unsigned long long)hit) - 1;        // lowest lane holding M
      const bool pop = lane == wl;
      scr[pop ? 64 + r : lane] = id[0];
      if (lane == 0) wkey[r] = M;
      ivec ks, is;
#pragma unroll
      for (int i = 0; i + 1 < PER; ++i) {
        ks[i] = key[i + 1];
        is[i] = id[i + 1];
      }
      ks[PER - 1] = KMIN;
      is[PER - 1] = id[PER - 1];
      key = pop ? ks : key;
      id = pop ? is : id;
    }
    wave_lds_sync();
    if (lane < k) wid[lane] = scr[64 + lane];
    wave_lds_sync();
  }
  const int mykey = wkey[lane < k ? lane : 0];
  const int key0 = wkey[0];
  const float z = lane < k ? __expf(order_key_float(mykey) - order_key_float(key0)) : 0.0f;
  const float sum = dpp_wave_sum(z);
  *out_id = wid[lane < k ? lane : 0];
  *out_w = z / sum;
}

// Input rescale of the full-depth decode stack (each layer's output brought
// back to a target RMS before the next layer): s = target / sqrt(mean_h x^2)
// of bf16 rows, by a 256-thread block, in one fixed order that every caller
// shares, so the same row gives the same s bits in the standalone rescale
// kernel, the router blocks and the quantizer blocks: thread t sums the
// squares of elements 8t .. 8t+7, 8t+2048 .. (fp32 FMAs in element order),
// then a DPP sum per wave and ((w0 + w1) + w2) + w3; IEEE division and square
// root; 0 for a zero row.  T rows at once (T <= 16): red holds 4 T floats,
// rsc receives the T scales (block-uniform after the call).  Every thread of
// the block must call it.
__device__ __forceinline__ void rows_rms_scales(const uint16_t* __restrict__ x, int T, int H, float target,
                                                int tid, float* red, float* rsc) {
  for (int t = 0; t < T; ++t) {
    const uint16_t* xr = x + (size_t)t * H;
    float ss = 0.0f;
    for (int c = tid * 8; c < H; c += 256 * 8) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = bf16_to_f32(vw[i] & 0xFFFF), b = bf16_to_f32(vw[i] >> 16);
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
      }
    }
    ss = dpp_wave_sum(ss);
    if ((tid & 63) == 0) red[4 * t + (tid >> 6)] = ss;
  }
  __syncthreads();
  if (tid < T) {
    const float total = ((red[4 * tid] + red[4 * tid + 1]) + red[4 * tid + 2]) + red[4 * tid + 3];
    const float ms = __fdiv_rn(total, (float)H);
    rsc[tid] = ms > 0.0f ? __fdiv_rn(target, __fsqrt_rn(ms)) : 0.0f;
  }
  __syncthreads();
}

// One router logit row (expert `row`) for T <= 16 tokens by a 256-thread
// block: thread t reads float4s t, t+256, ... of the fp32 row (all loads
// issued first) and the matching bf16 x; fp32 FMAs, a DPP sum per wave and a
// fixed-order sum of the four waves through LDS (red: 4*T floats).
constexpr int RROW_MAXF4 = 4;            // H <= 4096

// TB tokens of one router row: every x load of the batch is issued before
// the first sum (straight-line, clamped indices; a float4 past the row takes
// x = 0, which adds exactly 0), then one DPP sum per token.
template <int TB>
__device__ __forceinline__ void router_row_tokens(const uint16_t* __restrict__ x,
                                                  const float4_t (&wv)[RROW_MAXF4], int t0, int T,
                                                  int H, int tid, float* red, const float* rsc) {
  const int nf4 = H / 4;
  u32x2 xb[TB][RROW_MAXF4];
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    const u32x2* xr = reinterpret_cast<const u32x2*>(x + (size_t)min(t0 + tt, T - 1) * H);
#pragma unroll
    for (int i = 0; i < RROW_MAXF4; ++i) xb[tt][i] = xr[min(tid + 256 * i, nf4 - 1)];
  }
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    if (t0 + tt >= T) break;
    float acc = 0.0f;
    const float sc = rsc ? rsc[t0 + tt] : 1.0f;
#pragma unroll
    for (int i = 0; i < RROW_MAXF4; ++i) {
      const bool ok = tid + 256 * i < nf4;
      uint32_t lo = ok ? xb[tt][i].x : 0u, hi = ok ? xb[tt][i].y : 0u;
      if (rsc) {                                         // the rescaled input bf16(x s)
        lo = bf16x2_scaled(lo, sc);
        hi = bf16x2_scaled(hi, sc);
      }
      acc = fmaf(wv[i].x, bf16_to_f32(lo & 0xFFFF), acc);
      acc = fmaf(wv[i].y, bf16_to_f32(lo >> 16), acc);
      acc = fmaf(wv[i].z, bf16_to_f32(hi & 0xFFFF), acc);
      acc = fmaf(wv[i].w, bf16_to_f32(hi >> 16), acc);
    }
    acc = dpp_wave_sum(acc);
    if ((tid & 63) == 0) red[(tid >> 6) * 16 + t0 + tt] = acc;
  }
}

// One router logit row (expert `row`) for T <= 16 tokens by a 256-thread
// block: thread t holds float4s t, t+256, ... of the fp32 row (clamped
// loads, all issued first) and reads the matching bf16 x of up to eight
// tokens at once; fp32 FMAs, a DPP sum per wave and a fixed-order sum of the
// four waves through LDS (red: 4*16 floats).
// in_rms > 0: the input is rescaled to RMS in_rms per token (the logits are
// those of bf16(x s)); the scales are taken into rsc (T floats of LDS) while
// the weight row's loads are in flight.
__device__ __forceinline__ void router_row_block(const uint16_t* __restrict__ x,
                                                 const float* __restrict__ W,
                                                 const float* __restrict__ bias, int T, int E, int H,
                                                 int row, float* __restrict__ logits, int tid,
                                                 float* red, float in_rms = 0.0f, float* rsc = nullptr) {
  const int nf4 = H / 4;
  float4_t wv[RROW_MAXF4];
  const float4_t* wr = reinterpret_cast<const float4_t*>(W + (size_t)row * H);
#pragma unroll
  for (int i = 0; i < RROW_MAXF4; ++i) wv[i] = wr[min(tid + 256 * i, nf4 - 1)];
  if (in_rms > 0.0f) rows_rms_scales(x, T, H, in_rms, tid, red, rsc);
  else rsc = nullptr;
  if (T == 1) {
    router_row_tokens<1>(x, wv, 0, T, H, tid, red, rsc);
  } else {
    for (int t0 = 0; t0 < T; t0 += 8) router_row_tokens<8>(x, wv, t0, T, H, tid, red, rsc);
  }
  __syncthreads();
  if (tid < T) {
    const float v = ((red[tid] + red[16 + tid]) + red[32 + tid]) + red[48 + tid];
    logits[(size_t)tid * E + row] = v + (bias ? bias[row] : 0.0f);
  }
}

// Runtime dispatch on E (E <= 1024).  scr: 64 + k ints of LDS for this wave.
__device__ __forceinline__ void topk_wave_any(const float* __restrict__ lrow, int E, int k, int lane,
                                              int* scr, int* out_id, float* out_w) {
  if (E <= 64) topk_wave<1>(lrow, E, k, lane, scr, out_id, out_w);
  else if (E <= 128) topk_wave<2>(lrow, E, k, lane, scr, out_id, out_w);
  else if (E <= 256) topk_wave<4>(lrow, E, k, lane, scr, out_id, out_w);
  else if (E <= 512) topk_wave<8>(lrow, E, k, lane, scr, out_id, out_w);
  else topk_wave<16>(lrow, E, k, lane, scr, out_id, out_w);
}

// NVFP4 of one bf16 row by a whole block (one tensor scale for the row): each
// thread loads its 16-element blocks once, the row amax goes through DPP and
// LDS (red: one float per wave), then each thread quantizes its blocks.
// Every thread of the block must call it.
// rescale: quantize bf16(x s) instead of x (the stack's rescaled input).
__device__ __forceinline__ void quantize_row_bf16_block(const uint16_t* __restrict__ xr, int H,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales,
                                                        float* __restrict__ ts_out, int tid,
                                                        int nthreads, float* red,
                                                        bool rescale = false, float s = 1.0f) {
  constexpr int MAXB = 4;
  const int nblk = H / 16;
  u32x4 raw[MAXB][2];
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = tid + nthreads * i;
    if (b < nblk) {
      const u32x4* p = reinterpret_cast<const u32x4*>(xr + b * 16);
      raw[i][0] = p[0];
      raw[i][1] = p[1];
      if (rescale) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          raw[i][h] = u32x4{bf16x2_scaled(raw[i][h].x, s), bf16x2_scaled(raw[i][h].y, s),
                            bf16x2_scaled(raw[i][h].z, s), bf16x2_scaled(raw[i][h].w, s)};
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    if (tid + nthreads * i < nblk) {
      const uint32_t w[8] = {raw[i][0].x, raw[i][0].y, raw[i][0].z, raw[i][0].w,
                             raw[i][1].x, raw[i][1].y, raw[i][1].z, raw[i][1].w};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        amax = fmaxf(amax, fabsf(__uint_as_float(w[kk] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(w[kk] & 0xFFFF0000u)));
      }
    }
  }
  amax = dpp_wave_max(amax);
  const int nw = nthreads >> 6;
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
  for (int w = 1; w < nw; ++w) amax = fmaxf(amax, red[w]);
  const float ts = tensor_scale_from_amax(amax);
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = tid + nthreads * i;
    if (b < nblk) {
      const uint32_t w[8] = {raw[i][0].x, raw[i][0].y, raw[i][0].z, raw[i][0].w,
                             raw[i][1].x, raw[i][1].y, raw[i][1].z, raw[i][1].w};
      float v[16];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        v[2 * kk] = __uint_as_float(w[kk] << 16);
        v[2 * kk + 1] = __uint_as_float(w[kk] & 0xFFFF0000u);
      }
      uint32_t pk[2];
      const uint32_t sb = quantize_block16(v, ts, pk);
      *reinterpret_cast<u32x2*>(codes + b * 8) = u32x2{pk[0], pk[1]};
      scales[b] = (uint8_t)sb;
    }
  }
  if (tid == 0) *ts_out = ts;
}

// NVFP4 of one bf16 row by one wave (one tensor scale for the row): pass 1
// takes the row amax, pass 2 quantizes whole 16-element blocks per lane.
__device__ __forceinline__ void quantize_row_bf16_wave(const uint16_t* __restrict__ xr, int H,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       float* __restrict__ ts_out, int lane) {
  constexpr int MAXB = 4;                             // 16-element blocks per lane held (H <= 4096)
  const int nblk = H / 16;
  if (nblk <= 64 * MAXB) {                            // the row fits in registers: one read
    const int b0 = 0;
    u32x4 raw[MAXB][2];
#pragma unroll
    for (int i = 0; i < MAXB; ++i) {
      const int b = b0 + lane + 64 * i;
      if (b < nblk) {
        const u32x4* p = reinterpret_cast<const u32x4*>(xr + b * 16);
        raw[i][0] = p[0];
        raw[i][1] = p[1];
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXB; ++i) {
      if (b0 + lane + 64 * i < nblk) {
        const uint32_t w[8] = {raw[i][0].x, raw[i][0].y, raw[i][0].z, raw[i][0].w,
                               raw[i][1].x, raw[i][1].y, raw[i][1].z, raw[i][1].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          amax = fmaxf(amax, fabsf(__uint_as_float(w[k] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(w[k] & 0xFFFF0000u)));
        }
      }
    }
    amax = dpp_wave_max(amax);
    const float ts = tensor_scale_from_amax(amax);
#pragma unroll
    for (int i = 0; i < MAXB; ++i) {
      const int b = b0 + lane + 64 * i;
      if (b < nblk) {
        const uint32_t w[8] = {raw[i][0].x, raw[i][0].y, raw[i][0].z, raw[i][0].w,
                               raw[i][1].x, raw[i][1].y, raw[i][1].z, raw[i][1].w};
        float v[16];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v[2 * k] = __uint_as_float(w[k] << 16);
          v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
        uint32_t pk[2];
        const uint32_t sb = quantize_block16(v, ts, pk);
        *reinterpret_cast<u32x2*>(codes + b * 8) = u32x2{pk[0], pk[1]};
        scales[b] = (uint8_t)sb;
      }
    }
    if (lane == 0) *ts_out = ts;
    return;
  }
  // rows longer than 64 * MAXB blocks: two passes over memory
  float amax = 0.0f;
  for (int b = lane; b < nblk; b += 64) {
    const u32x4* p = reinterpret_cast<const u32x4*>(xr + b * 16);
    u32x4 a = p[0], c = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
    }
  }
  amax = dpp_wave_max(amax);
  const float ts = tensor_scale_from_amax(amax);
  for (int b = lane; b < nblk; b += 64) {
    const u32x4* p = reinterpret_cast<const u32x4*>(xr + b * 16);
    u32x4 a = p[0], c = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    uint32_t pk[2];
    const uint32_t sb = quantize_block16(v, ts, pk);
    *reinterpret_cast<u32x2*>(codes + b * 8) = u32x2{pk[0], pk[1]};
    scales[b] = (uint8_t)sb;
  }
  if (lane == 0) *ts_out = ts;
}

// E2M1 pair (one byte, low nibble first) -> f16x2, exact.
template <int SEL>
__device__ __forceinline__ half2_t fp4x2_to_f16x2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL);
}

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// 32 codebook elements: 3-bit indices from three index words (layout above:
// w0 and w1 hold bits 0-1 of elements 0-15 and 16-31, two bits per element,
// w2 bit 2 of all 32), 8 fp16 entries in cb (4 dwords).  The table is split
// into the entries' low bytes and high bytes (8 bytes each).  Per four
// elements 4q .. 4q+3: one shift and mask bring their bits 0-1 to bits 0-1 of
// bytes 0-3, one shift and one and-or add bit 2, so byte j holds element
// 4q + j's index, which is also the byte number of its entry in either table
// half; two byte permutes of the table halves by that word give the four low
// bytes and the four high bytes, and two more interleave them into two pairs
// of fp16 values.  Four VALU operations per element fewer than spreading three
// bit-planes by multiplies and building a selector per element pair.
template <int Q>
__device__ __forceinline__ uint32_t cb_quad_index(uint32_t w0, uint32_t w1, uint32_t w2) {
  static_assert(Q >= 0 && Q < 8, "quad of a 32-element chunk");
  const uint32_t lo = ((Q < 4 ? w0 : w1) >> (2 * (Q & 3))) & 0x03030303u;
  const uint32_t b2 = Q >= 2 ? (w2 >> (Q - 2)) : (w2 << (2 - Q));
  return (b2 & 0x04040404u) | lo;
}

// The table split of one group's entries: low bytes of entries 0..3 / 4..7,
// high bytes of entries 0..3 / 4..7.
struct CbTable {
  uint32_t lo0, lo1, hi0, hi1;
};
__device__ __forceinline__ CbTable cb_table(u32x4 cb) {
  return CbTable{__builtin_amdgcn_perm(cb.y, cb.x, 0x06040200u), __builtin_amdgcn_perm(cb.w, cb.z, 0x06040200u),
                 __builtin_amdgcn_perm(cb.y, cb.x, 0x07050301u), __builtin_amdgcn_perm(cb.w, cb.z, 0x07050301u)};
}

// Elements 4q .. 4q+3 (q = Q) as two f16 pairs.
template <int Q>
__device__ __forceinline__ void cb_decode4(uint32_t w0, uint32_t w1, uint32_t w2, const CbTable& t,
                                           half2_t& e01, half2_t& e23) {
  const uint32_t idx = cb_quad_index<Q>(w0, w1, w2);
  const uint32_t lo = __builtin_amdgcn_perm(t.lo1, t.lo0, idx);
  const uint32_t hi = __builtin_amdgcn_perm(t.hi1, t.hi0, idx);
  const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // {lo0, hi0, lo1, hi1}
  const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);   // {lo2, hi2, lo3, hi3}
  e01 = *reinterpret_cast<const half2_t*>(&a);
  e23 = *reinterpret_cast<const half2_t*>(&b);
}

// Elements 8*S8 .. 8*S8+7 of a 32-element chunk as four f16 pairs.
template <int S8>
__device__ __forceinline__ void cb_decode8(uint32_t w0, uint32_t w1, uint32_t w2, const CbTable& t,
                                           half2_t (&o)[4]) {
  cb_decode4<2 * S8>(w0, w1, w2, t, o[0], o[1]);
  cb_decode4<2 * S8 + 1>(w0, w1, w2, t, o[2], o[3]);
}

__device__ __forceinline__ void dequant32_cb(uint32_t w0, uint32_t w1, uint32_t w2, u32x4 cb,
                                             half2_t (&o)[16]) {
  const CbTable t = cb_table(cb);
  cb_decode8<0>(w0, w1, w2, t, *reinterpret_cast<half2_t(*)[4]>(&o[0]));
  cb_decode8<1>(w0, w1, w2, t, *reinterpret_cast<half2_t(*)[4]>(&o[4]));
  cb_decode8<2>(w0, w1, w2, t, *reinterpret_cast<half2_t(*)[4]>(&o[8]));
  cb_decode8<3>(w0, w1, w2, t, *reinterpret_cast<half2_t(*)[4]>(&o[12]));
}

}  // namespace moe
