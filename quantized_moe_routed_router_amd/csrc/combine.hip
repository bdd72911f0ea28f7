// Weighted combine of the k expert outputs of each token, with optional
// residual: y = bf16_rne(r + sum_i w_i o_i), fp32 accumulation in slot order,
// one rounding.  The pages keep expert partial sums in FP32 (release post
// "capy-flash v0.7.1", section "Why it matters").
#include "../../include/moe.h"
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// One thread per 8 consecutive hidden elements of one token: reads k x 32 B of
// o and 16 B of residual, writes 16 B of y.
// res_scale [T] or null: the residual is bf16(residual * res_scale[t]) (the
// stack's rescaled layer input).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ out,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ residual,
                                                      int T, int k, int H,
                                                      uint16_t* __restrict__ y,
                                                      const float* __restrict__ res_scale) {
  const int per_row = H / 8;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx % per_row);
  float acc[8] = {};
  // slots in batches of CB: every load of a batch in flight before its FMAs
  // (slots past k re-read slot k-1 and are not used); FMAs in slot order
  constexpr int CB = 5;
  for (int i0 = 0; i0 < k; i0 += CB) {
    float4_t a[CB], b[CB];
    float wi[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int i = min(i0 + u, k - 1);
      wi[u] = w[(size_t)t * k + i];
      const float4_t* o = reinterpret_cast<const float4_t*>(out + ((size_t)t * k + i) * H + c * 8);
      a[u] = o[0];
      b[u] = o[1];
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (i0 + u < k) {
        acc[0] = fmaf(wi[u], a[u].x, acc[0]); acc[1] = fmaf(wi[u], a[u].y, acc[1]);
        acc[2] = fmaf(wi[u], a[u].z, acc[2]); acc[3] = fmaf(wi[u], a[u].w, acc[3]);
        acc[4] = fmaf(wi[u], b[u].x, acc[4]); acc[5] = fmaf(wi[u], b[u].y, acc[5]);
        acc[6] = fmaf(wi[u], b[u].z, acc[6]); acc[7] = fmaf(wi[u], b[u].w, acc[7]);
      }
    }
  }
  if (residual) {
    u32x4 r = *reinterpret_cast<const u32x4*>(residual + (size_t)t * H + c * 8);
    if (res_scale) {
      const float rs = res_scale[t];
      r = u32x4{bf16x2_scaled(r.x, rs), bf16x2_scaled(r.y, rs), bf16x2_scaled(r.z, rs), bf16x2_scaled(r.w, rs)};
    }
    uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(rw[i] & 0xFFFF);
      acc[2 * i + 1] += bf16_to_f32(rw[i] >> 16);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4*>(y + (size_t)t * H + c * 8) = u32x4{o[0], o[1], o[2], o[3]};
}

hipError_t launch_combine(const float* out, const float* w, const uint16_t* residual, int T, int k,
                          int H, uint16_t* y, hipStream_t s, const float* res_scale) {
  if (T == 0) return hipSuccess;
  const size_t n = (size_t)T * (H / 8);
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(out, w, residual, T, k, H, y, res_scale);
  return hipGetLastError();
}

// Input rescaling between the layers of the full-depth decode stack (the
// reading of "routing near uniform" at every layer: each layer's output is
// brought back to the first layer's input RMS before the next layer; not one
// of the pages' steps).  Block = one token row: fp32 sum of squares (per
// thread, then a fixed-order DPP and cross-wave sum), s = target / sqrt(mean)
// with IEEE division and square root, y = bf16_rne(x * s); a zero row gives 0.
__global__ __launch_bounds__(256) void rms_norm_kernel(const uint16_t* __restrict__ x, int H,
                                                       float target, uint16_t* __restrict__ y) {
  __shared__ float red[4];
  __shared__ float rsc[1];
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint16_t* xr = x + (size_t)t * H;
  rows_rms_scales(xr, 1, H, target, tid, red, rsc);
  const float sc = rsc[0];
  for (int c = tid * 8; c < H; c += 256 * 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
    *reinterpret_cast<u32x4*>(y + (size_t)t * H + c) =
        u32x4{bf16x2_scaled(v.x, sc), bf16x2_scaled(v.y, sc), bf16x2_scaled(v.z, sc), bf16x2_scaled(v.w, sc)};
  }
}

hipError_t launch_rms_norm(const uint16_t* x, int T, int H, float target, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  rms_norm_kernel<<<T, 256, 0, s>>>(x, H, target, y);
  return hipGetLastError();
}

// Measurement helper: one streaming read of a buffer, the yardstick for a
// call that must read a given number of bytes once.  Each thread issues all
// its 16-byte loads of a pass (four, a grid-stride apart) before using any;
// the grid fills every CU.  The data only feed an XOR that is written out in
// the single case that it equals a fixed constant, so the loads stay.
constexpr int SR_THREADS = 256, SR_UNROLL = 4;
__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                 uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * SR_THREADS;
  size_t i = (size_t)blockIdx.x * SR_THREADS + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (SR_UNROLL - 1) * stride < n16; i += SR_UNROLL * stride) {
    u32x4 v[SR_UNROLL];
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + (size_t)SR_THREADS * SR_UNROLL - 1) / ((size_t)SR_THREADS * SR_UNROLL);
  if (blocks > MOE_STREAM_READ_MAX_BLOCKS) blocks = MOE_STREAM_READ_MAX_BLOCKS;
  if (blocks == 0) return hipSuccess;
  stream_read_kernel<<<(unsigned)blocks, SR_THREADS, 0, s>>>(reinterpret_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace moe
