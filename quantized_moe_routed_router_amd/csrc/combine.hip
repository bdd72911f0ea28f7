// Weighted combine of the k expert outputs of each token, with optional
// residual: y = bf16_rne(r + sum_i w_i o_i), fp32 accumulation in slot order,
// one rounding.  The pages keep expert partial sums in FP32 (release post
// "capy-flash v0.7.1", section "Why it matters").
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// One thread per 8 consecutive hidden elements of one token: reads k x 32 B of
// o and 16 B of residual, writes 16 B of y.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ out,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ residual,
                                                      int T, int k, int H,
                                                      uint16_t* __restrict__ y) {
  const int per_row = H / 8;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx % per_row);
  float acc[8] = {};
  for (int i = 0; i < k; ++i) {
    const float wi = w[(size_t)t * k + i];
    const float4_t* o = reinterpret_cast<const float4_t*>(out + ((size_t)t * k + i) * H + c * 8);
    float4_t a = o[0], b = o[1];
    acc[0] = fmaf(wi, a.x, acc[0]); acc[1] = fmaf(wi, a.y, acc[1]);
    acc[2] = fmaf(wi, a.z, acc[2]); acc[3] = fmaf(wi, a.w, acc[3]);
    acc[4] = fmaf(wi, b.x, acc[4]); acc[5] = fmaf(wi, b.y, acc[5]);
    acc[6] = fmaf(wi, b.z, acc[6]); acc[7] = fmaf(wi, b.w, acc[7]);
  }
  if (residual) {
    u32x4 r = *reinterpret_cast<const u32x4*>(residual + (size_t)t * H + c * 8);
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
                          int H, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const size_t n = (size_t)T * (H / 8);
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(out, w, residual, T, k, H, y);
  return hipGetLastError();
}

}  // namespace moe
