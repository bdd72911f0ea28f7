// Softmax top-k router: fp32 logits of the bf16 hidden state against fp32
// router weights (+ optional per-expert bias), then per token the k largest
// logits (ties to the lower expert id) and their softmax renormalised over the
// selected k.  The pages: every token activates a subset of the experts (blog
// "Capy Flash ...", section "Where the experts live"); picked experts are
// ranked (forum repost, paragraph "Where it stands").
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

// ---------------------------------------------------------------- top-k
// One wave per token; lane l holds logits l, l+64, ... (E <= 1024).  Each of
// the k rounds takes the wave maximum (DPP), then the lowest expert id holding
// it (exact ties go to the lower id), and retires that entry.  The winners'
// softmax, renormalised over the k, is summed on DPP as well.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  __shared__ int scr[4][64 + MOE_MAX_K];
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

hipError_t launch_router(const uint16_t* x, const float* W_r, const float* bias, int T, int E,
                         int H, int k, int32_t* ids, float* w, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= 16 && H % 4 == 0 && H <= 4096) {
    router_gemv_kernel<<<E, 256, 0, s>>>(x, W_r, bias, T, E, H, logits);
  } else {
    router_gemm_kernel<<<dim3((E + 63) / 64, (T + 63) / 64), 256, 0, s>>>(x, W_r, bias, T, E, H, logits);
  }
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
