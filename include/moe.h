/*
 * moe.h - C ABI of the routed-expert NVFP4 (W4A4) MoE layer for MI355X (gfx950).
 *
 * The operation is the routed-expert path of the engine described on the
 * pages: a token's hidden state goes through a softmax top-k router to k of E
 * routed experts, each a gated (SwiGLU) FFN with gate/up and down projections
 * (release post "capy-flash v0.7.1: a 125B MoE on 64 GB of RAM ...", section
 * "What shipped": 48 layers x 512 experts, gate/up weights and down
 * projections), on NVFP4 weights with NVFP4 activations ("W4A4", same post,
 * section "Why it matters"), and the k expert outputs are combined with the
 * renormalised router weights.  Every picked expert is computed (forum
 * repost, paragraph "Where it stands": no route tail skip).
 *
 * NVFP4 (public format): value = E2M1(code) * E4M3(block scale) * fp32 tensor
 * scale; one block scale per 16 consecutive elements along the contraction
 * axis.  Quantizer, in fp32 round-to-nearest-even, step by step:
 *   amax = max|v| over the scope; ts = amax / 2688 (0 if amax = 0);
 *   per block sb = E4M3_rne_satfinite(max|v_block| / (6*ts)) (0 if ts = 0);
 *   d = E4M3(sb) * ts; code = sign(v)<<3 | E2M1_rne_sat(|v / d|) (0 if d = 0).
 * Scopes: one weight matrix (expert, projection); one token row of x; one
 * (token, slot) row of h.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller, unless a
 *    comment says otherwise; arrays are dense, row-major, 16-byte aligned.
 *  - bf16 values are passed as their uint16_t bit patterns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work: they never allocate, free, synchronize or read
 *    device memory back; outputs are valid once the stream reaches the work.
 *  - Arguments are validated on the host before anything is enqueued.  On a
 *    failure the call returns a negative moe_status, enqueues nothing, and
 *    moe_last_error() (per host thread) describes the failure with the
 *    offending numbers.  Nothing throws across this boundary.
 *  - NaN / Inf inputs are outside the contract (not checked).
 *  - The library is built for gfx950 only.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 7
#define MOE_DECODE_MAX_T 64   /* largest token count moe_expert_ffn_decode takes */
#define MOE_LAYER_MAX_T 16    /* largest token count moe_layer_decode takes */
#define MOE_MAX_E 1024
#define MOE_MAX_K 32

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,      /* null pointer, misaligned pointer, bad enum     */
  MOE_ERR_SHAPE = -2,        /* sizes outside what the kernels take            */
  MOE_ERR_UNSUPPORTED = -3,  /* device is not gfx950, or format not supported  */
  MOE_ERR_CAPACITY = -4,     /* not enough free HBM for the request            */
  MOE_ERR_HIP = -5,          /* a HIP runtime call failed (message has it)     */
  MOE_ERR_WORKSPACE = -6     /* workspace smaller than *_workspace_bytes()     */
} moe_status;

enum { MOE_FMT_NVFP4 = 0, MOE_FMT_CB3G128 = 1 };

/* Layer shape.  E experts, hidden H, expert width I, k experts per token.
 * Requirements: 1 <= k <= min(E, MOE_MAX_K), E <= MOE_MAX_E, H % 128 == 0,
 * I % 128 == 0.  fmt_gate_up selects the gate/up weight format (down is
 * always NVFP4). */
typedef struct moe_dims {
  int32_t E, H, I, k;
  int32_t fmt_gate_up;
} moe_dims;

/* One layer's resident expert weights, in the packed layouts written by
 * moe_pack_nvfp4 / moe_pack_codebook (sizes from moe_packed_bytes).
 * ts_* are the per-(expert, projection) fp32 tensor scales, [E] each;
 * ts_gate / ts_up are ignored (may be NULL) for MOE_FMT_CB3G128.
 * h_ts [E] or NULL: a static (calibrated) NVFP4 tensor scale for h, the down
 * projection's input, per expert, as NVIDIA's NVFP4 checkpoints carry for
 * activations (the engine was built for that quantisation: forum repost,
 * paragraph "What it's for").  NULL: each (t, slot) row of h takes
 * amax / 2688 (dynamic).  With a static scale the quantizer skips the
 * amax step; values beyond 6 * 448 * h_ts[e] saturate.  Must be >= 0 and finite. */
typedef struct moe_experts {
  const void* gate_up;
  const void* down;
  const float* ts_gate;
  const float* ts_up;
  const float* ts_down;
  const float* h_ts;
} moe_experts;

/* NVFP4 activations, one tensor scale per token row:
 * codes [T, H/2] (element 2j in the low nibble), scales [T, H/16] E4M3,
 * ts [T] fp32. */
typedef struct moe_actq {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
} moe_actq;

/* Optional intermediate outputs of the expert FFN (any field may be NULL),
 * indexed by flat pair p = t*k + slot:
 *   h [T*k, I] fp32  = SiLU(gate) * up;  h_codes [T*k, I/2], h_scales
 *   [T*k, I/16], h_ts [T*k] = NVFP4 of each h row (the down projection's
 *   input).  Requesting any of them can route a call through its plainer
 *   path (with static h scales the prefill GEMM otherwise codes h^ in its
 *   epilogue and keeps no fp32 h); the results are the same bit for bit. */
typedef struct moe_ffn_debug {
  float* h;
  uint8_t* h_codes;
  uint8_t* h_scales;
  float* h_ts;
} moe_ffn_debug;

/* ------------------------------------------------------------------ */
/* Hot path                                                            */
/* ------------------------------------------------------------------ */

/* Router (blog "Capy Flash ...", section "Where the experts live": each
 * token runs only some of the experts; rank order per the forum repost,
 * "Where it stands").
 *   logits[t, e] = sum_h x[t, h] * W_r[e, h] (+ bias[e])   fp32
 *   keep the k largest (ties to the lower id), in descending order
 *   w[t, i] = exp(l_i - l_1) / sum_j exp(l_j - l_1)   (softmax over all
 *             experts restricted to the top k and renormalised)
 * x [T, H] bf16; W_r [E, H] fp32; bias [E] fp32 or NULL;
 * ids [T, k] int32 out; w [T, k] fp32 out; logits [T, E] fp32 out (also the
 * kernels' scratch; required).  T >= 0 (T = 0 enqueues nothing). */
int moe_router_topk(const uint16_t* x, const float* W_r, const float* bias, int T,
                    const moe_dims* dims, int32_t* ids, float* w, float* logits,
                    void* stream);

/* Activation quantizer: x [T, H] bf16 -> NVFP4 with one tensor scale per
 * row (see the quantizer above).  codes [T, H/2], scales [T, H/16], ts [T]
 * outputs.  H % 16 == 0.  Bit-exact with the fp32 step definition. */
int moe_quantize_act(const uint16_t* x, int T, int H, uint8_t* codes,
                     uint8_t* scales, float* ts, void* stream);

/* Expert FFN for a small batch (decode), 1 <= T <= MOE_DECODE_MAX_T: weight
 * GEMVs that read each distinct expert once (the faster expert FFN up to
 * about 16 tokens per call; from about 32 tokens the prefill entry's 32-row
 * expert tiles are).
 * For each (t, slot), e = ids[t, slot]:
 *   g = W^_gate[e] x^_t,  u = W^_up[e] x^_t,  h = SiLU(g) * u  (fp32)
 *   h^ = NVFP4(h) per (t, slot) row,  out[t, slot, :] = W^_down[e] h^
 * (release post, "What shipped": gate/up and down projections; "Why it
 * matters": W4A4).  Each distinct expert's weights are read once per call.
 * out [T, k, H] fp32.  ws: device workspace of at least
 * moe_ffn_workspace_bytes(dims, T, 0) bytes (contents need not be
 * initialised).  dbg may be NULL.  Both gate/up formats; the codebook format
 * needs whole 128-element groups per K split (H / 128 divisible by the split
 * count, 1 at one token up to H = 2560, else 2 or 4) and is refused with
 * MOE_ERR_UNSUPPORTED otherwise (the prefill entry takes every shape). */
int moe_expert_ffn_decode(const moe_dims* dims, const moe_experts* experts,
                          const moe_actq* xq, const int32_t* ids, int T, float* out,
                          void* ws, size_t ws_bytes, const moe_ffn_debug* dbg,
                          void* stream);

/* Expert FFN for any T >= 1 (prefill): same result as the decode entry, as a
 * grouped GEMM over the token-by-expert permutation (stable counting sort
 * of the (t, slot) pairs by expert) on matrix cores.  Takes both gate/up
 * formats; I <= 4096.  ws: at least moe_ffn_workspace_bytes(dims, T, 1) bytes.
 * Routing-dependent sizes never reach the host. */
int moe_expert_ffn_prefill(const moe_dims* dims, const moe_experts* experts,
                           const moe_actq* xq, const int32_t* ids, int T, float* out,
                           void* ws, size_t ws_bytes, const moe_ffn_debug* dbg,
                           void* stream);

/* Row-tile height of the grouped GEMMs moe_expert_ffn_prefill runs for these
 * dims at T tokens (a host-side query, no device work): 32 while the experts
 * hold few rows on average (T*k <= 96*E, 64*E for codebook gate/up: one wave per
 * 32-row expert tile and 64-row weight tile, operands straight to the matrix
 * cores, each expert tile's weights read once), else 256 where the shapes
 * allow 256 x 256 tiles (H % 256 == 0, I >= 256), else 128.  In the 256-row
 * tiling the experts routed fewer than 128 rows in the call take 32-row
 * tiles instead (a second tile list, run by trailing blocks of the 256-row
 * launches with the 32-row tile body).  All of them give
 * the same result up to fp32 accumulation order.  Returns a negative
 * MOE_ERR_* code on invalid dims or T < 1. */
int moe_ffn_prefill_tile_rows(const moe_dims* dims, int T);

/* The whole decode layer for 1 <= T <= MOE_LAYER_MAX_T tokens.  One token:
 * three kernels (router logits + NVFP4 of x; top-k, ranked in every gate/up
 * block, + gate/up; down + weighted combine).  Several tokens: the top-k and
 * h^ run once in kernels of their own, and the down projection carries the
 * combine up to 8 tokens (a block per column slice and token), else a
 * combine kernel follows.  The result is that of moe_router_topk,
 * moe_quantize_act, moe_expert_ffn_decode and moe_combine in sequence,
 *   y = bf16_rne( [x if add_residual] + sum_i w_i * FFN_{ids_i}(x^) ),
 * bit for bit where both run the same kernels (T*k <= 16, or T > 8); between
 * those the down dots sum in another fp32 order (ids, w and h^ equal, y one
 * bf16 rounding of the same sum).
 * x [T, H] bf16 (also the residual), W_r [E, H] fp32, bias [E] or NULL,
 * y [T, H] bf16 out; ids [T, k] int32 and w [T, k] fp32 outputs, or NULL.
 * ws: at least moe_layer_decode_workspace_bytes(dims, T) bytes (contents
 * need not be initialised); calls sharing a workspace must not overlap.
 * Both gate/up formats (as moe_expert_ffn_decode); H % 256 == 0, H <= 4096,
 * I <= 2560. */
size_t moe_layer_decode_workspace_bytes(const moe_dims* dims, int T);
int moe_layer_decode(const moe_dims* dims, const moe_experts* experts, const uint16_t* x,
                     const float* W_r, const float* bias, int T, int add_residual,
                     uint16_t* y, int32_t* ids, float* w, void* ws, size_t ws_bytes,
                     void* stream);

/* One layer of the full-depth decode stack in the kernels of
 * moe_layer_decode: x_in [T, H] bf16 is the previous layer's output, the
 * layer's input is x = bf16_rne(x_in * s) with s = target_rms / sqrt(mean_h
 * x_in^2) per token (fp32, the same fixed-order sum and IEEE division and
 * square root as moe_rms_norm, so x is bit-identical to moe_rms_norm's
 * output), and y = bf16_rne(x + sum_i w_i FFN_{ids_i}(x^)) (the residual is
 * the rescaled input).  The same result as moe_rms_norm followed by
 * moe_layer_decode with add_residual = 1; at one token the rescale runs
 * inside the layer's first kernel (one launch fewer), at several tokens a
 * rescale kernel writes the rows into the workspace first.  The rescale is
 * the glue this project puts between the 48 stacked layers (not one of the
 * pages' steps; see moe_rms_norm).  Arguments and workspace as for
 * moe_layer_decode; target_rms positive and finite. */
int moe_layer_decode_rescaled(const moe_dims* dims, const moe_experts* experts, const uint16_t* x_in,
                              float target_rms, const float* W_r, const float* bias, int T,
                              uint16_t* y, int32_t* ids, float* w, void* ws, size_t ws_bytes,
                              void* stream);

/* The fused decode layer without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, arithmetic and
 * results as moe_layer_decode, whose kernels it runs; the workspace is a
 * MOE_NOALLOC_SCRATCH_BYTES array in the library's device memory, one per
 * GPU, held until the process ends (its address is looked up on the first
 * call on each device, with that device current).  The call allocates and
 * frees nothing.  Refused (MOE_ERR_WORKSPACE, with the numbers) when
 * moe_layer_decode_workspace_bytes(dims, T) exceeds MOE_NOALLOC_SCRATCH_BYTES
 * (the Flash-Next layer, H 2560, I 640, E 512, k 10, needs about 3.4 MB at
 * T = 16).  Every call on a GPU uses that GPU's one array: calls that overlap
 * on one GPU (other streams, other host threads) race and must be ordered by
 * the caller.  The array's contents left by the last call are never read
 * before being written.  The stream must belong to the current device. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_layer_decode_noalloc(const moe_dims* dims, const moe_experts* experts, const uint16_t* x,
                             const float* W_r, const float* bias, int T, int add_residual,
                             uint16_t* y, int32_t* ids, float* w, void* stream);

/* Weighted combine (release post, "Why it matters": partial sums are kept in
 * FP32): y[t, :] = bf16_rne( r[t, :] + sum_i w[t, i] * out[t, i, :] ), summed
 * in fp32 in slot order and rounded once.  out [T, k, H] fp32, w [T, k] fp32,
 * residual [T, H] bf16 or NULL (r = 0), y [T, H] bf16 out. */
int moe_combine(const float* out, const float* w, const uint16_t* residual, int T,
                int k, int H, uint16_t* y, void* stream);

/* Row-wise RMS rescale, the glue between the layers of the full-depth
 * decode stack (48 layers, residual add, routing near uniform at every
 * layer): y[t, :] = bf16_rne( x[t, :] * target_rms / sqrt(mean_h x[t, h]^2) ),
 * fp32 sum of squares, IEEE division and square root; a zero row gives 0.
 * Not one of the pages' steps: it keeps each layer's input at the first
 * layer's scale, without which the residual stream of random-weight layers
 * grows until the routing is one-hot and bf16 overflows.  x, y [T, H] bf16
 * (may alias); H % 8 == 0; target_rms positive and finite. */
int moe_rms_norm(const uint16_t* x, int T, int H, float target_rms, uint16_t* y, void* stream);

/* ------------------------------------------------------------------ */
/* Sizes, weight preparation, permute, capacity                        */
/* ------------------------------------------------------------------ */

/* Workspace bytes for moe_expert_ffn_decode (prefill = 0) or
 * moe_expert_ffn_prefill (prefill = 1) at T tokens; 0 on invalid dims. */
size_t moe_ffn_workspace_bytes(const moe_dims* dims, int T, int prefill);

/* Bytes of one layer's packed gate/up (which = 0) or down (which = 1)
 * weights for all E experts; 0 on invalid dims. */
size_t moe_packed_bytes(const moe_dims* dims, int which);

/* NVFP4 weight quantizer (the experts' weight format: release post
 * "capy-flash v0.7.1 ...", section "What shipped", NVFP4 experts; the format's
 * steps as at the top of this header), batched over n_mat matrices of
 * [rows, cols], each with its own tensor scale (one expert projection each).
 * W [n_mat, rows, cols] fp32 -> codes [n_mat, rows, cols/2],
 * scales [n_mat, rows, cols/16], ts [n_mat].  cols % 16 == 0.
 * Bit-exact with the fp32 step definition.  ts is also used as scratch. */
int moe_quantize_weights(const float* W, int n_mat, int rows, int cols,
                         uint8_t* codes, uint8_t* scales, float* ts, void* stream);

/* Write experts e0 .. e0+n-1 of a layer into the packed layouts (the resident
 * expert weights: release post, section "What shipped": every layer's routed
 * experts with gate/up weights and down projections; here all of them stay in
 * device memory, where the pages split them between host RAM and a GPU
 * cache).
 * Plain inputs per expert, NVFP4 (codes element 2j in the low nibble):
 *   gate/up codes [n, I, H/2], scales [n, I, H/16];
 *   down codes [n, H, I/2], scales [n, H, I/16].
 * The gate/up group (4 pointers) or the down group may all be NULL to skip
 * it.  gate_up / down: the whole layer's packed buffers. */
int moe_pack_nvfp4(const moe_dims* dims, int e0, int n,
                   const uint8_t* gate_codes, const uint8_t* gate_scales,
                   const uint8_t* up_codes, const uint8_t* up_scales,
                   const uint8_t* down_codes, const uint8_t* down_scales,
                   void* gate_up, void* down, void* stream);

/* Inverse of moe_pack_nvfp4 (same argument meaning, plain arrays written). */
int moe_unpack_nvfp4(const moe_dims* dims, int e0, int n,
                     uint8_t* gate_codes, uint8_t* gate_scales,
                     uint8_t* up_codes, uint8_t* up_scales,
                     uint8_t* down_codes, uint8_t* down_scales,
                     const void* gate_up, const void* down, void* stream);

/* 3-bit group-128 fp16-codebook gate/up weights (release post, "What shipped":
 * q3_g128_fp16 codebooks): each group of 128 consecutive elements of a row
 * has 8 fp16 entries and every weight a 3-bit index.  Inputs for experts
 * e0 .. e0+n-1: gate_cb / up_cb [n, I, H/128, 8] fp16 bits, gate_idx /
 * up_idx [n, I, H] uint8 (0..7).  dims->fmt_gate_up must be
 * MOE_FMT_CB3G128; gate_up is the layer's packed buffer. */
int moe_pack_codebook(const moe_dims* dims, int e0, int n,
                      const uint16_t* gate_cb, const uint8_t* gate_idx,
                      const uint16_t* up_cb, const uint8_t* up_idx,
                      void* gate_up, void* stream);

/* Stable token-by-expert counting sort of the T*k (t, slot) pairs (each
 * expert then runs over the tokens routed to it, as a batch: the routing of
 * the blog "Capy Flash ...", section "Where the experts live", grouped by
 * expert id as in the release post, section "Why it matters"), flat index
 * i = t*k + slot: counts [E], offsets [E+1] (exclusive prefix sum),
 * perm [T*k] (perm[j] = i at sorted position j, sorted by (expert, i)),
 * inv [T*k] (inv[perm[j]] = j).  ws: moe_permute_workspace_bytes bytes. */
size_t moe_permute_workspace_bytes(int T, int k, int E);
int moe_permute(const int32_t* ids, int T, int k, int E, int32_t* counts,
                int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                size_t ws_bytes, void* stream);

/* Refuse up front, with the numbers, when `device` is not gfx950 or has less
 * free HBM than bytes_needed (the blog "Capy Flash ...", section "Where the
 * experts live", describes the same startup refusal for host RAM).  The
 * free-memory check is skipped when the environment sets MOE_HBM_GUARD=0. */
int moe_check_capacity(int device, size_t bytes_needed);

/* The capacity rule alone, on given numbers (host only, no device call):
 * MOE_OK when bytes_needed <= bytes_free, else MOE_ERR_CAPACITY with a
 * message naming both. */
int moe_capacity_verdict(size_t bytes_free, size_t bytes_needed);

/* Measurement helper (not a step of the layer): one streaming read of
 * `bytes` bytes at `src` (device, 16-byte aligned, bytes % 16 == 0) with
 * 16-byte loads spread over the whole GPU, each thread's loads of a pass in
 * flight together: the yardstick for a call that must read that many bytes
 * once.  sink: device buffer of MOE_STREAM_READ_MAX_BLOCKS uint32; its words
 * are written only when a block's XOR of the data equals 0x9E3779B9 (so the
 * loads cannot be dropped); the contents are not a result.  bytes = 0
 * enqueues nothing. */
#define MOE_STREAM_READ_MAX_BLOCKS 2048
int moe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Message of the last failure on this host thread ("" if none). */
const char* moe_last_error(void);

int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
