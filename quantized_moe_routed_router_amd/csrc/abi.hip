// C ABI of the MoE library: argument validation (host only, before any
// launch), error codes and per-thread messages, and dispatch to the kernels'
// launchers.  The refusal style - fail up front and say the numbers - follows
// the engine's startup guard (blog "Capy Flash ...", section "Where the
// experts live"), here for device memory.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "common.hpp"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return MOE_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define NEED_PTR(p)                                                                       \
  do {                                                                                    \
    if (!(p)) return fail(MOE_ERR_INVALID, "%s: %s is NULL", fn, #p);                    \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID, "%s: %s = %p is not 16-byte aligned", \
                                   fn, #p, (const void*)(p));                             \
  } while (0)

#define OPT_PTR(p)                                                                        \
  do {                                                                                    \
    if ((p) && !aligned16(p))                                                             \
      return fail(MOE_ERR_INVALID, "%s: %s = %p is not 16-byte aligned", fn, #p,          \
                  (const void*)(p));                                                      \
  } while (0)

int check_dims(const char* fn, const moe_dims* d) {
  if (!d) return fail(MOE_ERR_INVALID, "%s: dims is NULL", fn);
  if (d->E < 1 || d->E > MOE_MAX_E)
    return fail(MOE_ERR_SHAPE, "%s: E = %d outside [1, %d]", fn, d->E, MOE_MAX_E);
  if (d->k < 1 || d->k > d->E || d->k > MOE_MAX_K)
    return fail(MOE_ERR_SHAPE, "%s: k = %d outside [1, min(E = %d, %d)]", fn, d->k, d->E, MOE_MAX_K);
  if (d->H < 128 || d->H % 128)
    return fail(MOE_ERR_SHAPE, "%s: H = %d is not a positive multiple of 128", fn, d->H);
  if (d->I < 128 || d->I % 128)
    return fail(MOE_ERR_SHAPE, "%s: I = %d is not a positive multiple of 128", fn, d->I);
  if (d->fmt_gate_up != MOE_FMT_NVFP4 && d->fmt_gate_up != MOE_FMT_CB3G128)
    return fail(MOE_ERR_INVALID, "%s: fmt_gate_up = %d is not a known format", fn, d->fmt_gate_up);
  return MOE_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err; }

int moe_capacity_verdict(size_t bytes_free, size_t bytes_needed) {
  if (bytes_needed <= bytes_free) return ok();
  return fail(MOE_ERR_CAPACITY,
              "moe_check_capacity: need %zu bytes (%.2f GiB) of HBM, %zu bytes (%.2f GiB) free; "
              "set MOE_HBM_GUARD=0 to skip this check",
              bytes_needed, bytes_needed / 1073741824.0, bytes_free, bytes_free / 1073741824.0);
}

int moe_check_capacity(int device, size_t bytes_needed) {
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_status(e, "moe_check_capacity: hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_check_capacity: device %d is %s, the library is built for gfx950",
                device, prop.gcnArchName);
  const char* guard = getenv("MOE_HBM_GUARD");
  if (guard && strcmp(guard, "0") == 0) return ok();
  int prev = 0;
  e = hipGetDevice(&prev);
  if (e != hipSuccess) return hip_status(e, "moe_check_capacity: hipGetDevice");
  if (prev != device && (e = hipSetDevice(device)) != hipSuccess)
    return hip_status(e, "moe_check_capacity: hipSetDevice");
  size_t free_b = 0, total_b = 0;
  e = hipMemGetInfo(&free_b, &total_b);
  if (prev != device) (void)hipSetDevice(prev);
  if (e != hipSuccess) return hip_status(e, "moe_check_capacity: hipMemGetInfo");
  return moe_capacity_verdict(free_b, bytes_needed);
}

size_t moe_packed_bytes(const moe_dims* d, int which) {
  if (check_dims("moe_packed_bytes", d) != MOE_OK) return 0;
  if (which == 0)
    return (size_t)d->E * (d->fmt_gate_up == MOE_FMT_NVFP4 ? moe::gate_up_expert_bytes(d->H, d->I)
                                                           : moe::cb_gate_up_expert_bytes(d->H, d->I));
  if (which == 1) return (size_t)d->E * moe::down_expert_bytes(d->H, d->I);
  fail(MOE_ERR_INVALID, "moe_packed_bytes: which = %d is not 0 or 1", which);
  return 0;
}

size_t moe_ffn_workspace_bytes(const moe_dims* d, int T, int prefill) {
  if (check_dims("moe_ffn_workspace_bytes", d) != MOE_OK) return 0;
  if (T < 0) return 0;
  size_t b = prefill ? moe::prefill_workspace_bytes(d->E, d->H, d->I, d->k, T)
                     : moe::decode_workspace_bytes(d->E, d->H, d->I, d->k, T);
  return b ? b : 256;
}

size_t moe_permute_workspace_bytes(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_E) return 0;
  return moe::permute_workspace_bytes(T, k, E);
}

int moe_quantize_act(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales, float* ts,
                     void* stream) {
  const char* fn = "moe_quantize_act";
  if (T < 0) return fail(MOE_ERR_SHAPE, "%s: T = %d is negative", fn, T);
  if (H < 16 || H % 16) return fail(MOE_ERR_SHAPE, "%s: H = %d is not a positive multiple of 16", fn, H);
  if (T == 0) return ok();
  NEED_PTR(x); NEED_PTR(codes); NEED_PTR(scales); NEED_PTR(ts);
  return hip_status(moe::launch_act_quant(x, T, H, codes, scales, ts, as_stream(stream)), fn);
}

int moe_quantize_weights(const float* W, int n_mat, int rows, int cols, uint8_t* codes,
                         uint8_t* scales, float* ts, void* stream) {
  const char* fn = "moe_quantize_weights";
  if (n_mat < 0 || rows < 0) return fail(MOE_ERR_SHAPE, "%s: n_mat = %d, rows = %d must be >= 0", fn, n_mat, rows);
  if (cols < 16 || cols % 16) return fail(MOE_ERR_SHAPE, "%s: cols = %d is not a positive multiple of 16", fn, cols);
  if ((size_t)rows * cols / 16 * (size_t)n_mat > ((size_t)1 << 40))
    return fail(MOE_ERR_SHAPE, "%s: %d x %d x %d elements is too large", fn, n_mat, rows, cols);
  if (n_mat == 0) return ok();
  NEED_PTR(ts);
  if (rows > 0) { NEED_PTR(W); NEED_PTR(codes); NEED_PTR(scales); }
  return hip_status(moe::launch_weight_quant(W, n_mat, rows, cols, codes, scales, ts, as_stream(stream)), fn);
}

int moe_pack_nvfp4(const moe_dims* d, int e0, int n, const uint8_t* gc, const uint8_t* gs,
                   const uint8_t* uc, const uint8_t* us, const uint8_t* dc, const uint8_t* ds,
                   void* gate_up, void* down, void* stream) {
  const char* fn = "moe_pack_nvfp4";
  int st = check_dims(fn, d);
  if (st) return st;
  if (e0 < 0 || n < 0 || e0 + n > d->E)
    return fail(MOE_ERR_SHAPE, "%s: experts [%d, %d) outside [0, E = %d)", fn, e0, e0 + n, d->E);
  if (n == 0) return ok();
  const bool gu = gc || gs || uc || us, dn = dc || ds;
  if (gu) {
    if (d->fmt_gate_up != MOE_FMT_NVFP4)
      return fail(MOE_ERR_UNSUPPORTED, "%s: gate/up format is %d, not NVFP4", fn, d->fmt_gate_up);
    NEED_PTR(gc); NEED_PTR(gs); NEED_PTR(uc); NEED_PTR(us); NEED_PTR(gate_up);
  }
  if (dn) { NEED_PTR(dc); NEED_PTR(ds); NEED_PTR(down); }
  if (!gu && !dn) return fail(MOE_ERR_INVALID, "%s: no gate/up and no down inputs", fn);
  return hip_status(moe::launch_pack_nvfp4(false, d->H, d->I, e0, n, (uint8_t*)gc, (uint8_t*)gs,
                                           (uint8_t*)uc, (uint8_t*)us, (uint8_t*)dc, (uint8_t*)ds,
                                           (uint8_t*)gate_up, (uint8_t*)down, as_stream(stream)),
                    fn);
}

int moe_unpack_nvfp4(const moe_dims* d, int e0, int n, uint8_t* gc, uint8_t* gs, uint8_t* uc,
                     uint8_t* us, uint8_t* dc, uint8_t* ds, const void* gate_up, const void* down,
                     void* stream) {
  const char* fn = "moe_unpack_nvfp4";
  int st = check_dims(fn, d);
  if (st) return st;
  if (e0 < 0 || n < 0 || e0 + n > d->E)
    return fail(MOE_ERR_SHAPE, "%s: experts [%d, %d) outside [0, E = %d)", fn, e0, e0 + n, d->E);
  if (n == 0) return ok();
  const bool gu = gc || gs || uc || us, dn = dc || ds;
  if (gu) {
    if (d->fmt_gate_up != MOE_FMT_NVFP4)
      return fail(MOE_ERR_UNSUPPORTED, "%s: gate/up format is %d, not NVFP4", fn, d->fmt_gate_up);
    NEED_PTR(gc); NEED_PTR(gs); NEED_PTR(uc); NEED_PTR(us); NEED_PTR(gate_up);
  }
  if (dn) { NEED_PTR(dc); NEED_PTR(ds); NEED_PTR(down); }
  if (!gu && !dn) return fail(MOE_ERR_INVALID, "%s: no gate/up and no down outputs", fn);
  return hip_status(moe::launch_pack_nvfp4(true, d->H, d->I, e0, n, gc, gs, uc, us, dc, ds,
                                           (uint8_t*)gate_up, (uint8_t*)down, as_stream(stream)),
                    fn);
}

int moe_pack_codebook(const moe_dims* d, int e0, int n, const uint16_t* gcb, const uint8_t* gidx,
                      const uint16_t* ucb, const uint8_t* uidx, void* gate_up, void* stream) {
  const char* fn = "moe_pack_codebook";
  int st = check_dims(fn, d);
  if (st) return st;
  if (d->fmt_gate_up != MOE_FMT_CB3G128)
    return fail(MOE_ERR_INVALID, "%s: dims->fmt_gate_up = %d, expected MOE_FMT_CB3G128", fn, d->fmt_gate_up);
  if (e0 < 0 || n < 0 || e0 + n > d->E)
    return fail(MOE_ERR_SHAPE, "%s: experts [%d, %d) outside [0, E = %d)", fn, e0, e0 + n, d->E);
  if (n == 0) return ok();
  NEED_PTR(gcb); NEED_PTR(gidx); NEED_PTR(ucb); NEED_PTR(uidx); NEED_PTR(gate_up);
  return hip_status(moe::launch_pack_codebook(d->H, d->I, e0, n, gcb, gidx, ucb, uidx,
                                              (uint8_t*)gate_up, as_stream(stream)),
                    fn);
}

int moe_router_topk(const uint16_t* x, const float* W_r, const float* bias, int T,
                    const moe_dims* d, int32_t* ids, float* w, float* logits, void* stream) {
  const char* fn = "moe_router_topk";
  int st = check_dims(fn, d);
  if (st) return st;
  if (T < 0) return fail(MOE_ERR_SHAPE, "%s: T = %d is negative", fn, T);
  if (T == 0) return ok();
  NEED_PTR(x); NEED_PTR(W_r); OPT_PTR(bias); NEED_PTR(ids); NEED_PTR(w); NEED_PTR(logits);
  return hip_status(moe::launch_router(x, W_r, bias, T, d->E, d->H, d->k, ids, w, logits,
                                       as_stream(stream)),
                    fn);
}

static int check_ffn(const char* fn, const moe_dims* d, const moe_experts* ex, const moe_actq* xq,
                     const int32_t* ids, int T, float* out, void* ws, size_t ws_bytes,
                     const moe_ffn_debug* dbg, bool prefill) {
  int st = check_dims(fn, d);
  if (st) return st;
  if (!ex) return fail(MOE_ERR_INVALID, "%s: experts is NULL", fn);
  if (!xq) return fail(MOE_ERR_INVALID, "%s: xq is NULL", fn);
  NEED_PTR(ex->gate_up); NEED_PTR(ex->down); NEED_PTR(ex->ts_down);
  if (d->fmt_gate_up == MOE_FMT_NVFP4) { NEED_PTR(ex->ts_gate); NEED_PTR(ex->ts_up); }
  NEED_PTR(xq->codes); NEED_PTR(xq->scales); NEED_PTR(xq->ts);
  NEED_PTR(ids); NEED_PTR(out); NEED_PTR(ws);
  if (dbg) { OPT_PTR(dbg->h); OPT_PTR(dbg->h_codes); OPT_PTR(dbg->h_scales); OPT_PTR(dbg->h_ts); }
  OPT_PTR(ex->h_ts);
  const size_t need = moe_ffn_workspace_bytes(d, T, prefill ? 1 : 0);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace is %zu bytes, %zu needed for T = %d", fn, ws_bytes, need, T);
  return MOE_OK;
}

static moe::FfnArgs make_args(const moe_dims* d, const moe_experts* ex, const moe_actq* xq,
                              const int32_t* ids, int T, float* out, const moe_ffn_debug* dbg) {
  moe::FfnArgs a{};
  a.E = d->E; a.H = d->H; a.I = d->I; a.k = d->k; a.T = T; a.fmt = d->fmt_gate_up;
  a.gate_up = (const uint8_t*)ex->gate_up; a.down = (const uint8_t*)ex->down;
  a.ts_gate = ex->ts_gate; a.ts_up = ex->ts_up; a.ts_down = ex->ts_down;
  a.h_ts = ex->h_ts;
  a.x_codes = xq->codes; a.x_scales = xq->scales; a.x_ts = xq->ts;
  a.ids = ids; a.out = out;
  if (dbg) { a.dbg_h = dbg->h; a.dbg_h_codes = dbg->h_codes; a.dbg_h_scales = dbg->h_scales; a.dbg_h_ts = dbg->h_ts; }
  return a;
}

int moe_expert_ffn_decode(const moe_dims* d, const moe_experts* ex, const moe_actq* xq,
                          const int32_t* ids, int T, float* out, void* ws, size_t ws_bytes,
                          const moe_ffn_debug* dbg, void* stream) {
  const char* fn = "moe_expert_ffn_decode";
  if (T < 1 || T > MOE_DECODE_MAX_T)
    return fail(MOE_ERR_SHAPE, "%s: T = %d outside [1, %d]", fn, T, MOE_DECODE_MAX_T);
  int st = check_ffn(fn, d, ex, xq, ids, T, out, ws, ws_bytes, dbg, false);
  if (st) return st;
  if (!moe::decode_fmt_ok(d->H, T, d->fmt_gate_up))
    return fail(MOE_ERR_UNSUPPORTED, "%s: codebook gate/up at H = %d, T = %d: the decode kernels need whole "
                "128-element groups per K split and at most 3 groups per wave (use moe_expert_ffn_prefill)",
                fn, d->H, T);
  if (T > 1 && d->H > 3072)
    return fail(MOE_ERR_SHAPE, "%s: H = %d above 3072 needs T = 1 (activation staging is 8*H*2 bytes of LDS)", fn, d->H);
  if (d->H > 10240 || d->I > 2560)
    return fail(MOE_ERR_SHAPE, "%s: H = %d, I = %d: decode takes H <= 10240, I <= 2560", fn, d->H, d->I);
  return hip_status(moe::launch_ffn_decode(make_args(d, ex, xq, ids, T, out, dbg), ws, as_stream(stream)), fn);
}

size_t moe_layer_decode_workspace_bytes(const moe_dims* d, int T) {
  if (check_dims("moe_layer_decode_workspace_bytes", d) != MOE_OK) return 0;
  if (T < 1 || T > MOE_LAYER_MAX_T) return 0;
  return moe::layer_decode_workspace_bytes(d->E, d->H, d->I, d->k, T);
}

}  // extern "C"

namespace {

// Validation and launch shared by moe_layer_decode and
// moe_layer_decode_noalloc (which passes the device's scratch array).
int layer_decode_checked(const char* fn, const moe_dims* d, const moe_experts* ex, const uint16_t* x,
                         const float* W_r, const float* bias, int T, int add_residual, uint16_t* y,
                         int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream,
                         float in_rms = 0.0f) {
  int st = check_dims(fn, d);
  if (st) return st;
  if (T < 1 || T > MOE_LAYER_MAX_T)
    return fail(MOE_ERR_SHAPE, "%s: T = %d outside [1, %d]", fn, T, MOE_LAYER_MAX_T);
  if (!moe::decode_fmt_ok(d->H, T, d->fmt_gate_up))
    return fail(MOE_ERR_UNSUPPORTED, "%s: codebook gate/up at H = %d, T = %d: the decode kernels need whole "
                "128-element groups per K split and at most 3 groups per wave", fn, d->H, T);
  if (d->H % 256 || d->H > 4096)
    return fail(MOE_ERR_SHAPE, "%s: H = %d must be a multiple of 256 and <= 4096", fn, d->H);
  if (d->I > 2560) return fail(MOE_ERR_SHAPE, "%s: I = %d above 2560", fn, d->I);
  if (T > 1 && d->H > 3072)
    return fail(MOE_ERR_SHAPE, "%s: H = %d above 3072 needs T = 1", fn, d->H);
  if (!ex) return fail(MOE_ERR_INVALID, "%s: experts is NULL", fn);
  NEED_PTR(ex->gate_up); NEED_PTR(ex->down); NEED_PTR(ex->ts_down);
  if (d->fmt_gate_up == MOE_FMT_NVFP4) { NEED_PTR(ex->ts_gate); NEED_PTR(ex->ts_up); }
  OPT_PTR(ex->h_ts);
  NEED_PTR(x); NEED_PTR(W_r); OPT_PTR(bias); NEED_PTR(y); OPT_PTR(ids); OPT_PTR(w); NEED_PTR(ws);
  const size_t need = moe::layer_decode_workspace_bytes(d->E, d->H, d->I, d->k, T);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace is %zu bytes, %zu needed for T = %d", fn, ws_bytes, need, T);
  moe::LayerArgs L{};
  L.E = d->E; L.H = d->H; L.I = d->I; L.k = d->k; L.T = T;
  L.x = x; L.W_r = W_r; L.bias = bias; L.residual = add_residual != 0;
  L.gate_up = (const uint8_t*)ex->gate_up; L.down = (const uint8_t*)ex->down;
  L.ts_gate = ex->ts_gate; L.ts_up = ex->ts_up; L.ts_down = ex->ts_down;
  L.h_ts = ex->h_ts;
  L.y = y; L.ids_out = ids; L.w_out = w;
  L.in_rms = in_rms;
  L.fmt = d->fmt_gate_up;
  return hip_status(moe::launch_layer_decode(L, ws, as_stream(stream)), fn);
}

}  // namespace

// The no-allocation variant's workspace: one array per GPU, in the library's
// device code, held until the process ends.  Host code never passes this
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current, on the entry point's first call there.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int scratch_of_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "moe_layer_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d outside the %d the library tracks", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "moe_layer_decode_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress(scratch) gave NULL on device %d", fn, dev);
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_decode(const moe_dims* d, const moe_experts* ex, const uint16_t* x, const float* W_r,
                     const float* bias, int T, int add_residual, uint16_t* y, int32_t* ids, float* w,
                     void* ws, size_t ws_bytes, void* stream) {
  return layer_decode_checked("moe_layer_decode", d, ex, x, W_r, bias, T, add_residual, y, ids, w, ws,
                              ws_bytes, stream);
}

int moe_layer_decode_rescaled(const moe_dims* d, const moe_experts* ex, const uint16_t* x_in,
                              float target_rms, const float* W_r, const float* bias, int T, uint16_t* y,
                              int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_layer_decode_rescaled";
  if (!(target_rms > 0.0f) || !(target_rms < 3.0e38f))
    return fail(MOE_ERR_INVALID, "%s: target_rms = %g must be positive and finite", fn, (double)target_rms);
  if (d && d->H % 8) return fail(MOE_ERR_SHAPE, "%s: H = %d is not a multiple of 8", fn, d->H);
  return layer_decode_checked(fn, d, ex, x_in, W_r, bias, T, 1, y, ids, w, ws, ws_bytes, stream, target_rms);
}

int moe_layer_decode_noalloc(const moe_dims* d, const moe_experts* ex, const uint16_t* x,
                             const float* W_r, const float* bias, int T, int add_residual, uint16_t* y,
                             int32_t* ids, float* w, void* stream) {
  const char* fn = "moe_layer_decode_noalloc";
  int st = check_dims(fn, d);
  if (st) return st;
  if (T < 1 || T > MOE_LAYER_MAX_T)
    return fail(MOE_ERR_SHAPE, "%s: T = %d outside [1, %d]", fn, T, MOE_LAYER_MAX_T);
  const size_t need = moe::layer_decode_workspace_bytes(d->E, d->H, d->I, d->k, T);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "%s: E = %d, H = %d, I = %d, k = %d, T = %d need %zu bytes of workspace, above the "
                "%zu-byte scratch array (use moe_layer_decode with a workspace)",
                fn, d->E, d->H, d->I, d->k, T, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_of_current_device(fn, &ws);
  if (st) return st;
  return layer_decode_checked(fn, d, ex, x, W_r, bias, T, add_residual, y, ids, w, ws,
                              (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

int moe_ffn_prefill_tile_rows(const moe_dims* d, int T) {
  const char* fn = "moe_ffn_prefill_tile_rows";
  int st = check_dims(fn, d);
  if (st) return st;
  if (T < 1) return fail(MOE_ERR_SHAPE, "%s: T = %d must be >= 1", fn, T);
  ok();
  return moe::prefill_tile_rows(d->E, d->H, d->I, d->k, T, d->fmt_gate_up);
}

int moe_expert_ffn_prefill(const moe_dims* d, const moe_experts* ex, const moe_actq* xq,
                           const int32_t* ids, int T, float* out, void* ws, size_t ws_bytes,
                           const moe_ffn_debug* dbg, void* stream) {
  const char* fn = "moe_expert_ffn_prefill";
  if (T < 1) return fail(MOE_ERR_SHAPE, "%s: T = %d must be >= 1", fn, T);
  if (d && d->I > 4096) return fail(MOE_ERR_SHAPE, "%s: I = %d above 4096", fn, d->I);
  if ((long long)T * (d ? d->k : 1) > (1LL << 30)) return fail(MOE_ERR_SHAPE, "%s: T = %d too large", fn, T);
  int st = check_ffn(fn, d, ex, xq, ids, T, out, ws, ws_bytes, dbg, true);
  if (st) return st;
  return hip_status(moe::launch_ffn_prefill(make_args(d, ex, xq, ids, T, out, dbg), ws, as_stream(stream)), fn);
}

int moe_combine(const float* out, const float* w, const uint16_t* residual, int T, int k, int H,
                uint16_t* y, void* stream) {
  const char* fn = "moe_combine";
  if (T < 0) return fail(MOE_ERR_SHAPE, "%s: T = %d is negative", fn, T);
  if (k < 1 || k > MOE_MAX_K) return fail(MOE_ERR_SHAPE, "%s: k = %d outside [1, %d]", fn, k, MOE_MAX_K);
  if (H < 8 || H % 8) return fail(MOE_ERR_SHAPE, "%s: H = %d is not a positive multiple of 8", fn, H);
  if (T == 0) return ok();
  NEED_PTR(out); NEED_PTR(w); OPT_PTR(residual); NEED_PTR(y);
  return hip_status(moe::launch_combine(out, w, residual, T, k, H, y, as_stream(stream)), fn);
}

int moe_rms_norm(const uint16_t* x, int T, int H, float target_rms, uint16_t* y, void* stream) {
  const char* fn = "moe_rms_norm";
  if (T < 0) return fail(MOE_ERR_SHAPE, "%s: T = %d is negative", fn, T);
  if (H < 8 || H % 8) return fail(MOE_ERR_SHAPE, "%s: H = %d is not a positive multiple of 8", fn, H);
  if (!(target_rms > 0.0f) || !(target_rms < 3.0e38f))
    return fail(MOE_ERR_INVALID, "%s: target_rms = %g must be positive and finite", fn, (double)target_rms);
  if (T == 0) return ok();
  NEED_PTR(x); NEED_PTR(y);
  return hip_status(moe::launch_rms_norm(x, T, H, target_rms, y, as_stream(stream)), fn);
}

int moe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  const char* fn = "moe_stream_read";
  if (bytes % 16) return fail(MOE_ERR_SHAPE, "%s: bytes = %zu is not a multiple of 16", fn, bytes);
  if (bytes == 0) return ok();
  NEED_PTR(src); NEED_PTR(sink);
  return hip_status(moe::launch_stream_read(src, bytes, sink, as_stream(stream)), fn);
}

int moe_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_permute";
  if (T < 0) return fail(MOE_ERR_SHAPE, "%s: T = %d is negative", fn, T);
  if (k < 1 || k > MOE_MAX_K) return fail(MOE_ERR_SHAPE, "%s: k = %d outside [1, %d]", fn, k, MOE_MAX_K);
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_SHAPE, "%s: E = %d outside [1, %d]", fn, E, MOE_MAX_E);
  if ((long long)T * k > (1LL << 30)) return fail(MOE_ERR_SHAPE, "%s: T*k = %lld too large", fn, (long long)T * k);
  NEED_PTR(counts); NEED_PTR(offsets); NEED_PTR(ws);
  if (T > 0) { NEED_PTR(ids); NEED_PTR(perm); NEED_PTR(inv); }
  const size_t need = moe::permute_workspace_bytes(T, k, E);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace is %zu bytes, %zu needed", fn, ws_bytes, need);
  return hip_status(moe::launch_permute(ids, T, k, E, counts, offsets, perm, inv, ws, nullptr, nullptr, 0,
                                        as_stream(stream)),
                    fn);
}

}  // extern "C"
