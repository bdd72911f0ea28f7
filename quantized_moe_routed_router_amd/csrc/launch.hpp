// Host-side launchers of the kernels (one per .hip file); the C ABI in
// abi.hip validates arguments and calls these.  Each returns the launch's
// hipError_t and enqueues on stream s only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_act_quant(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales,
                            float* ts, hipStream_t s);
hipError_t launch_weight_quant(const float* W, int n_mat, int rows, int cols, uint8_t* codes,
                               uint8_t* scales, float* ts, hipStream_t s);
hipError_t launch_pack_nvfp4(bool unpack, int H, int I, int e0, int n, uint8_t* gc, uint8_t* gs,
                             uint8_t* uc, uint8_t* us, uint8_t* dc, uint8_t* ds,
                             uint8_t* gate_up, uint8_t* down, hipStream_t s);
hipError_t launch_pack_codebook(int H, int I, int e0, int n, const uint16_t* gcb,
                                const uint8_t* gidx, const uint16_t* ucb, const uint8_t* uidx,
                                uint8_t* gate_up, hipStream_t s);

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);
hipError_t launch_router(const uint16_t* x, const float* W_r, const float* bias, int T, int E,
                         int H, int k, int32_t* ids, float* w, float* logits, hipStream_t s);

struct FfnArgs {
  int E, H, I, k, T, fmt;
  const uint8_t* gate_up;
  const uint8_t* down;
  const float* ts_gate;
  const float* ts_up;
  const float* ts_down;
  const uint8_t* x_codes;
  const uint8_t* x_scales;
  const float* x_ts;
  const int32_t* ids;
  float* out;
  float* dbg_h;
  uint8_t* dbg_h_codes;
  uint8_t* dbg_h_scales;
  float* dbg_h_ts;
  const float* h_ts;   // static h tensor scale per expert, or null (per-row amax)
};

size_t decode_workspace_bytes(int E, int H, int I, int k, int T);

struct LayerArgs {
  int E, H, I, k, T;
  const uint16_t* x;
  const float* W_r;
  const float* bias;
  bool residual;
  const uint8_t* gate_up;
  const uint8_t* down;
  const float* ts_gate;
  const float* ts_up;
  const float* ts_down;
  const float* h_ts;
  uint16_t* y;
  int32_t* ids_out;
  float* w_out;
  float in_rms;        // > 0: the layer's input is bf16(x s), s = in_rms / rms(x) per token
  int fmt;             // gate/up weight format
};
// Whether the decode kernels take gate/up format fmt at these shapes.
bool decode_fmt_ok(int H, int T, int fmt);
size_t layer_decode_workspace_bytes(int E, int H, int I, int k, int T);
hipError_t launch_layer_decode(const LayerArgs& L, void* ws, hipStream_t s);
hipError_t launch_ffn_decode(const FfnArgs& a, void* ws, hipStream_t s);

size_t prefill_workspace_bytes(int E, int H, int I, int k, int T);
hipError_t launch_ffn_prefill(const FfnArgs& a, void* ws, hipStream_t s);
// Row-tile height (32, 128 or 256) launch_ffn_prefill uses for these shapes.
int prefill_tile_rows(int E, int H, int I, int k, int T, int fmt);

// res_scale [T] or null: the residual is bf16(residual * res_scale[t]).
hipError_t launch_combine(const float* out, const float* w, const uint16_t* residual, int T, int k,
                          int H, uint16_t* y, hipStream_t s, const float* res_scale = nullptr);
hipError_t launch_rms_norm(const uint16_t* x, int T, int H, float target, uint16_t* y, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);

size_t permute_workspace_bytes(int T, int k, int E);
// A second list of row tiles: experts with fewer than split_rows rows are
// tiled there, by BM rows, instead of in the first list (unused when
// tile_map is nullptr).
struct TileSplit {
  int32_t* tile_prefix = nullptr;
  int32_t* tile_map = nullptr;
  int BM = 0;
  int split_rows = 0;
};
// Counting sort of ids; also writes the per-expert tile prefix for grouped
// GEMMs with BM-row tiles when tile_prefix != nullptr ([E+1] entries), and
// when tile_map != nullptr one record per tile {expert, first row, end row of
// the expert, 0} (4 ints each, tile_prefix[E] records); the same for the
// second list when split.tile_map is set.
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                          int32_t* tile_prefix, int32_t* tile_map, int BM, hipStream_t s,
                          const TileSplit& split = TileSplit{});

}  // namespace moe
