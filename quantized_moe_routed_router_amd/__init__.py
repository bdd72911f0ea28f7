"""Python binding of libmoe.so, the MI355X (gfx950) routed-expert NVFP4 MoE
layer.  Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI (include/moe.h); torch supplies device memory and
streams.

Functions carry the C names and take torch tensors (device memory) where the
C ABI takes device pointers.  A non-zero status raises MoeError with the
library's message.  Loading fails loudly when libmoe.so is missing: there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED = 0, -1, -2, -3
MOE_ERR_CAPACITY, MOE_ERR_HIP, MOE_ERR_WORKSPACE = -4, -5, -6
MOE_FMT_NVFP4, MOE_FMT_CB3G128 = 0, 1
MOE_DECODE_MAX_T = 64      # moe_expert_ffn_decode
MOE_LAYER_MAX_T = 16       # moe_layer_decode


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class moe_dims(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("k", ctypes.c_int32), ("fmt_gate_up", ctypes.c_int32)]


class moe_experts(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("ts_gate", ctypes.c_void_p), ("ts_up", ctypes.c_void_p),
                ("ts_down", ctypes.c_void_p), ("h_ts", ctypes.c_void_p)]


class moe_actq(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("ts", ctypes.c_void_p)]


class moe_ffn_debug(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("h_codes", ctypes.c_void_p),
                ("h_scales", ctypes.c_void_p), ("h_ts", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGS = {
    "moe_abi_version": (_I, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_capacity_verdict": (_I, [_SZ, _SZ]),
    "moe_check_capacity": (_I, [_I, _SZ]),
    "moe_packed_bytes": (_SZ, [ctypes.POINTER(moe_dims), _I]),
    "moe_ffn_workspace_bytes": (_SZ, [ctypes.POINTER(moe_dims), _I, _I]),
    "moe_permute_workspace_bytes": (_SZ, [_I, _I, _I]),
    "moe_ffn_prefill_tile_rows": (_I, [ctypes.POINTER(moe_dims), _I]),
    "moe_quantize_act": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "moe_quantize_weights": (_I, [_P, _I, _I, _I, _P, _P, _P, _P]),
    "moe_pack_nvfp4": (_I, [ctypes.POINTER(moe_dims), _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_unpack_nvfp4": (_I, [ctypes.POINTER(moe_dims), _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_pack_codebook": (_I, [ctypes.POINTER(moe_dims), _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_router_topk": (_I, [_P, _P, _P, _I, ctypes.POINTER(moe_dims), _P, _P, _P, _P]),
    "moe_expert_ffn_decode": (_I, [ctypes.POINTER(moe_dims), ctypes.POINTER(moe_experts),
                                   ctypes.POINTER(moe_actq), _P, _I, _P, _P, _SZ,
                                   ctypes.POINTER(moe_ffn_debug), _P]),
    "moe_expert_ffn_prefill": (_I, [ctypes.POINTER(moe_dims), ctypes.POINTER(moe_experts),
                                    ctypes.POINTER(moe_actq), _P, _I, _P, _P, _SZ,
                                    ctypes.POINTER(moe_ffn_debug), _P]),
    "moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "moe_rms_norm": (_I, [_P, _I, _I, ctypes.c_float, _P, _P]),
    "moe_layer_decode_workspace_bytes": (_SZ, [ctypes.POINTER(moe_dims), _I]),
    "moe_layer_decode": (_I, [ctypes.POINTER(moe_dims), ctypes.POINTER(moe_experts), _P, _P, _P, _I,
                              _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_decode_rescaled": (_I, [ctypes.POINTER(moe_dims), ctypes.POINTER(moe_experts), _P,
                                       ctypes.c_float, _P, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_decode_noalloc": (_I, [ctypes.POINTER(moe_dims), ctypes.POINTER(moe_experts), _P, _P, _P,
                                      _I, _I, _P, _P, _P, _P]),
    "moe_permute": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_stream_read": (_I, [_P, _SZ, _P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m quantized_moe_routed_router_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return sorted(_SIGS)


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dims(E: int, H: int, I: int, k: int, fmt_gate_up: int = MOE_FMT_NVFP4) -> moe_dims:
    return moe_dims(E, H, I, k, fmt_gate_up)


# ------------------------------------------------------------------ sizes

def moe_packed_bytes(d: moe_dims, which: int) -> int:
    return lib().moe_packed_bytes(ctypes.byref(d), which)


def moe_ffn_workspace_bytes(d: moe_dims, T: int, prefill: bool) -> int:
    return lib().moe_ffn_workspace_bytes(ctypes.byref(d), T, 1 if prefill else 0)


def moe_ffn_prefill_tile_rows(d: moe_dims, T: int) -> int:
    """Row-tile height (32, 128 or 256) the prefill entry uses at T tokens
    (with 256, the experts routed fewer than 128 rows take 32-row tiles)."""
    rc = lib().moe_ffn_prefill_tile_rows(ctypes.byref(d), T)
    if rc < 0:
        _check(rc)
    return rc


def moe_permute_workspace_bytes(T: int, k: int, E: int) -> int:
    return lib().moe_permute_workspace_bytes(T, k, E)


def moe_capacity_verdict(bytes_free: int, bytes_needed: int) -> int:
    return lib().moe_capacity_verdict(bytes_free, bytes_needed)


def moe_check_capacity(device: int, bytes_needed: int):
    _check(lib().moe_check_capacity(device, bytes_needed))


def moe_abi_version() -> int:
    return lib().moe_abi_version()


# ------------------------------------------------------------------ hot path

def moe_router_topk(x, W_r, bias, T: int, d: moe_dims, ids, w, logits, stream=None):
    _check(lib().moe_router_topk(_ptr(x), _ptr(W_r), _ptr(bias), T, ctypes.byref(d),
                                 _ptr(ids), _ptr(w), _ptr(logits), _stream(stream)))


def moe_quantize_act(x, T: int, H: int, codes, scales, ts, stream=None):
    _check(lib().moe_quantize_act(_ptr(x), T, H, _ptr(codes), _ptr(scales), _ptr(ts),
                                  _stream(stream)))


def _experts(ex) -> moe_experts:
    return moe_experts(_ptr(ex["gate_up"]), _ptr(ex["down"]), _ptr(ex.get("ts_gate")),
                       _ptr(ex.get("ts_up")), _ptr(ex["ts_down"]), _ptr(ex.get("h_ts")))


def _actq(xq) -> moe_actq:
    return moe_actq(_ptr(xq[0]), _ptr(xq[1]), _ptr(xq[2]))


def _debug(dbg):
    if dbg is None:
        return None
    return ctypes.byref(moe_ffn_debug(_ptr(dbg.get("h")), _ptr(dbg.get("h_codes")),
                                      _ptr(dbg.get("h_scales")), _ptr(dbg.get("h_ts"))))


def moe_expert_ffn_decode(d: moe_dims, experts: dict, xq, ids, T: int, out, ws, ws_bytes: int,
                          dbg: Optional[dict] = None, stream=None):
    ex, aq = _experts(experts), _actq(xq)
    _check(lib().moe_expert_ffn_decode(ctypes.byref(d), ctypes.byref(ex), ctypes.byref(aq),
                                       _ptr(ids), T, _ptr(out), _ptr(ws), ws_bytes,
                                       _debug(dbg), _stream(stream)))


def moe_expert_ffn_prefill(d: moe_dims, experts: dict, xq, ids, T: int, out, ws, ws_bytes: int,
                           dbg: Optional[dict] = None, stream=None):
    ex, aq = _experts(experts), _actq(xq)
    _check(lib().moe_expert_ffn_prefill(ctypes.byref(d), ctypes.byref(ex), ctypes.byref(aq),
                                        _ptr(ids), T, _ptr(out), _ptr(ws), ws_bytes,
                                        _debug(dbg), _stream(stream)))


def moe_combine(out, w, residual, T: int, k: int, H: int, y, stream=None):
    _check(lib().moe_combine(_ptr(out), _ptr(w), _ptr(residual), T, k, H, _ptr(y),
                             _stream(stream)))


def moe_rms_norm(x, T: int, H: int, target_rms: float, y, stream=None):
    _check(lib().moe_rms_norm(_ptr(x), T, H, float(target_rms), _ptr(y), _stream(stream)))


MOE_STREAM_READ_MAX_BLOCKS = 2048


def moe_stream_read(src, nbytes: int, sink, stream=None):
    """Measurement helper: one streaming read of nbytes at src (the
    yardstick for a call that reads that many bytes once); sink is a device
    buffer of MOE_STREAM_READ_MAX_BLOCKS uint32 whose contents are not a
    result."""
    _check(lib().moe_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)))


def moe_layer_decode_workspace_bytes(d: moe_dims, T: int) -> int:
    return lib().moe_layer_decode_workspace_bytes(ctypes.byref(d), T)


def moe_layer_decode(d: moe_dims, experts: dict, x, W_r, bias, T: int, add_residual: bool, y,
                     ids, w, ws, ws_bytes: int, stream=None):
    ex = _experts(experts)
    _check(lib().moe_layer_decode(ctypes.byref(d), ctypes.byref(ex), _ptr(x), _ptr(W_r), _ptr(bias),
                                  T, 1 if add_residual else 0, _ptr(y), _ptr(ids), _ptr(w),
                                  _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer_decode_rescaled(d: moe_dims, experts: dict, x_in, target_rms: float, W_r, bias, T: int, y,
                              ids, w, ws, ws_bytes: int, stream=None):
    """One stack layer: input bf16(x_in * target_rms / rms(x_in)), then the
    fused layer with the residual add (moe_rms_norm + moe_layer_decode in one
    call, bit for bit)."""
    ex = _experts(experts)
    _check(lib().moe_layer_decode_rescaled(ctypes.byref(d), ctypes.byref(ex), _ptr(x_in), float(target_rms),
                                           _ptr(W_r), _ptr(bias), T, _ptr(y), _ptr(ids), _ptr(w), _ptr(ws),
                                           ws_bytes, _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 8 << 20


def moe_layer_decode_noalloc(d: moe_dims, experts: dict, x, W_r, bias, T: int, add_residual: bool, y,
                             ids, w, stream=None):
    """moe_layer_decode on the library's per-GPU scratch array (no workspace
    argument; calls that overlap on one GPU race)."""
    ex = _experts(experts)
    _check(lib().moe_layer_decode_noalloc(ctypes.byref(d), ctypes.byref(ex), _ptr(x), _ptr(W_r),
                                          _ptr(bias), T, 1 if add_residual else 0, _ptr(y), _ptr(ids),
                                          _ptr(w), _stream(stream)))


# ------------------------------------------------------------------ preparation

def moe_quantize_weights(W, n_mat: int, rows: int, cols: int, codes, scales, ts, stream=None):
    _check(lib().moe_quantize_weights(_ptr(W), n_mat, rows, cols, _ptr(codes), _ptr(scales),
                                      _ptr(ts), _stream(stream)))


def moe_pack_nvfp4(d: moe_dims, e0: int, n: int, gate_codes, gate_scales, up_codes, up_scales,
                   down_codes, down_scales, gate_up, down, stream=None):
    _check(lib().moe_pack_nvfp4(ctypes.byref(d), e0, n, _ptr(gate_codes), _ptr(gate_scales),
                                _ptr(up_codes), _ptr(up_scales), _ptr(down_codes),
                                _ptr(down_scales), _ptr(gate_up), _ptr(down), _stream(stream)))


def moe_unpack_nvfp4(d: moe_dims, e0: int, n: int, gate_codes, gate_scales, up_codes, up_scales,
                     down_codes, down_scales, gate_up, down, stream=None):
    _check(lib().moe_unpack_nvfp4(ctypes.byref(d), e0, n, _ptr(gate_codes), _ptr(gate_scales),
                                  _ptr(up_codes), _ptr(up_scales), _ptr(down_codes),
                                  _ptr(down_scales), _ptr(gate_up), _ptr(down), _stream(stream)))


def moe_pack_codebook(d: moe_dims, e0: int, n: int, gate_cb, gate_idx, up_cb, up_idx, gate_up,
                      stream=None):
    _check(lib().moe_pack_codebook(ctypes.byref(d), e0, n, _ptr(gate_cb), _ptr(gate_idx),
                                   _ptr(up_cb), _ptr(up_idx), _ptr(gate_up), _stream(stream)))


def moe_permute(ids, T: int, k: int, E: int, counts, offsets, perm, inv, ws, ws_bytes: int,
                stream=None):
    _check(lib().moe_permute(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm),
                             _ptr(inv), _ptr(ws), ws_bytes, _stream(stream)))


def __getattr__(name):
    # Layer (allocation helpers over the ABI) needs torch; the bare C-ABI
    # wrappers above do not, so torch is imported only when Layer is used
    if name == "Layer":
        from .layer import Layer
        return Layer
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
