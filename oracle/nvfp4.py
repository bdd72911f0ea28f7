"""NVFP4 block quantizer and dequantizer (test infrastructure only).

Format (public NVFP4 definition; the pages name it in the release post
"capy-flash v0.7.1", section "What shipped", and say activations run the same
4-bit path, "W4A4", section "Why it matters"):
  value = E2M1(code) * E4M3(block scale) * fp32 tensor scale,
  one block scale per 16 consecutive elements along the contraction axis.

Quantizer Q(v; scope), every step an fp32 IEEE operation rounded to nearest
even, in this order (a reading: the pages name the format, not these steps):
  1. amax = max |v| over the tensor-scale scope (a whole weight matrix, one
     token row of x, one (token, slot) row of h);
  2. ts = amax / 2688   (2688 = 6 * 448, the largest E2M1 times the largest
     E4M3), ts = 0 when amax = 0;
  3. per block: ab = max |v| over the 16 elements; sb = E4M3(ab / (6 * ts))
     with 6 * ts rounded first; sb = 0 when ts = 0;
  4. d = E4M3value(sb) * ts; if d = 0 the block's codes are all 0, otherwise
     code = sign(v) << 3 | E2M1(|v / d|).
With a static (calibrated) tensor scale, as NVIDIA's NVFP4 checkpoints carry
for activations (the engine was built for that quantisation: forum repost,
paragraph "What it's for"), ts is given per row and steps 1-2 are skipped; values
beyond 6 * 448 * ts saturate to the largest code and block scale.
The sign bit is kept even when the magnitude rounds to 0 (so a small negative
value encodes as 0x8).
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_decode, e2m1_encode_magnitude, e4m3_decode, e4m3_encode_nonneg

BLOCK = 16
TS_DIVISOR = np.float32(2688.0)   # 6 * 448


def quantize(v, per_row: bool, ts_given=None):
    """Quantize a 2-D fp32 array v [R, K] (K a multiple of 16).

    per_row=True : one tensor scale per row (activation rows).
    per_row=False: one tensor scale for the whole array (a weight matrix).
    ts_given     : per-row static tensor scales [R] (per_row only): used
                   as ts instead of amax / 2688.

    Returns (codes uint8 [R, K] unpacked 0..15, scales uint8 [R, K/16],
    ts float32 [R] (per_row) or float32 scalar).
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    R, K = v.shape
    assert K % BLOCK == 0
    a = np.abs(v)
    if per_row:
        amax = a.max(axis=1) if K else np.zeros(R, np.float32)
    else:
        amax = np.float32(a.max()) if a.size else np.float32(0)
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        if ts_given is not None:
            assert per_row
            ts = np.ascontiguousarray(ts_given, dtype=np.float32).reshape(R)
        else:
            ts = np.where(amax == 0, np.float32(0), amax / TS_DIVISOR).astype(np.float32)
        ts_rows = np.broadcast_to(ts, (R,)) if not per_row else ts
        six_ts = (np.float32(6.0) * ts_rows).astype(np.float32)
        blocks = v.reshape(R, K // BLOCK, BLOCK)
        ab = np.abs(blocks).max(axis=2)                                 # fp32
        ratio = (ab / six_ts[:, None]).astype(np.float32)
        sb = np.where(ts_rows[:, None] == 0, 0, e4m3_encode_nonneg(ratio))
        d = (e4m3_decode(sb).astype(np.float32) * ts_rows[:, None]).astype(np.float32)
        q = (blocks / d[:, :, None]).astype(np.float32)
        mag = e2m1_encode_magnitude(np.abs(q))
    sign = np.signbit(blocks).astype(np.int64)
    codes = np.where(d[:, :, None] == 0, 0, (sign << 3) | mag)
    codes = codes.reshape(R, K).astype(np.uint8)
    return codes, sb.astype(np.uint8), (ts if per_row else np.float32(ts))


def dequantize(codes, scales, ts) -> np.ndarray:
    """fp64 values of unpacked codes [R, K], scales [R, K/16] and a tensor scale
    (scalar, or one per row).  Exact: E2M1 * E4M3 has at most 6 significant
    bits and times an fp32 scale at most 30, well inside fp64."""
    codes = np.asarray(codes)
    R, K = codes.shape
    e = e2m1_decode(codes).reshape(R, K // BLOCK, BLOCK)
    s = e4m3_decode(scales)[:, :, None]
    ts = np.asarray(ts, dtype=np.float64)
    ts = ts.reshape(-1, 1, 1) if ts.ndim else ts
    return (e * s * ts).reshape(R, K)


def pack_nibbles(codes) -> np.ndarray:
    """[R, K] codes -> [R, K/2] bytes, element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def expert_bytes(H: int, I: int) -> int:
    """Bytes of one expert's NVFP4 gate, up and down codes plus block scales
    (tensor scales excluded): 3*H*I*(1/2 + 1/16)."""
    return 3 * H * I // 2 + 3 * H * I // BLOCK
