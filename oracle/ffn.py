"""Routed-expert SwiGLU FFN on W4A4 NVFP4 operands, and the weighted combine
(test infrastructure only).

The pages: each routed expert has gate/up weights and a down projection
(release post "capy-flash v0.7.1", section "What shipped"); expert math runs
on a W4A4 path and tensor-parallel partial sums are exchanged in FP32
(section "Why it matters").  Per (token t, slot i) with expert e = ids[t, i]:

  x^     = Q(x_t)              NVFP4, one tensor scale per token row
  g, u   = W^_gate[e] x^, W^_up[e] x^
  h      = SiLU(g) * u,  SiLU(z) = z / (1 + exp(-z))   (fp64, then fp32)
  h^     = Q(h)                NVFP4, one tensor scale per (t, i) row
  o[t,i] = W^_down[e] h^       (kept in fp64 here; fp32 on the device)

  y[t]   = r[t] + sum_i w[t,i] o[t,i], rounded once to bf16 (r = residual or 0)

Every product of two dequantized NVFP4 values is exact in fp64; the matmuls
are fp64 (BLAS), so the results are the exact quantized computation up to fp64
rounding order.  Stages are exposed separately so that a comparison can feed
the device's own ids and h into the next stage.
"""
from __future__ import annotations

from typing import Dict, NamedTuple, Optional

import numpy as np

from . import nvfp4
from .formats import bf16_bits_to_f64, f64_to_bf16_bits


class QMatrix(NamedTuple):
    codes: np.ndarray    # uint8 [N, K] unpacked 0..15
    scales: np.ndarray   # uint8 [N, K/16] E4M3
    ts: np.float32       # tensor scale


class QExpert(NamedTuple):
    gate: object         # QMatrix, or codebook.CBMatrix
    up: object
    down: QMatrix


def quantize_matrix(W) -> QMatrix:
    c, s, ts = nvfp4.quantize(W, per_row=False)
    return QMatrix(c, s, np.float32(ts))


def quantize_expert(gate, up, down) -> QExpert:
    return QExpert(quantize_matrix(gate), quantize_matrix(up), quantize_matrix(down))


def dequant_matrix(m) -> np.ndarray:
    if isinstance(m, QMatrix):
        return nvfp4.dequantize(m.codes, m.scales, m.ts)
    return m.dequantize()     # codebook matrix


def dequant_expert(q: QExpert):
    return dequant_matrix(q.gate), dequant_matrix(q.up), dequant_matrix(q.down)


def quantize_act(x_bf16_bits):
    """x^ = Q(x), one tensor scale per token: (codes [T,H], scales, ts [T])."""
    x = bf16_bits_to_f64(x_bf16_bits).astype(np.float32)
    return nvfp4.quantize(x, per_row=True)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def _groups(ids):
    """(expert, flat (t*k+slot) indices) for each expert present, ascending."""
    flat = np.asarray(ids).reshape(-1)
    for e in np.unique(flat):
        yield int(e), np.nonzero(flat == e)[0]


def gate_up(deq: Dict[int, tuple], xq, ids) -> np.ndarray:
    """h fp32 [T, k, I].  deq maps expert -> (Wg, Wu, Wd) fp64; xq from
    quantize_act."""
    ids = np.asarray(ids)
    T, k = ids.shape
    xd = nvfp4.dequantize(*xq)                         # [T, H] fp64
    I = next(iter(deq.values()))[0].shape[0]
    h = np.zeros((T * k, I), dtype=np.float64)
    for e, rows in _groups(ids):
        Wg, Wu, _ = deq[e]
        xs = xd[rows // k]                              # [n, H]
        g = xs @ Wg.T
        u = xs @ Wu.T
        h[rows] = silu(g) * u
    return h.astype(np.float32).reshape(T, k, I)


def quantize_h(h, ts_rows=None):
    """h^ = Q(h), one tensor scale per (t, slot) row: codes [T*k, I], ...
    ts_rows: static tensor scales per row (the row's expert's calibrated h
    scale), or None for the row's own amax / 2688."""
    h = np.asarray(h, dtype=np.float32)
    return nvfp4.quantize(h.reshape(-1, h.shape[-1]), per_row=True, ts_given=ts_rows)


def down(deq: Dict[int, tuple], hq, ids) -> np.ndarray:
    """o fp64 [T, k, H] from h^ (codes [T*k, I], scales, ts [T*k])."""
    ids = np.asarray(ids)
    T, k = ids.shape
    hd = nvfp4.dequantize(*hq)                          # [T*k, I]
    H = next(iter(deq.values()))[2].shape[0]
    o = np.zeros((T * k, H), dtype=np.float64)
    for e, rows in _groups(ids):
        Wd = deq[e][2]
        o[rows] = hd[rows] @ Wd.T
    return o.reshape(T, k, H)


def combine(o, w, residual_bits: Optional[np.ndarray] = None) -> np.ndarray:
    """y* fp64 [T, H] = r + sum_i w_i o_i (unrounded)."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = np.einsum("tk,tkh->th", w, o)
    if residual_bits is not None:
        y = y + bf16_bits_to_f64(residual_bits)
    return y


def to_bf16(y) -> np.ndarray:
    return f64_to_bf16_bits(y)


def layer(x_bf16_bits, W_r, bias, experts: Dict[int, QExpert], k: int,
          residual: bool = False, h_ts=None):
    """The whole layer with the oracle's own ids and h (no teacher forcing).
    `experts` must hold every expert the router can pick for these tokens.
    h_ts: static h tensor scale per expert ([E]) or None (per-row amax).
    Returns a dict of every stage."""
    from . import router
    ids, w, near, tau, l = router.route(x_bf16_bits, W_r, k, bias)
    xq = quantize_act(x_bf16_bits)
    deq = {e: dequant_expert(experts[e]) for e in np.unique(ids)}
    h = gate_up(deq, xq, ids)
    hq = quantize_h(h, None if h_ts is None else np.asarray(h_ts, np.float32)[ids].reshape(-1))
    o = down(deq, hq, ids)
    y = combine(o, w, x_bf16_bits if residual else None)
    return dict(ids=ids, w=w, near=near, tau=tau, logits=l, xq=xq, h=h, hq=hq,
                o=o, y=y, y_bf16=to_bf16(y))
