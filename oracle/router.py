"""Softmax top-k router (test infrastructure only).

Each token runs only some of the experts (blog "Capy Flash ... two consumer
GPUs", section "Where the experts live"), and the engine computes all of the
experts the model picks, in rank order (forum repost, paragraph "Where it
stands").  The router computed here: fp32-exact logits of
the unquantized bf16 activations against fp32 router weights (plus an optional
per-expert bias), softmax over all experts, keep the k largest, renormalise.
Renormalising the top-k of a softmax is the softmax over the k selected
logits, which is what is evaluated.

Order and ties (reading): ids come out by descending logit; exactly equal
logits go to the lower expert id.  A token is a near-tie when the gap between
the k-th and (k+1)-th logit is below tau = 1e-4 * max(1, max_e |l_e|); for
such a token any experts within tau of the k-th logit may be exchanged, and
downstream stages are then compared on the device's own ids.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64

NEAR_TIE_REL = 1e-4


def logits(x_bf16_bits, W_r, bias=None) -> np.ndarray:
    """fp64 [T, E] = x . W_r^T (+ bias), x given as bf16 bits [T, H]."""
    x = bf16_bits_to_f64(x_bf16_bits)
    l = x @ np.asarray(W_r, dtype=np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def topk(l, k: int):
    """ids int32 [T, k] (descending logit, ties to lower id), weights fp64
    [T, k] (softmax over the selected logits), near_tie bool [T], tau [T]."""
    l = np.asarray(l, dtype=np.float64)
    T, E = l.shape
    e_idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((e_idx, -l), axis=1)          # primary -l, then e
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l, ids, axis=1)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    tau = NEAR_TIE_REL * np.maximum(1.0, np.abs(l).max(axis=1))
    if k < E:
        nxt = np.take_along_axis(l, order[:, k:k + 1], axis=1)[:, 0]
        near = (sel[:, -1] - nxt) < tau
    else:
        near = np.zeros(T, dtype=bool)
    return ids, w, near, tau


def route(x_bf16_bits, W_r, k: int, bias=None):
    """Convenience: logits then top-k.  Returns (ids, w, near_tie, tau, logits)."""
    l = logits(x_bf16_bits, W_r, bias)
    ids, w, near, tau = topk(l, k)
    return ids, w, near, tau, l
