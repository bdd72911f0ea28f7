"""Glue of the full-depth decode stack (test infrastructure only).

The 48-layer workload stacks the Flash-Next layer with a residual add
between layers and asks for near-uniform routing at every layer.  The pages
do not describe what sits between two MoE layers; with random N(0, 0.02)
experts and no normalisation the residual stream grows until the routing is
one-hot and bf16 overflows, so each layer's output is brought back to the
first layer's input RMS before the next layer (the "Add & Norm" of a
post-norm transformer block, without a learned gain):

  x_{l+1}[t, :] = y_l[t, :] * target / sqrt(mean_h y_l[t, h]^2),
  y_l = layer_l(x_l) with the residual add, a zero row stays zero.

Exact in fp64 here; the result before the one bf16 rounding is returned.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64


def rms_norm(x_bf16_bits: np.ndarray, target_rms: float) -> np.ndarray:
    """[T, H] bf16 bits -> fp64 [T, H]: x * target / sqrt(mean(x^2)) per row."""
    x = bf16_bits_to_f64(np.asarray(x_bf16_bits, np.uint16))
    ms = np.mean(x * x, axis=-1, keepdims=True)
    s = np.where(ms > 0, target_rms / np.sqrt(np.where(ms > 0, ms, 1.0)), 0.0)
    return x * s
