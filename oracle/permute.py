"""Token-by-expert counting sort (test infrastructure only).

Groups the (token, slot) pairs of a batch by expert so each expert's weights
are read once per batch; the pages' engine computes "every expert the model
picks" for every token (forum repost, paragraph "Where it stands").

Definitions: with flat index i = t*k + slot and id[i] the expert of that pair,
  counts[e]  = #{i : id[i] = e}
  offsets    = exclusive prefix sum of counts (length E + 1)
  perm[j]    = the i at sorted position j, sorted by (expert, i) (stable)
  inv[i]     = j such that perm[j] = i
"""
from __future__ import annotations

import numpy as np


def permute(ids, E: int):
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return counts, offsets, perm, inv
