"""3-bit group-128 fp16-codebook weights (test infrastructure only).

The release post ("capy-flash v0.7.1", section "What shipped") names 3-bit GSQ
weights with q3_g128_fp16 codebooks.  Format as read here: a group is 128
consecutive elements of a gate or up row along the contraction axis; the group
has its own 8-entry fp16 codebook; each weight stores a 3-bit index and its
value is codebook[index] (exact in fp16).  Plain storage packs a group's 128
indices least-significant-bit first into 48 bytes: index j occupies bits
3j .. 3j+2 of the group's little-endian 384-bit string.
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np

GROUP = 128


class CBMatrix(NamedTuple):
    codebooks: np.ndarray   # fp16 [N, K/128, 8]
    indices: np.ndarray     # uint8 [N, K] in 0..7

    def dequantize(self) -> np.ndarray:
        return dequantize(self.codebooks, self.indices)


def dequantize(codebooks, indices) -> np.ndarray:
    """fp64 [N, K]: each weight is its group's codebook entry."""
    cb = np.asarray(codebooks, dtype=np.float16).astype(np.float64)
    idx = np.asarray(indices).astype(np.int64)
    N, K = idx.shape
    g = np.arange(K) // GROUP
    return cb[np.arange(N)[:, None], g[None, :], idx]


def pack_indices(indices) -> np.ndarray:
    """[N, K] indices -> [N, K/128, 48] bytes (3 bits each, LSB first)."""
    idx = np.asarray(indices, dtype=np.uint8)
    N, K = idx.shape
    bits = np.zeros((N, K // GROUP, GROUP * 3), dtype=np.uint8)
    grp = idx.reshape(N, K // GROUP, GROUP)
    for b in range(3):
        bits[:, :, b::3] = (grp >> b) & 1
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_indices(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    N, G, _ = p.shape
    bits = np.unpackbits(p, axis=-1, bitorder="little")        # [N, G, 384]
    idx = bits[:, :, 0::3] | (bits[:, :, 1::3] << 1) | (bits[:, :, 2::3] << 2)
    return idx.reshape(N, G * GROUP).astype(np.uint8)


def expert_bytes_cb(H: int, I: int) -> int:
    """Bytes of one expert with codebook gate/up (64 B per 128-group: 16 B of
    fp16 codebook + 48 B of indices) and NVFP4 down."""
    gate_up = 2 * I * (H // GROUP) * 64
    down = H * I // 2 + H * I // 16
    return gate_up + down
