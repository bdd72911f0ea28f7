"""Pins for oracle.codebook: lookups, 3-bit packing, degenerate codebooks."""
import numpy as np

import synth
from oracle import codebook


def test_dequant_is_table_lookup():
    wl = synth.WORKLOADS["tiny"]
    cb, idx = synth.codebook_weights(wl, 0, 1, synth.PROJ_GATE)
    W = codebook.dequantize(cb, idx)
    for (n, kk) in [(0, 0), (5, 127), (5, 128), (127, 255), (64, 200)]:
        assert W[n, kk] == float(cb[n, kk // 128, idx[n, kk]])
    # codebooks are sorted and fp16
    assert np.all(np.diff(cb.astype(np.float32), axis=-1) >= 0)


def test_constant_codebook_gives_constant_weights():
    cb = np.full((4, 2, 8), np.float16(0.0123), np.float16)
    idx = np.random.default_rng(1).integers(0, 8, (4, 256)).astype(np.uint8)
    W = codebook.dequantize(cb, idx)
    assert np.all(W == float(np.float16(0.0123)))


def test_pack_round_trip_and_bit_order():
    idx = np.random.default_rng(2).integers(0, 8, (3, 256)).astype(np.uint8)
    p = codebook.pack_indices(idx)
    assert p.shape == (3, 2, 48)
    assert np.array_equal(codebook.unpack_indices(p), idx)
    one = np.zeros((1, 128), np.uint8)
    one[0, 0] = 5           # bits 0..2 = 101
    one[0, 3] = 7           # bits 9..11
    p = codebook.pack_indices(one)[0, 0]
    assert p[0] == 0x05 and p[1] == 0x0E and not p[2:].any()


def test_sizes():
    assert codebook.expert_bytes_cb(2560, 640) == 2_560_000
