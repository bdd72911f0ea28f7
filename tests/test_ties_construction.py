"""The tie inputs of the device quantizer tests really sit on exact ties
(counted with the oracle's own scales), and the oracle resolves them to the
even code (CPU; the GPU tests then compare the device with the oracle)."""
import numpy as np

import synth
from oracle import ffn as offn, nvfp4
from tests import brute, ties


def test_act_tie_rows_hit_ties():
    v = ties.act_tie_rows(20, 512, seed=31)
    xbits = synth.f32_to_bf16_bits(v)
    assert np.array_equal(synth.bf16_bits_to_f32(xbits), v)          # bf16-exact
    c, s, ts = offn.quantize_act(xbits)
    el, sc = ties.count_ties(v, s, ts)
    assert el >= 1000 and sc >= 40, (el, sc)
    # tensor scales are not powers of two
    assert np.all(np.frexp(ts)[0] != 0.5)
    bc, bs, _ = brute.quantize_rows(v[:3], per_row=True)
    assert np.array_equal(c[:3], bc) and np.array_equal(s[:3], bs)


def test_act_tie_rows_resolve_to_even():
    """Every exact element tie takes the even E2M1 code of the two."""
    v = ties.act_tie_rows(10, 256, seed=32)
    c, s, ts = offn.quantize_act(synth.f32_to_bf16_bits(v))
    vals = ties.e4m3_values()
    d = (vals[s].astype(np.float32) * ts[:, None].astype(np.float32)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.abs(v.reshape(v.shape[0], -1, 16).astype(np.float64)) / d[:, :, None]
    mag = (c.reshape(q.shape) & 7)
    even = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    n = 0
    for m, code in even.items():
        sel = q == m
        n += sel.sum()
        assert np.all(mag[sel] == code), m
    assert n > 100


def test_weight_tie_matrix_hits_ties():
    W = ties.weight_tie_matrix(48, 256, seed=33)
    c, s, ts = nvfp4.quantize(W, per_row=False)
    el, sc = ties.count_ties(W, s, ts)
    assert el >= 3000 and sc >= 200, (el, sc)
    assert np.frexp(ts)[0] != 0.5
    # the first rows hold the matrix amax, so their tensor scale is the matrix's
    bc, bs, _ = brute.quantize_rows(W[:4], per_row=False)
    assert np.array_equal(c[:4], bc) and np.array_equal(s[:4], bs)


def test_tie_layer_h_is_exact_and_tied():
    """The oracle's h on the tie layer is 64 N exactly; its h^ has exact
    element ties (dynamic ts = 3) and scale-ratio ties (static ts = 6)."""
    H, I, E = 256, 128, 4
    for mode, ts_given in (("dynamic", None), ("static", 6.0)):
        N = ties.h_pattern(I, mode, seed=5)
        gate, up, down, xrow = ties.tie_layer(H, I, E, N, seed=6)
        xbits = synth.f32_to_bf16_bits(xrow[None])
        assert np.array_equal(synth.bf16_bits_to_f32(xbits)[0], xrow)
        q = offn.quantize_expert(gate[1], up[1], down[1])
        deq = {1: offn.dequant_expert(q)}
        h = offn.gate_up(deq, offn.quantize_act(xbits), np.array([[1]]))[0]
        assert np.array_equal(h[0], (64 * N).astype(np.float32))
        ts_rows = None if ts_given is None else np.array([ts_given], np.float32)
        hc, hs, hts = offn.quantize_h(h, ts_rows)
        assert hts[0] == (3.0 if ts_given is None else 6.0)
        el, sc = ties.count_ties(h, hs, hts)
        assert el >= 40, (mode, el)
        if mode == "static":
            assert sc >= 2, sc
            # the two scale-ratio ties: 272 -> 256 (0x78), 304 -> 320 (0x7A)
            blocks = np.abs(N.reshape(-1, 16)).max(1)
            assert set(hs[0][blocks == 153]) <= {0x78} and set(hs[0][blocks == 171]) <= {0x7A}
