"""Pins for oracle.ffn on the tiny layer (H256 I128 E16 k2 T4): exact brute
force for every expert densely, then the top-k mask; plus closed forms."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import ffn, nvfp4, router
from tests import brute


@pytest.fixture(scope="module")
def tiny():
    wl = synth.WORKLOADS["tiny"]
    x = synth.activations(wl)
    W_r = synth.router_weights(wl)
    experts = {e: ffn.quantize_expert(*synth.expert_weights(wl, 0, e)) for e in range(wl.E)}
    out = ffn.layer(x, W_r, None, experts, wl.k)
    return wl, x, W_r, experts, out


def test_activation_quant_matches_brute(tiny):
    wl, x, _, _, out = tiny
    bc, bs, bts = brute.quantize_rows(synth.bf16_bits_to_f32(x), per_row=True)
    c, s, ts = out["xq"]
    assert np.array_equal(c, bc) and np.array_equal(s, bs)
    assert [float(v) for v in ts] == [float(v) for v in bts]


def test_dense_layer_exact_brute_force(tiny):
    wl, x, _, experts, out = tiny
    xc, xs, xts = out["xq"]
    T, k, E, I, H = wl.T, wl.k, wl.E, wl.I, wl.H
    ids, w = out["ids"], out["w"]
    # exact g, u for every (token, expert): dense over all experts
    h_exact = {}
    for e in range(E):
        q = experts[e]
        G = brute.exact_matvec(q.gate.codes, q.gate.scales, float(q.gate.ts), xc, xs, xts)
        U = brute.exact_matvec(q.up.codes, q.up.scales, float(q.up.ts), xc, xs, xts)
        for t in range(T):
            h_exact[(t, e)] = [brute.round_f32(brute.dec_to_fraction(brute.silu_exact(g)) * u)
                               for g, u in zip(G[t], U[t])]
    # the oracle's h at the picked experts is the correctly rounded fp32 h,
    # up to one fp32 ulp (the oracle rounds SiLU(g)*u through fp64)
    h = out["h"]
    for t in range(T):
        for i in range(k):
            ref = np.array([float(v) for v in h_exact[(t, int(ids[t, i]))]], np.float32)
            got = h[t, i]
            ulp = np.spacing(np.maximum(np.abs(ref), np.float32(1e-38)))
            assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)
    # re-quantized h: brute quantizer on the oracle's own h
    hc, hs, hts = out["hq"]
    bc, bs, bts = brute.quantize_rows(h.reshape(T * k, I), per_row=True)
    assert np.array_equal(hc, bc) and np.array_equal(hs, bs)
    assert [float(v) for v in hts] == [float(v) for v in bts]
    # exact down projection for every expert, masked to the picked ones
    o = out["o"]
    for e in range(E):
        q = experts[e]
        O = brute.exact_matvec(q.down.codes, q.down.scales, float(q.down.ts), hc, hs, bts)
        for t in range(T):
            for i in range(k):
                if int(ids[t, i]) != e:
                    continue
                ref = np.array([float(v) for v in O[t * k + i]])
                np.testing.assert_allclose(o[t, i], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # combine
    y_ref = np.einsum("tk,tkh->th", w, o)
    np.testing.assert_allclose(out["y"], y_ref, rtol=1e-14, atol=1e-15)


def test_zero_input_gives_residual():
    wl = synth.WORKLOADS["tiny"]
    x = np.zeros((2, wl.H), np.uint16)
    W_r = synth.router_weights(wl)
    experts = {e: ffn.quantize_expert(*synth.expert_weights(wl, 0, e)) for e in range(wl.E)}
    out = ffn.layer(x, W_r, None, experts, wl.k, residual=True)
    assert np.all(out["y"] == 0) and np.all(out["o"] == 0)
    # with a nonzero residual and zero expert input, y = r exactly
    r = synth.activations(wl, T=2)
    xq = ffn.quantize_act(x)
    deq = {e: ffn.dequant_expert(experts[e]) for e in range(wl.E)}
    ids = np.array([[0, 1], [2, 3]], np.int32)
    h = ffn.gate_up(deq, xq, ids)
    o = ffn.down(deq, ffn.quantize_h(h), ids)
    y = ffn.combine(o, np.full((2, 2), 0.5), r)
    np.testing.assert_array_equal(y, synth.bf16_bits_to_f32(r).astype(np.float64))
    np.testing.assert_array_equal(ffn.to_bf16(y), r)


def test_zero_up_gives_zero_h():
    wl = synth.WORKLOADS["tiny"]
    g, u, d = synth.expert_weights(wl, 0, 0)
    q = ffn.quantize_expert(g, np.zeros_like(u), d)
    x = synth.activations(wl)
    deq = {0: ffn.dequant_expert(q)}
    h = ffn.gate_up(deq, ffn.quantize_act(x), np.zeros((wl.T, 1), np.int32))
    assert np.all(h == 0)


def test_silu_closed_form():
    z = np.array([0.0, 1.0, -1.0, 20.0, -800.0])
    s = ffn.silu(z)
    np.testing.assert_allclose(s[:4], z[:4] * (1 / (1 + np.exp(-z[:4]))), rtol=1e-15)
    assert s[0] == 0 and s[4] == 0


def test_layer_combines_in_fp64_and_rounds_once():
    wl = synth.WORKLOADS["tiny"]
    r = np.random.default_rng(7)
    o = r.standard_normal((3, 2, wl.H))
    w = np.array([[0.75, 0.25]] * 3)
    y = ffn.combine(o, w)
    np.testing.assert_allclose(y, 0.75 * o[:, 0] + 0.25 * o[:, 1], rtol=1e-15)
    b = ffn.to_bf16(y)
    back = synth.bf16_bits_to_f32(b).astype(np.float64)
    assert np.all(np.abs(back - y) <= np.abs(y) * 2.0 ** -8)
