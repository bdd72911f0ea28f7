"""Pins for oracle.router: exact brute force, closed forms and invariants."""
import decimal
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import router
from tests import brute


def test_router_matches_exact_brute_force_tiny():
    wl = synth.WORKLOADS["tiny"]
    x = synth.activations(wl)
    W = synth.router_weights(wl)
    ids, w, near, tau, l = router.route(x, W, wl.k)
    xf = synth.bf16_bits_to_f32(x)
    for t in range(wl.T):
        xs = [Fraction(float(v)) for v in xf[t]]
        exact = [sum(a * Fraction(float(b)) for a, b in zip(xs, W[e])) for e in range(wl.E)]
        for e in range(wl.E):
            assert abs(Fraction(float(l[t, e])) - exact[e]) <= abs(exact[e]) * Fraction(1, 10**12) + Fraction(1, 10**14)
        order = sorted(range(wl.E), key=lambda e: (-exact[e], e))
        assert list(ids[t]) == order[:wl.k]
        # softmax over the selected logits, 60 digits
        sel = [brute.dec(exact[e]) for e in order[:wl.k]]
        z = [brute._CTX.exp(s - sel[0]) for s in sel]
        tot = sum(z, decimal.Decimal(0))
        for i in range(wl.k):
            assert abs(float(z[i] / tot) - w[t, i]) < 1e-13


def test_renormalised_topk_equals_full_softmax_restricted():
    r = np.random.default_rng(21)
    l = r.standard_normal((50, 512)) * 3
    ids, w, _, _ = router.topk(l, 10)
    full = np.exp(l - l.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, ids, 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    # the selected are the k largest of the full softmax
    thr = np.sort(full, 1)[:, -10]
    assert np.all(sel >= thr[:, None])


def test_weights_sum_to_one_and_descend():
    r = np.random.default_rng(22)
    l = r.standard_normal((100, 64))
    ids, w, _, _ = router.topk(l, 7)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)
    sel = np.take_along_axis(l, ids, 1)
    assert np.all(np.diff(sel, axis=1) <= 0)


def test_k1_weight_exactly_one():
    l = np.random.default_rng(23).standard_normal((20, 16))
    ids, w, _, _ = router.topk(l, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], l.argmax(1))


def test_constant_logits_ties_to_lower_ids():
    l = np.full((3, 32), 0.25)
    ids, w, near, _ = router.topk(l, 5)
    assert np.array_equal(ids, np.tile(np.arange(5), (3, 1)))
    np.testing.assert_allclose(w, 0.2, rtol=1e-15)
    assert np.all(near)                       # gap 0 < tau


def test_permutation_equivariance():
    r = np.random.default_rng(24)
    x = synth.f32_to_bf16_bits(r.standard_normal((6, 64)).astype(np.float32))
    W = (r.standard_normal((32, 64)) * 0.1).astype(np.float32)
    ids, w, _, _, _ = router.route(x, W, 4)
    p = r.permutation(32)                     # new expert j is old expert p[j]
    ids2, w2, _, _, _ = router.route(x, W[p], 4)
    np.testing.assert_array_equal(p[ids2], ids)
    np.testing.assert_allclose(w2, w, rtol=1e-12)


def test_bias_shifts_logits():
    wl = synth.WORKLOADS["prefill8k"].with_(T=4, H=64, E=32)
    x = synth.activations(wl)
    W = synth.router_weights(wl)
    b = synth.router_bias(wl)
    l0 = router.logits(x, W)
    l1 = router.logits(x, W, b)
    np.testing.assert_allclose(l1 - l0, np.broadcast_to(b.astype(np.float64), l0.shape), atol=1e-12)


def test_near_tie_flag():
    l = np.zeros((2, 8))
    l[0, :4] = [5, 4, 3, 2]
    l[0, 4] = 2 - 0.5e-4              # gap 5e-5 < tau = 1e-4 * 5
    l[1, :4] = [5, 4, 3, 2]
    l[1, 4] = 2 - 1e-3               # gap 1e-3 > 5e-4
    _, _, near, tau = router.topk(l, 4)
    assert list(near) == [True, False]
    np.testing.assert_allclose(tau, 5e-4)
