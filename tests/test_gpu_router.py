"""GPU parity: router (fp32 logits, top-k ids, renormalised weights)."""
import numpy as np
import pytest
import torch

import synth
import quantized_moe_routed_router_amd as moe
from oracle import router as orouter
from tests.gpu_helpers import say, t2n, bf16_tensor

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_router(xbits, W, bias, k):
    T, H = xbits.shape
    E = W.shape[0]
    d = moe.dims(E, H, 128, k)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    moe.moe_router_topk(bf16_tensor(xbits, DEV), torch.from_numpy(W).to(DEV),
                        None if bias is None else torch.from_numpy(bias).to(DEV), T, d, ids, w, logits)
    torch.cuda.synchronize()
    return t2n(ids), t2n(w), t2n(logits)


def check_router(xbits, W, bias, k):
    ids, w, l = run_router(xbits, W, bias, k)
    oids, ow, near, tau, ol = orouter.route(xbits, W, k, bias)
    T = xbits.shape[0]
    # logits within tau/4 of the fp64 logits
    assert np.all(np.abs(l - ol) <= tau[:, None] / 4), np.abs(l - ol).max()
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    ok = 0
    for t in range(T):
        if near[t]:
            # exchanged ids allowed only among logits within tau of the k-th
            kth = np.sort(ol[t])[::-1][k - 1]
            diff = set(ids[t]) ^ set(oids[t])
            assert all(abs(ol[t, e] - kth) < tau[t] for e in diff)
            continue
        assert list(ids[t]) == list(oids[t]) or set(ids[t]) == set(oids[t]), t
        ow_by_id = dict(zip(oids[t], ow[t]))
        for e, wv in zip(ids[t], w[t]):
            assert abs(wv - ow_by_id[e]) <= 1e-5
        ok += 1
    # tau flags ~1% of tokens at these scales; most must be fully comparable
    assert ok >= max(1, int(0.8 * T)), (ok, T)
    return ok


@pytest.mark.parametrize("name,T", [("tiny", 4), ("decode", 1), ("decode_b8", 8), ("decode", 16),
                                    ("decode", 17), ("decode", 200), ("decode", 1100), ("decode", 1300), ("decode", 2600),
                                    ("decode", 4000), ("decode", 16400), ("decode", 18332)])
def test_router_parity(name, T):
    """Every router kernel: GEMV (T <= 16), split-K tiles (<= 1280), 128-token
    x 64-expert tiles (< 16384) and 256-token tiles; 4000 and 18332 tokens
    give tile counts divisible by eight (the XCD-grouped block order) with a
    ragged last tile, 1300, 2600 and 16400 the plain order."""
    say("router", name, T)
    wl = synth.WORKLOADS[name]
    x = synth.activations(wl, T=T, stream=3)
    W = synth.router_weights(wl)
    assert check_router(x, W, synth.router_bias(wl), wl.k) > 0


def test_router_ragged_tiles():
    """Token and expert counts off the tiles of every router kernel (16 x 16
    up to 128 tokens, 32 x 32 up to 1280, 128 x 64 up to 16383, 256 x 128
    above; 50 experts: less than one expert tile), with a bias."""
    r = np.random.default_rng(4)
    H, E, k = 384, 50, 3
    W = (r.standard_normal((E, H)) * 0.05).astype(np.float32)
    bias = (r.standard_normal(E) * 0.01).astype(np.float32)
    for T in (45, 1030, 2600, 16400):
        say("router ragged", T)
        x = synth.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
        check_router(x, W, bias, k)


def test_router_zipf_bias():
    say("router zipf")
    wl = synth.WORKLOADS["prefill8k"]
    x = synth.activations(wl, T=256, stream=1)
    check_router(x, synth.router_weights(wl), synth.router_bias(wl), wl.k)


def test_router_k1_and_ties():
    say("router k=1 and ties")
    r = np.random.default_rng(3)
    H, E = 256, 64
    x = synth.f32_to_bf16_bits(r.standard_normal((5, H)).astype(np.float32))
    W = (r.standard_normal((E, H)) * 0.05).astype(np.float32)
    ids, w, _ = run_router(x, W, None, 1)
    assert np.all(w == 1.0)
    oids, _, _, _, _ = orouter.route(x, W, 1)
    assert np.array_equal(ids, oids)
    # identical router rows -> exactly equal logits -> lower ids win, w = 1/k
    W2 = np.tile(W[:1], (E, 1))
    ids, w, _ = run_router(x, W2, None, 4)
    assert np.array_equal(ids, np.tile(np.arange(4), (5, 1)))
    assert np.allclose(w, 0.25, atol=1e-7)
