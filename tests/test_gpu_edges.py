"""GPU parity at the routing extremes and on empty batches.

k = 1: one expert per token (the renormalised weight is exactly 1).
k = E = 16: every expert for every token (the weights are the full softmax;
one token then has 16 pairs, the most the one-token down kernel serves in a
block, and three tokens take the many-pair down path).  Each runs through
the decode FFN, the prefill grouped GEMM and the fused decode layer, stage
by stage against the oracle.  T = 0 calls enqueue nothing."""
import numpy as np
import pytest
import torch

import synth
import quantized_moe_routed_router_amd as moe
from oracle import router as orouter
from tests.gpu_helpers import say, t2n, bf16_tensor, case, run_layer, check_stages, check_fused_against_separate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("name", ["tiny_k1", "tiny_all"])
@pytest.mark.parametrize("T", [1, 3])
def test_routing_extremes_all_paths(name, T):
    c = case(name, "host")
    wl = c.wl
    x = synth.activations(wl, T=T, stream=30 + T)
    dec = run_layer(c, x, residual=True)
    oids, ow, near, _, _ = orouter.route(x, c.W_r, wl.k)
    for t in range(T):
        if wl.k == wl.E:
            assert sorted(dec["ids"][t]) == list(range(wl.E))
        elif not near[t]:
            assert set(dec["ids"][t]) == set(oids[t])
        assert abs(float(dec["w"][t].astype(np.float64).sum()) - 1.0) <= 1e-6
        np.testing.assert_allclose(dec["w"][t].astype(np.float64), ow[t], atol=1e-5)
    if wl.k == 1:
        assert np.all(dec["w"] == 1.0)
    r_dec = check_stages(c, x, dec, residual=True)
    pre = run_layer(c, x, residual=True, prefill=True)
    assert np.array_equal(pre["ids"], dec["ids"])
    r_pre = check_stages(c, x, pre, residual=True)
    # the fused layer computes the same as the separate entry points
    fb = c.L.alloc_fused(T)
    c.L.forward_fused(bf16_tensor(x, DEV), fb, residual=True)
    torch.cuda.synchronize()
    f = {k: t2n(v) for k, v in fb.items() if isinstance(v, torch.Tensor) and k != "ws"}
    check_fused_against_separate(f, dec, x, True, (name, T))
    say(name, T, "decode", r_dec, "prefill", r_pre)


def test_empty_batch_enqueues_nothing():
    c = case("tiny", "host")
    L = c.L
    b = L.alloc(1, prefill=False)
    for key in ("ids", "w", "logits", "x_codes", "x_scales", "x_ts", "out", "y"):
        b[key].fill_(7)
    before = {k: t2n(v).copy() for k, v in b.items() if isinstance(v, torch.Tensor) and k != "ws"}
    x = bf16_tensor(synth.activations(c.wl, T=1), DEV)
    moe.moe_router_topk(x, L.W_r, L.bias, 0, L.d, b["ids"], b["w"], b["logits"])
    moe.moe_quantize_act(x, 0, L.H, b["x_codes"], b["x_scales"], b["x_ts"])
    moe.moe_combine(b["out"], b["w"], x, 0, L.k, L.H, b["y"])
    torch.cuda.synchronize()
    for k, v in before.items():
        assert np.array_equal(t2n(b[k]), v), k
    # the decode FFN takes 1 <= T <= MOE_DECODE_MAX_T and says so
    with pytest.raises(moe.MoeError):
        moe.moe_expert_ffn_decode(L.d, L.experts(), (b["x_codes"], b["x_scales"], b["x_ts"]), b["ids"], 0,
                                  b["out"], b["ws"], b["ws_bytes"], None)
    with pytest.raises(moe.MoeError):
        moe.moe_expert_ffn_decode(L.d, L.experts(), (b["x_codes"], b["x_scales"], b["x_ts"]), b["ids"],
                                  moe.MOE_DECODE_MAX_T + 1, b["out"], b["ws"], b["ws_bytes"], None)


@pytest.mark.parametrize("T,path", [(1, "decode"), (16, "decode"), (64, "decode"), (40, "prefill"),
                                    (3100, "prefill")])
def test_largest_expert_count_and_topk(T, path):
    """E = 1024 experts and k = 32, the largest the library takes: the top-k
    over 16 logits per lane, 2048 (t, slot) pairs through the decode GEMVs at
    64 tokens (the most their pair lists hold), 512 pairs through the fused
    layer at 16 tokens, the 32-row and 128-row grouped GEMMs; every stage of
    every token (sampled tokens at 3100) against the oracle, the router
    against the oracle outside near-ties, the fused layer equal to the
    separate entry points."""
    c = case("max_ek", "device")
    wl = c.wl
    x = synth.activations(wl, T=T, stream=60 + T)
    g = run_layer(c, x, residual=True, prefill=(path == "prefill"))
    oids, ow, near, _, _ = orouter.route(x, c.W_r, wl.k)
    for t in range(T):
        assert len(set(g["ids"][t].tolist())) == wl.k
        if not near[t]:
            assert set(g["ids"][t].tolist()) == set(oids[t].tolist()), t
    if path == "prefill":
        assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == (32 if T * wl.k <= 96 * wl.E else 128)
    toks = None if T <= 64 else sorted({0, 1, T // 3, T // 2, T - 2, T - 1})
    say("max E/k", T, path, check_stages(c, x, g, residual=True, check_tokens=toks))
    if path == "decode" and T <= moe.MOE_LAYER_MAX_T:
        fb = c.L.alloc_fused(T)
        fb["ws"].fill_(0xFF)
        c.L.forward_fused(bf16_tensor(x, DEV), fb, residual=True)
        torch.cuda.synchronize()
        assert np.array_equal(t2n(fb["ids"]), g["ids"])
        assert np.array_equal(t2n(fb["y"]), g["y"])


@pytest.mark.parametrize("path", ["decode", "prefill", "fused"])
def test_zero_input(path):
    """x = 0 (with and without the residual): every logit is 0, an exact tie,
    so the ids are 0 .. k-1 in order with weights 1/k; x^ has tensor scale 0,
    so h, h^, o and y are exactly 0."""
    c = case("tiny", "host")
    T, k = 5, c.wl.k
    x = np.zeros((T, c.wl.H), np.uint16)
    if path == "fused":
        fb = c.L.alloc_fused(T)
        fb["ws"].fill_(0xFF)
        c.L.forward_fused(bf16_tensor(x, DEV), fb, residual=True)
        torch.cuda.synchronize()
        g = {kk: t2n(v) for kk, v in fb.items() if isinstance(v, torch.Tensor) and kk != "ws"}
    else:
        g = run_layer(c, x, residual=True, prefill=(path == "prefill"))
        assert not g["out"].any() and not g["dbg_h"].any() and not g["dbg_h_codes"].any()
        assert not g["dbg_h_scales"].any() and not g["dbg_h_ts"].any()
    assert np.array_equal(g["ids"], np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.all(g["w"] == np.float32(1.0 / k))
    assert not g["y"].view(np.uint16).any()
