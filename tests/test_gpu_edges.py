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
from tests.gpu_helpers import say, t2n, bf16_tensor, case, run_layer, check_stages

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
    assert np.array_equal(t2n(fb["ids"]), dec["ids"])
    assert np.array_equal(t2n(fb["y"]), dec["y"])
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
