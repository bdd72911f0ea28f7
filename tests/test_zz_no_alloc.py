"""The no-allocation decode layer entry (moe_layer_decode_noalloc) against
moe_layer_decode with a caller workspace: same ids, weights and y bit for
bit, on two calls in a row, the second with fewer tokens (the scratch array
keeps the first call's contents); and the entry captured into a HIP graph,
each replay equal to the eager call on the same input."""
import numpy as np
import pytest
import torch

import synth
import quantized_moe_routed_router_amd as moe
from tests.gpu_helpers import say, t2n, bf16_tensor, case, SENT_BF16, SENT_ID

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _with_workspace(L, x, T, residual):
    fb = L.alloc_fused(T)
    fb["ws"].fill_(0xFF)
    L.forward_fused(x, fb, residual=residual)
    torch.cuda.synchronize()
    return t2n(fb["ids"]), t2n(fb["w"]), t2n(fb["y"])


def _noalloc(L, x, T, residual):
    ids = torch.full((T, L.k), SENT_ID, dtype=torch.int32, device=DEV)
    w = torch.full((T, L.k), float("nan"), dtype=torch.float32, device=DEV)
    y = torch.full((T, L.H), SENT_BF16, dtype=torch.int16, device=DEV)
    torch.cuda.synchronize()
    moe.moe_layer_decode_noalloc(L.d, L.experts(), x, L.W_r, L.bias, T, residual, y, ids, w)
    torch.cuda.synchronize()
    return t2n(ids), t2n(w), t2n(y)


@pytest.mark.parametrize("name,src,Ts", [("decode", "device", (8, 1)), ("tiny", "host", (16, 3))])
def test_noalloc_equals_workspace_entry(name, src, Ts):
    c = case(name, src)
    wl = synth.WORKLOADS["decode_b8" if name == "decode" else name]
    need = max(moe.moe_layer_decode_workspace_bytes(c.L.d, T) for T in Ts)
    assert 0 < need <= moe.MOE_NOALLOC_SCRATCH_BYTES
    for i, T in enumerate(Ts):
        x = bf16_tensor(synth.activations(wl, T=T, stream=1300 + T), DEV)
        residual = i == 0
        a = _noalloc(c.L, x, T, residual)
        b = _with_workspace(c.L, x, T, residual)
        assert not np.any(a[0] == SENT_ID) and not np.isnan(a[1]).any()
        assert not np.any(a[2].view(np.uint16) == 0xFFFF)
        assert np.array_equal(a[0], b[0])
        assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
        assert np.array_equal(a[2], b[2])
        say("noalloc == workspace entry", name, "T", T)


def test_noalloc_refuses_oversized_layer():
    d = moe.dims(1024, 4096, 2560, 32)
    L = case("tiny", "host").L
    assert moe.moe_layer_decode_workspace_bytes(d, 16) > moe.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_decode_noalloc(d, L.experts(), L.W_r, L.W_r, None, 16, True, L.W_r, None, None)
    assert ei.value.code == moe.MOE_ERR_WORKSPACE and "scratch" in str(ei.value)


@pytest.mark.parametrize("T", [1, 8])
def test_noalloc_replays_under_graph_capture(T):
    """The entry's use case: the call captured into a HIP graph (after one
    eager call on the device, which takes the scratch array's address) and
    replayed with new inputs copied into the captured input buffer; every
    replay, with eager work between replays, equals the eager call on the same
    input bit for bit."""
    c = case("decode", "device")
    L = c.L
    wl = synth.WORKLOADS["decode_b8"]
    xs = [bf16_tensor(synth.activations(wl, T=T, stream=1400 + 8 * T + i), DEV) for i in range(3)]
    xin = torch.empty_like(xs[0])
    ids = torch.empty((T, L.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, L.k), dtype=torch.float32, device=DEV)
    y = torch.empty((T, L.H), dtype=torch.int16, device=DEV)
    eager = [_noalloc(L, x, T, True) for x in xs]
    s = torch.cuda.Stream()
    xin.copy_(xs[0])
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        moe.moe_layer_decode_noalloc(L.d, L.experts(), xin, L.W_r, L.bias, T, True, y, ids, w, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_layer_decode_noalloc(L.d, L.experts(), xin, L.W_r, L.bias, T, True, y, ids, w, stream=s)
    for rep in range(3):
        for i, x in enumerate(xs):
            xin.copy_(x)
            y.fill_(SENT_BF16)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(t2n(ids), eager[i][0]), (rep, i)
            assert np.array_equal(t2n(w).view(np.uint32), eager[i][1].view(np.uint32)), (rep, i)
            assert np.array_equal(t2n(y), eager[i][2]), (rep, i)
            _ = (y.float() * 2).sum().item()                   # eager work between replays
    say("noalloc graph replays match eager, T", T)
