"""The no-allocation decode layer entry (moe_layer_decode_noalloc) against
moe_layer_decode with a caller workspace: same ids, weights and y bit for
bit, on two calls in a row, the second with fewer tokens (the scratch array
keeps the first call's contents)."""
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
