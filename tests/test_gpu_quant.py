"""GPU parity: NVFP4 quantizers and the packed layout, bit-exact against the
oracle on the same inputs."""
import numpy as np
import pytest
import torch

import synth
import quantized_moe_routed_router_amd as moe
from oracle import nvfp4, ffn as offn
from tests.gpu_helpers import say, t2n, bf16_tensor

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _act_quant_gpu(xbits: np.ndarray):
    T, H = xbits.shape
    x = bf16_tensor(xbits, DEV)
    codes = torch.empty((T, H // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((T, H // 16), dtype=torch.uint8, device=DEV)
    ts = torch.empty(T, dtype=torch.float32, device=DEV)
    moe.moe_quantize_act(x, T, H, codes, scales, ts)
    torch.cuda.synchronize()
    return t2n(codes), t2n(scales), t2n(ts)


def _check_act(xbits):
    c, s, ts = _act_quant_gpu(xbits)
    oc, os_, ots = offn.quantize_act(xbits)
    assert np.array_equal(c, nvfp4.pack_nibbles(oc))
    assert np.array_equal(s, os_)
    assert np.array_equal(ts.view(np.uint32), np.asarray(ots, np.float32).view(np.uint32))


@pytest.mark.parametrize("name,T", [("tiny", 4), ("decode", 1), ("decode_b8", 8), ("decode", 37),
                                    ("prefill8k", 300)])
def test_act_quant_bit_exact(name, T):
    say("act quant", name, T)
    wl = synth.WORKLOADS[name]
    _check_act(synth.activations(wl, T=T, stream=7))


def test_act_quant_adversarial_rows():
    say("act quant adversarial")
    H = 256
    rows = []
    r = np.random.default_rng(5)
    rows.append(np.zeros(H, np.float32))                         # all zero -> ts 0
    z = np.zeros(H, np.float32); z[::3] = -0.0; rows.append(z)   # negative zeros
    rows.append(np.full(H, 0.37, np.float32))                    # all equal
    v = r.standard_normal(H).astype(np.float32); v[7] = 5000.0; rows.append(v)    # outlier
    v = (r.standard_normal(H) * np.exp2(r.integers(-60, 60, H))).astype(np.float32); rows.append(v)
    d = 2.0 ** -4                                                 # exact E2M1 midpoints
    v = np.zeros(H, np.float32); v[0] = 168.0
    v[32:40] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]) * d
    v[16] = 0.375 * 1.1875                                        # E4M3 tie in a block scale
    rows.append(v)
    v = np.full(H, 1e-38, np.float32); v[1] = -3e-38; rows.append(v)   # subnormal-range ts
    xbits = synth.f32_to_bf16_bits(np.stack(rows))
    _check_act(xbits)


def test_act_quant_midpoint_search_cases():
    """Rows aimed within a few ulps of E2M1 midpoints (after bf16 rounding)."""
    say("act quant midpoint cases")
    r = np.random.default_rng(6)
    H, T = 512, 64
    x = r.standard_normal((T, H)).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for t in range(T):
        amax = np.float32(np.abs(x[t]).max())
        ts = np.float32(amax / np.float32(2688))
        d = np.float32(np.float32(0.5) * ts * np.float32(448))  # a plausible block d
        sel = r.integers(0, H, 40)
        x[t, sel] = (mids[r.integers(0, 7, 40)] * d).astype(np.float32)
    _check_act(synth.f32_to_bf16_bits(x))


@pytest.mark.parametrize("name,n,rows,cols", [("tiny", 3, 128, 256), ("decode", 2, 640, 2560),
                                              ("decode", 1, 2560, 640), ("tiny", 1, 16, 16)])
def test_weight_quant_bit_exact(name, n, rows, cols):
    say("weight quant", name, n, rows, cols)
    r = np.random.default_rng(rows + cols + n)
    W = (r.standard_normal((n, rows, cols)) * 0.02).astype(np.float32)
    W[0, 0, :16] = 0.0
    if n > 1:
        W[1] *= np.float32(1e-3)
    Wd = torch.from_numpy(W).to(DEV)
    codes = torch.empty((n, rows, cols // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((n, rows, cols // 16), dtype=torch.uint8, device=DEV)
    ts = torch.empty(n, dtype=torch.float32, device=DEV)
    moe.moe_quantize_weights(Wd, n, rows, cols, codes, scales, ts)
    torch.cuda.synchronize()
    c, s, t = t2n(codes), t2n(scales), t2n(ts)
    for i in range(n):
        oc, os_, ots = nvfp4.quantize(W[i], per_row=False)
        assert np.array_equal(c[i], nvfp4.pack_nibbles(oc)), i
        assert np.array_equal(s[i], os_), i
        assert np.float32(t[i]).view(np.uint32) == np.float32(ots).view(np.uint32), i


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_pack_unpack_round_trip(name):
    say("pack/unpack", name)
    wl = synth.WORKLOADS[name]
    n = 3
    d = moe.dims(wl.E, wl.H, wl.I, wl.k)
    r = np.random.default_rng(9)
    plain = dict(
        gc=r.integers(0, 256, (n, wl.I, wl.H // 2), dtype=np.uint8),
        gs=r.integers(0, 127, (n, wl.I, wl.H // 16), dtype=np.uint8),
        uc=r.integers(0, 256, (n, wl.I, wl.H // 2), dtype=np.uint8),
        us=r.integers(0, 127, (n, wl.I, wl.H // 16), dtype=np.uint8),
        dc=r.integers(0, 256, (n, wl.H, wl.I // 2), dtype=np.uint8),
        ds=r.integers(0, 127, (n, wl.H, wl.I // 16), dtype=np.uint8))
    dev = {k: torch.from_numpy(v).to(DEV) for k, v in plain.items()}
    gu = torch.zeros(moe.moe_packed_bytes(d, 0), dtype=torch.uint8, device=DEV)
    dn = torch.zeros(moe.moe_packed_bytes(d, 1), dtype=torch.uint8, device=DEV)
    e0 = wl.E - n
    moe.moe_pack_nvfp4(d, e0, n, dev["gc"], dev["gs"], dev["uc"], dev["us"], dev["dc"], dev["ds"], gu, dn)
    back = {k: torch.zeros_like(v) for k, v in dev.items()}
    moe.moe_unpack_nvfp4(d, e0, n, back["gc"], back["gs"], back["uc"], back["us"], back["dc"], back["ds"], gu, dn)
    torch.cuda.synchronize()
    for k in plain:
        assert np.array_equal(t2n(back[k]), plain[k]), k
    # layout spot check: expert e0, gate/up tile 0, chunk 1, lane 33 = up row 1, elements 32..63
    tile = t2n(gu[e0 * (wl.I // 32) * 36 * wl.H:][:36 * wl.H])
    assert np.array_equal(tile[1024 + 33 * 16:1024 + 34 * 16], plain["uc"][0, 1, 16:32])
    # untouched experts stay zero
    assert not t2n(gu[:e0 * (wl.I // 32) * 36 * wl.H]).any()
