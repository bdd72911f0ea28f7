"""GPU parity: decode expert FFN and combine, stage by stage.

Stages (each compared on the device's own upstream values where a discrete
decision could legitimately differ):
  h    vs oracle gate/up on the device's ids        max row rel <= 1e-5
  h^   vs oracle quantizer on the device's h        bit-exact
  o    vs oracle down projection of the device's h^ max row rel <= 2e-3
  o    vs the pure oracle (its own h^)              rows without an h^ flip <= 2e-3
  y    vs oracle combine of the device's o and w    max row rel <= 2e-3
"""
import numpy as np
import pytest
import torch

import synth
import quantized_moe_routed_router_amd as moe
from oracle import ffn as offn, nvfp4, router as orouter
from tests.gpu_helpers import (LayerCase, say, t2n, bf16_tensor, rowwise_rel, assert_bf16_rounding_of,
                               case, run_layer, check_stages, check_fused_against_separate)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

def test_decode_tiny_all_stages():
    c = case("tiny", "host")
    x = synth.activations(c.wl, T=4)
    g = run_layer(c, x)
    # ids against the oracle router (no near-ties expected at this scale)
    oids, ow, near, _, _ = orouter.route(x, c.W_r, c.wl.k)
    for t in range(4):
        if not near[t]:
            assert set(g["ids"][t]) == set(oids[t])
    say("tiny stages", check_stages(c, x, g))


def test_decode_tiny_residual_and_pure_oracle():
    c = case("tiny", "host")
    x = synth.activations(c.wl, T=4, stream=2)
    g = run_layer(c, x, residual=True)
    check_stages(c, x, g, residual=True)
    experts = {e: c.oracle_expert(e) for e in range(c.wl.E)}
    pure = offn.layer(x, c.W_r, None, experts, c.wl.k, residual=True)
    ok = ~pure["near"]
    # the FFN part within 2e-3 of the pure oracle's; y a bf16 rounding of it
    o_dev = np.einsum("tk,tkh->th", g["w"].astype(np.float64), g["out"].astype(np.float64))
    o_ref = np.einsum("tk,tkh->th", pure["w"], pure["o"])
    assert rowwise_rel(o_dev[ok], o_ref[ok]).max() <= 2e-3
    assert_bf16_rounding_of(g["y"][ok], pure["y"][ok], slack_rel=2e-3)


@pytest.mark.parametrize("T", [1, 2, 3, 8, 16, 17, 33, 64])
def test_decode_tiny_batch_sizes(T):
    c = case("tiny", "host")
    x = synth.activations(c.wl, T=T, stream=10 + T)
    check_stages(c, x, run_layer(c, x))


@pytest.mark.parametrize("name", ["wide4k", "wide10k"])
def test_decode_one_token_split_k(name):
    """One token with H above 2560 (H/32 over one block's 80 chunks): gate/up
    split over K, the separate h^ kernel summing the split partials, and the
    slice down kernel reading h^ (the path the one-split h mode bypasses)."""
    c = case(name, "host")
    for stream, residual in ((5, False), (6, True)):
        x = synth.activations(c.wl, T=1, stream=stream)
        say(name, "split-K decode stages", check_stages(c, x, run_layer(c, x, residual=residual), residual=residual))


def test_decode_shared_experts_and_batching():
    """Several tokens on the same experts (one weight read serves them all),
    including more than 8 pairs on one expert (second pass of a block)."""
    c = case("tiny", "host")
    T = 12
    x = synth.activations(c.wl, T=T, stream=40)
    ids = np.tile(np.array([[3, 5]], np.int32), (T, 1))
    ids[5] = [5, 3]
    ids[7] = [0, 15]
    g = run_layer(c, x, ids_override=ids)
    assert np.array_equal(g["ids"], ids)
    check_stages(c, x, g)


def test_decode_invalid_ids_give_zero():
    c = case("tiny", "host")
    x = synth.activations(c.wl, T=2, stream=41)
    ids = np.array([[1, -1], [99, 2]], np.int32)
    g = run_layer(c, x, ids_override=ids)
    assert np.all(g["out"][0, 1] == 0) and np.all(g["out"][1, 0] == 0)
    assert np.abs(g["out"][0, 0]).max() > 0


def test_decode_deterministic():
    c = case("tiny", "host")
    x = synth.activations(c.wl, T=8, stream=42)
    a = run_layer(c, x)
    b = run_layer(c, x)
    for k in ("ids", "w", "out", "y", "dbg_h", "dbg_h_codes"):
        assert np.array_equal(a[k], b[k]), k


def test_decode_flash_next_b1():
    c = case("decode", "device")
    for s in (0, 1):
        x = synth.activations(c.wl, T=1, stream=100 + s)
        g = run_layer(c, x)
        oids, ow, near, _, _ = orouter.route(x, c.W_r, c.wl.k)
        if not near[0]:
            assert set(g["ids"][0]) == set(oids[0])
        say("decode b1 stages", check_stages(c, x, g))


def test_decode_flash_next_b8():
    """Eight tokens at Flash-Next shapes: every token through every stage."""
    c = case("decode", "device")
    x = synth.activations(synth.WORKLOADS["decode_b8"], T=8, stream=200)
    g = run_layer(c, x, residual=True)
    say("decode b8 stages", check_stages(c, x, g, residual=True))


@pytest.mark.parametrize("T", [32, 64])
def test_decode_flash_next_many_tokens(T):
    """Decode GEMVs at 32 and 64 tokens (320 and 640 (t, slot) pairs; above 512
    pairs the kernels hold 32 chunks of pair ids per lane): every token
    through every stage, and the whole output against the grouped-GEMM
    (prefill) entry on the same ids."""
    c = case("decode", "device")
    x = synth.activations(synth.WORKLOADS["decode_b8"], T=T, stream=300 + T)
    g = run_layer(c, x, residual=True, prefill=False)
    say(f"decode T={T} stages", check_stages(c, x, g, residual=True))
    gp = run_layer(c, x, residual=True, prefill=True)
    assert np.array_equal(g["ids"], gp["ids"])
    assert rowwise_rel(g["out"], gp["out"]).max() <= 2e-3


@pytest.mark.parametrize("name,T", [("tiny", 1), ("tiny", 5), ("wide4k", 1), ("decode", 1), ("decode", 8)])
def test_decode_static_h_scale(name, T):
    """Static (calibrated) h tensor scales per expert: h^ bit-exact with the
    oracle quantizer at those scales (one token: quantized in the gate/up
    kernel; otherwise in the h^ kernel), every other stage as usual; the fused
    layer against the separate entry points."""
    c = case(name, "host" if name in ("tiny", "wide4k") else "device")
    h_ts = synth.static_h_scales(c.wl)
    c.L.set_static_h_scales(torch.from_numpy(h_ts).to(DEV))
    try:
        x = synth.activations(synth.WORKLOADS["decode_b8"] if name == "decode" else c.wl, T=T, stream=700 + T)
        g = run_layer(c, x, residual=True)
        say(name, T, "static h stages",
            check_stages(c, x, g, residual=True, h_ts=h_ts, check_tokens=None if T <= 5 else [0, T - 1]))
        if c.wl.H <= 4096:
            fb = c.L.alloc_fused(T)
            c.L.forward_fused(bf16_tensor(x, DEV), fb, residual=True)
            torch.cuda.synchronize()
            f = {k: t2n(v) for k, v in fb.items() if isinstance(v, torch.Tensor) and k != "ws"}
            check_fused_against_separate(f, g, x, True, ("static h", name, T))
    finally:
        c.L.set_static_h_scales(None)


def test_combine_parity():
    say("combine")
    r = np.random.default_rng(8)
    for T, k, H in [(1, 10, 2560), (7, 2, 256), (33, 3, 128)]:
        o = r.standard_normal((T, k, H)).astype(np.float32)
        w = r.random((T, k)).astype(np.float32)
        w /= w.sum(1, keepdims=True)
        res = synth.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
        for use_res in (False, True):
            y = torch.empty((T, H), dtype=torch.int16, device=DEV)
            moe.moe_combine(torch.from_numpy(o).to(DEV), torch.from_numpy(w).to(DEV),
                            bf16_tensor(res, DEV) if use_res else None, T, k, H, y)
            torch.cuda.synchronize()
            ref = offn.combine(o, w, res if use_res else None)
            assert_bf16_rounding_of(t2n(y), ref)


@pytest.mark.parametrize("name,src,Ts", [("tiny", "host", (1, 5, 12)), ("decode", "device", (1, 8, 12))])
def test_decode_codebook_gate_up(name, src, Ts):
    """The decode GEMVs on 3-bit group-128 codebook gate/up weights (down
    NVFP4): every token through every stage (h against the oracle's codebook
    dequantization, h^ bit-exact, o, y), and the fused layer against the
    separate entry points (ids and w bit for bit; y bit for bit where both
    run the same down kernel, else one rounding of the same sum)."""
    c = case(name, src, moe.MOE_FMT_CB3G128)
    wl = synth.WORKLOADS["decode_b8" if name == "decode" else name]
    for T in Ts:
        x = synth.activations(wl, T=T, stream=1400 + T)
        g = run_layer(c, x, residual=True, prefill=False)
        say(name, "codebook decode T", T, check_stages(c, x, g, residual=True))
        fb = c.L.alloc_fused(T)
        fb["ws"].fill_(0xFF)
        c.L.forward_fused(bf16_tensor(x, DEV), fb, residual=True)
        torch.cuda.synchronize()
        f = {k: t2n(v) for k, v in fb.items() if isinstance(v, torch.Tensor) and k != "ws"}
        check_fused_against_separate(f, g, x, True, ("codebook", name, T))


def test_decode_codebook_static_h_scale():
    c = case("tiny", "host", moe.MOE_FMT_CB3G128)
    h_ts = synth.static_h_scales(c.wl)
    c.L.set_static_h_scales(torch.from_numpy(h_ts).to(DEV))
    try:
        for T in (1, 4):
            x = synth.activations(c.wl, T=T, stream=1500 + T)
            g = run_layer(c, x, residual=True, prefill=False)
            say("codebook static h T", T, check_stages(c, x, g, residual=True, h_ts=h_ts))
    finally:
        c.L.set_static_h_scales(None)
