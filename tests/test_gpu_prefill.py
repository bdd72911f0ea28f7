"""GPU parity: prefill expert FFN (grouped MFMA GEMMs over the permutation),
NVFP4 and codebook gate/up, stage by stage against the oracle."""
import numpy as np
import pytest
import torch

import synth
import quantized_moe_routed_router_amd as moe
from oracle import ffn as offn, router as orouter
from tests.gpu_helpers import (say, t2n, rowwise_rel, case, run_layer, check_stages, check_pairs,
                               check_y_all, pick_experts)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("T", [1, 4, 37, 300, 800])
def test_prefill_tiny(T):
    c = case("tiny", "host")
    x = synth.activations(c.wl, T=T, stream=300 + T)
    g = run_layer(c, x, prefill=True, residual=True)
    say("prefill tiny", T, check_stages(c, x, g, residual=True))


@pytest.mark.parametrize("T", [4, 300])
def test_prefill_static_h_scale(T):
    """Static h tensor scales per expert in the grouped-GEMM path: h^
    bit-exact with the oracle quantizer at those scales, other stages as
    usual; without debug copies o and y bit for bit the same."""
    c = case("tiny", "host")
    h_ts = synth.static_h_scales(c.wl)
    c.L.set_static_h_scales(torch.from_numpy(h_ts).to(DEV))
    try:
        x = synth.activations(c.wl, T=T, stream=800 + T)
        g = run_layer(c, x, prefill=True, residual=True)
        say("prefill static h", T, moe.moe_ffn_prefill_tile_rows(c.L.d, T),
            check_stages(c, x, g, residual=True, h_ts=h_ts))
        g2 = run_layer(c, x, prefill=True, residual=True, debug=False)
        assert np.array_equal(g2["out"], g["out"]) and np.array_equal(g2["y"], g["y"])
    finally:
        c.L.set_static_h_scales(None)


@pytest.mark.parametrize("fmt,T", [(moe.MOE_FMT_NVFP4, 16), (moe.MOE_FMT_NVFP4, 1024), (moe.MOE_FMT_CB3G128, 16),
                                   (moe.MOE_FMT_CB3G128, 1024)])
def test_prefill_static_h_32row_tiles(fmt, T):
    """Static h scales at Flash-Next shapes on the 32-row tiles (16 tokens:
    the gate/up K split across waves; 1,024 tokens: one wave per item): every
    stage against the oracle at the given scales (16 tokens), and the run
    without debug copies bit for bit equal in o and y to the run with them."""
    c = case("decode", "device", fmt)
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == 32
    h_ts = synth.static_h_scales(c.wl)
    c.L.set_static_h_scales(torch.from_numpy(h_ts).to(DEV))
    try:
        x = synth.activations(synth.WORKLOADS["decode_b8"], T=T, stream=870 + T)
        g = run_layer(c, x, prefill=True, residual=True)
        if T <= 16:
            say("static h 32-row", T, check_stages(c, x, g, residual=True, h_ts=h_ts))
        g2 = run_layer(c, x, prefill=True, residual=True, debug=False)
        assert np.array_equal(g2["ids"], g["ids"])
        assert np.array_equal(g2["out"], g["out"]) and np.array_equal(g2["y"], g["y"])
    finally:
        c.L.set_static_h_scales(None)


def _mixed_ids(T):
    """500 tokens, two slots: expert 5 at 372 rows and 3 at 128 (256-row
    tiles), 2 at 127, 6 at one row and 0, 1, 4, 7 at about 60 (32-row tiles)."""
    ids = np.zeros((T, 2), np.int32)
    ids[:372, 0] = 5
    ids[372:, 0] = 3
    rest = [0, 1, 4, 7]
    ids[:, 1] = [rest[t % 4] for t in range(T)]
    ids[:127, 1] = 2
    ids[200, 1] = 6
    return ids


@pytest.mark.parametrize("fmt", [moe.MOE_FMT_NVFP4, moe.MOE_FMT_CB3G128])
def test_prefill_static_h_256_tiling(fmt):
    """Static h scales on the 256-row tiling, both gate/up formats.  With the
    debug copies requested the h quantizer codes every h^ row (stage-checked
    against the oracle at the given scales); without them the 256-row gate/up
    epilogue codes its own rows' h^ and the h quantizer only the 32-row tiles'
    rows and the ids outside [0, E): o and y must come out bit for bit the
    same, also with two such ids."""
    c = case("wide_i", "host", fmt)
    h_ts = synth.static_h_scales(c.wl)
    c.L.set_static_h_scales(torch.from_numpy(h_ts).to(DEV))
    try:
        T = 500
        assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == 256
        x = synth.activations(c.wl, T=T, stream=85)
        ids = _mixed_ids(T)
        g = run_layer(c, x, prefill=True, ids_override=ids, residual=True)
        say("static h, 256-row tiling", check_stages(c, x, g, residual=True, h_ts=h_ts))
        g2 = run_layer(c, x, prefill=True, ids_override=ids, residual=True, debug=False)
        assert np.array_equal(g2["out"], g["out"]) and np.array_equal(g2["y"], g["y"])
        ids[3, 1] = -4
        ids[401, 1] = 8
        g = run_layer(c, x, prefill=True, ids_override=ids, residual=True)
        g2 = run_layer(c, x, prefill=True, ids_override=ids, residual=True, debug=False)
        assert np.all(g2["out"][3, 1] == 0) and np.all(g2["out"][401, 1] == 0)
        assert np.array_equal(g2["out"], g["out"]) and np.array_equal(g2["y"], g["y"])
    finally:
        c.L.set_static_h_scales(None)


def test_prefill_static_h_8k_epilogue_coding():
    """Static h scales at Flash-Next shapes, 8,192 tokens (the 256-row tiling,
    every expert on 256-row tiles or 32-row tiles by its count): the run
    without debug copies, where the 256-row gate/up epilogue codes h^, gives
    o and y bit for bit equal to the run with them, where the h quantizer
    codes every row."""
    c = case("decode", "device")
    h_ts = synth.static_h_scales(c.wl)
    c.L.set_static_h_scales(torch.from_numpy(h_ts).to(DEV))
    try:
        T = 8192
        assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == 256
        x = synth.activations(c.wl, T=T, stream=86)
        g = run_layer(c, x, prefill=True, residual=True)
        g2 = run_layer(c, x, prefill=True, residual=True, debug=False)
        assert np.array_equal(g2["ids"], g["ids"])
        assert np.array_equal(g2["out"], g["out"]) and np.array_equal(g2["y"], g["y"])
        say("static h 8k: o and y bit for bit")
    finally:
        c.L.set_static_h_scales(None)


def test_prefill_matches_decode_path():
    """Same tokens through both paths: identical ids and h^ codes (modulo
    accumulation-order flips), outputs within fp32 accumulation noise."""
    c = case("tiny", "host")
    x = synth.activations(c.wl, T=16, stream=77)
    gd = run_layer(c, x, prefill=False)
    gp = run_layer(c, x, prefill=True)
    assert np.array_equal(gd["ids"], gp["ids"])
    assert rowwise_rel(gp["dbg_h"], gd["dbg_h"]).max() <= 1e-5
    same = np.all(gd["dbg_h_codes"] == gp["dbg_h_codes"], axis=1)
    assert same.mean() >= 0.9
    r = rowwise_rel(gp["out"].reshape(-1, c.wl.H)[same], gd["out"].reshape(-1, c.wl.H)[same])
    assert r.max() <= 1e-5


@pytest.mark.parametrize("T,rows", [(700, 32), (800, 128)])
def test_prefill_skewed_ids_many_tiles(T, rows):
    """One expert holds most pairs (many m-tiles, ragged last tile), others
    few or none; includes ids outside [0, E) which give zero rows."""
    c = case("tiny", "host")
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == rows
    x = synth.activations(c.wl, T=T, stream=78)
    r = np.random.default_rng(1)
    ids = np.stack([np.array([5, r.integers(0, 16)]) for _ in range(T)]).astype(np.int32)
    ids[ids[:, 1] == 5, 1] = 6
    g = run_layer(c, x, prefill=True, ids_override=ids)
    check_stages(c, x, g, check_tokens=range(0, T, 7))
    ids2 = ids.copy()
    ids2[3, 1] = -4
    ids2[9, 0] = 16
    g2 = run_layer(c, x, prefill=True, ids_override=ids2)
    assert np.all(g2["out"][3, 1] == 0) and np.all(g2["out"][9, 0] == 0)
    ok = np.ones(ids.shape, bool)
    ok[3, 1] = ok[9, 0] = False
    assert np.array_equal(g2["out"][ok], g["out"][ok])


@pytest.mark.parametrize("T,rows", [(37, 32), (300, 32), (800, 128)])
def test_prefill_tiling_covered(T, rows):
    """The tiny prefill cases above run the 32-row and the 128-row tilings."""
    c = case("tiny", "host")
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == rows


def test_prefill_mid_tiles_skewed():
    """32-row expert tiles: one expert holds every token's first slot (120
    rows: three full tiles and a ragged one), the others a few rows each;
    then ids outside [0, E), which give zero rows."""
    c = case("tiny", "host")
    T = 120
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == 32
    x = synth.activations(c.wl, T=T, stream=79)
    r = np.random.default_rng(2)
    ids = np.stack([np.array([5, r.integers(0, 16)]) for _ in range(T)]).astype(np.int32)
    ids[ids[:, 1] == 5, 1] = 6
    g = run_layer(c, x, prefill=True, ids_override=ids)
    say("mid tiles skewed", check_stages(c, x, g, check_tokens=range(0, T, 3)))
    ids2 = ids.copy()
    ids2[3, 1] = -4
    ids2[9, 0] = 16
    g2 = run_layer(c, x, prefill=True, ids_override=ids2)
    assert np.all(g2["out"][3, 1] == 0) and np.all(g2["out"][9, 0] == 0)
    ok = np.ones(ids.shape, bool)
    ok[3, 1] = ok[9, 0] = False
    assert np.array_equal(g2["out"][ok], g["out"][ok])


@pytest.mark.parametrize("T", [1, 128, 4915])
def test_prefill_flash_next_mid(T):
    """Flash-Next shapes on the 32-row tiling (one token: gate/up split over K
    in four; 4915 tokens: the largest T it takes at k = 10, E = 512): every
    stage on every token up to 128 tokens; at 4915 every (t, slot) row of the
    chosen experts (most rows, ragged last tiles, low / middle / high ids) and
    y of every token."""
    c = case("decode", "device")
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == 32
    x = synth.activations(synth.WORKLOADS["decode_b8"], T=T, stream=900 + T)
    g = run_layer(c, x, residual=True, prefill=True)
    if T <= 128:
        say(f"prefill mid T={T}", check_stages(c, x, g, residual=True))
        return
    for e in pick_experts(g["ids"], c.wl.E, 32):
        say(f"prefill mid T={T} expert {e}", check_pairs(c, x, g, np.nonzero(g["ids"].reshape(-1) == e)[0]))
    say(f"prefill mid T={T} y all tokens", check_y_all(g, x, residual=True))


@pytest.mark.parametrize("T,rows", [(4, 32), (300, 32), (500, 256)])
def test_prefill_wide_intermediate(T, rows):
    """I = 1152: each h row has 72 NVFP4 blocks, so the h quantization's lanes
    hold two blocks each; on the 32-row tiles (split K at 4 tokens) and the
    256-row tiles."""
    c = case("wide_i", "host")
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == rows
    x = synth.activations(c.wl, T=T, stream=40 + T)
    g = run_layer(c, x, prefill=True, residual=True)
    say("prefill wide I", T, check_stages(c, x, g, residual=True,
                                          check_tokens=None if T <= 4 else range(0, T, 9)))


@pytest.mark.parametrize("fmt", [moe.MOE_FMT_NVFP4, moe.MOE_FMT_CB3G128])
def test_prefill_mixed_tiles_skewed(fmt):
    """The 256-row tiling with experts on both sides of the 128-row split, for
    both gate/up formats:
    expert 5 has 372 rows (two 256-row tiles, the second ragged) and expert 3
    exactly 128 (one 256-row tile), expert 2 has 127 (four 32-row tiles, the
    last ragged), expert 6 one row and the others about 60 each (32-row
    tiles); then two ids outside [0, E), which give zero rows.  Every token
    through every stage."""
    c = case("wide_i", "host", fmt)
    T = 500
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == 256
    x = synth.activations(c.wl, T=T, stream=81)
    ids = np.zeros((T, 2), np.int32)
    ids[:372, 0] = 5
    ids[372:, 0] = 3
    rest = [0, 1, 4, 7]
    ids[:, 1] = [rest[t % 4] for t in range(T)]
    ids[:127, 1] = 2
    ids[200, 1] = 6
    counts = np.bincount(ids.reshape(-1), minlength=8)
    assert counts[5] == 372 and counts[3] == 128 and counts[2] == 127 and counts[6] == 1
    g = run_layer(c, x, prefill=True, ids_override=ids, residual=True)
    say("mixed tiles", check_stages(c, x, g, residual=True))
    # each expert stays in its list, so every other row is bit for bit the same
    ids2 = ids.copy()
    ids2[3, 1] = -4
    ids2[401, 1] = 8
    g2 = run_layer(c, x, prefill=True, ids_override=ids2, residual=True)
    assert np.all(g2["out"][3, 1] == 0) and np.all(g2["out"][401, 1] == 0)
    ok = np.ones(ids.shape, bool)
    ok[3, 1] = ok[401, 1] = False
    assert np.array_equal(g2["out"][ok], g["out"][ok])


@pytest.mark.parametrize("fmt", [moe.MOE_FMT_NVFP4, moe.MOE_FMT_CB3G128])
def test_prefill_256_tiling_all_small(fmt):
    """The 256-row tiling with every expert under 128 rows (125 each): the
    256-row tile list is empty, so the launches' trailing 32-row-tile blocks
    do all of both GEMMs.  Every token through every stage."""
    c = case("wide_i", "host", fmt)
    T = 500
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == 256
    x = synth.activations(c.wl, T=T, stream=83)
    t = np.arange(T)
    ids = np.stack([t % 8, (t + 3) % 8], axis=1).astype(np.int32)
    counts = np.bincount(ids.reshape(-1), minlength=8)
    assert counts.max() < 128 and counts.min() > 96
    g = run_layer(c, x, prefill=True, ids_override=ids, residual=True)
    say("all experts on 32-row tiles", check_stages(c, x, g, residual=True))


@pytest.mark.parametrize("T,rows", [(40, 32), (800, 128)])
def test_prefill_codebook_tiny(T, rows):
    c = case("tiny", "host", moe.MOE_FMT_CB3G128)
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == rows
    x = synth.activations(c.wl, T=T, stream=79)
    g = run_layer(c, x, prefill=True, residual=True)
    say("prefill codebook tiny", T, check_stages(c, x, g, residual=True,
                                                 check_tokens=None if T <= 40 else range(0, T, 5)))


@pytest.mark.parametrize("T", [1, 128, 3276])
def test_prefill_codebook_flash_next_mid(T):
    """Codebook gate/up at Flash-Next shapes on the 32-row tiles (3276 tokens
    is the largest T on them): every stage on every token up to 128 tokens;
    at 3276 every (t, slot) row of the chosen experts and y of every token."""
    c = case("decode", "device", moe.MOE_FMT_CB3G128)
    assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == 32
    x = synth.activations(synth.WORKLOADS["decode_b8"], T=T, stream=950 + T)
    g = run_layer(c, x, residual=True, prefill=True)
    if T <= 128:
        say(f"prefill codebook mid T={T}", check_stages(c, x, g, residual=True))
        return
    for e in pick_experts(g["ids"], c.wl.E, 32):
        say(f"prefill codebook mid T={T} expert {e}", check_pairs(c, x, g, np.nonzero(g["ids"].reshape(-1) == e)[0]))
    say(f"prefill codebook mid T={T} y all tokens", check_y_all(g, x, residual=True))


@pytest.mark.parametrize("fmt", [moe.MOE_FMT_NVFP4, moe.MOE_FMT_CB3G128])
def test_prefill_zipf_8k_full_rows(fmt):
    """The 8192-token Zipf-routed layer at full size (256-row tiles for both
    gate/up formats): every output element written (sentinels), every
    (t, slot) row of the chosen experts (the most popular, the ragged last
    tiles, low / middle / high ids, a tail expert) through all stages, y of
    every token, and the router against the oracle on sampled tokens."""
    c = case("decode", "device", fmt)
    wl = synth.WORKLOADS["prefill8k"]
    c.L.set_router(torch.from_numpy(synth.router_weights(wl)).to(DEV),
                   torch.from_numpy(synth.router_bias(wl)).to(DEV))
    try:
        assert moe.moe_ffn_prefill_tile_rows(c.L.d, wl.T) == 256
        x = synth.activations(wl, T=wl.T)
        g = run_layer(c, x, prefill=True, residual=True)
        counts = np.bincount(g["ids"].reshape(-1), minlength=wl.E)
        say("zipf top counts", np.sort(counts)[::-1][:5], "zero experts", int((counts == 0).sum()))
        assert counts.max() > 1000 and (counts == 0).sum() > 100
        experts = pick_experts(g["ids"], wl.E, 256)
        say("zipf experts", [(e, int(counts[e])) for e in experts])
        for e in experts:
            pairs = np.nonzero(g["ids"].reshape(-1) == e)[0]
            say("zipf expert", e, check_pairs(c, x, g, pairs))
        say("zipf y all tokens", check_y_all(g, x, residual=True))
        top = int(counts.argmax())
        t_top = int(np.nonzero((g["ids"] == top).any(1))[0][-1])
        toks = [0, t_top, wl.T - 1]
        oids, _, near, _, _ = orouter.route(x[toks], synth.router_weights(wl), wl.k, synth.router_bias(wl))
        for i, t in enumerate(toks):
            if not near[i]:
                assert set(g["ids"][t]) == set(oids[i])
    finally:
        c.L.set_router(torch.from_numpy(c.W_r).to(DEV), None)


@pytest.mark.parametrize("fmt", [moe.MOE_FMT_NVFP4, moe.MOE_FMT_CB3G128])
def test_prefill_64k_full_rows(fmt):
    """65536 tokens with uniform routing at full size (the long-prefill
    workload): every output element written (sentinels), every (t, slot) row
    of the chosen experts through all stages (about 1,300 rows each over six
    256-row tiles), y of every token."""
    c = case("decode", "device", fmt)
    wl = synth.WORKLOADS["prefill64k"]
    c.L.set_router(torch.from_numpy(synth.router_weights(wl)).to(DEV), None)
    try:
        assert moe.moe_ffn_prefill_tile_rows(c.L.d, wl.T) == 256
        xt = synth.activations_torch(wl, wl.T, 0, DEV)
        xb = xt.view(torch.int16).cpu().numpy().view(np.uint16)
        del xt
        g = run_layer(c, xb, prefill=True, residual=True)
        counts = np.bincount(g["ids"].reshape(-1), minlength=wl.E)
        assert counts.min() > 900 and counts.max() < 1700          # ~1280 each
        experts = pick_experts(g["ids"], wl.E, 256)
        say("64k experts", fmt, [(e, int(counts[e])) for e in experts])
        for e in experts:
            pairs = np.nonzero(g["ids"].reshape(-1) == e)[0]
            say("64k expert", e, check_pairs(c, xb, g, pairs))
        say("64k y all tokens", check_y_all(g, xb, residual=True))
    finally:
        c.L.set_router(torch.from_numpy(c.W_r).to(DEV), None)
