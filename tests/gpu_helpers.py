"""Shared set-up for the GPU parity tests: builds a layer on the device from
the seeded generators, and hands the oracle the very same fp32 inputs.

Nothing the oracle receives comes from the HIP path except where a test says
so explicitly (the staged comparisons feed the device's ids and h forward).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
import quantized_moe_routed_router_amd as moe
from oracle import ffn as offn, nvfp4

DEV = "cuda:0"


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


class LayerCase:
    """A layer on the device plus lazy oracle views of its experts."""

    def __init__(self, wl: synth.Workload, layer: int = 0, source: str = "host",
                 fmt: int = moe.MOE_FMT_NVFP4):
        self.wl, self.layer, self.source = wl, layer, source
        self.dev = torch.device("cuda:0")
        self.L = moe.Layer(wl.E, wl.H, wl.I, wl.k, fmt_gate_up=fmt, device=self.dev)
        self.W_r = synth.router_weights(wl, layer)
        b = synth.router_bias(wl, layer)
        self.bias = b
        self.L.set_router(torch.from_numpy(self.W_r).to(self.dev),
                          None if b is None else torch.from_numpy(b).to(self.dev))
        self._q = {}
        chunk = 32
        for e0 in range(0, wl.E, chunk):
            e1 = min(wl.E, e0 + chunk)
            if source == "host":
                ws = [synth.expert_weights(wl, layer, e) for e in range(e0, e1)]
                g = torch.from_numpy(np.stack([w[0] for w in ws])).to(self.dev)
                u = torch.from_numpy(np.stack([w[1] for w in ws])).to(self.dev)
                d = torch.from_numpy(np.stack([w[2] for w in ws])).to(self.dev)
            else:
                g, u, d = synth.expert_weights_torch(wl, layer, e0, e1, self.dev)
            if fmt == moe.MOE_FMT_NVFP4:
                self.L.load_experts_fp32(e0, g, u, d)
            else:
                self.L.load_experts_fp32(e0, None, None, d)
                cbg, ixg, cbu, ixu = self._codebooks(e0, e1)
                self.L.load_codebook(e0, cbg, ixg, cbu, ixu)
            del g, u, d
        torch.cuda.synchronize()

    def _codebooks(self, e0, e1):
        wl = self.wl
        if self.source == "host":
            gs = [synth.codebook_weights(wl, self.layer, e, synth.PROJ_GATE) for e in range(e0, e1)]
            us = [synth.codebook_weights(wl, self.layer, e, synth.PROJ_UP) for e in range(e0, e1)]
            f = lambda xs, i: torch.from_numpy(np.stack([x[i] for x in xs])).to(self.dev)
            return f(gs, 0), f(gs, 1), f(us, 0), f(us, 1)
        cbg, ixg = synth.codebook_weights_torch(wl, self.layer, e0, e1, synth.PROJ_GATE, self.dev)
        cbu, ixu = synth.codebook_weights_torch(wl, self.layer, e0, e1, synth.PROJ_UP, self.dev)
        return cbg, ixg, cbu, ixu

    def fp32_expert(self, e: int):
        """The fp32 weights the device layer was built from, on the host."""
        if self.source == "host":
            return synth.expert_weights(self.wl, self.layer, e)
        g, u, d = synth.expert_weights_torch(self.wl, self.layer, e, e + 1, self.dev)
        return g[0].cpu().numpy(), u[0].cpu().numpy(), d[0].cpu().numpy()

    def oracle_expert(self, e: int):
        """Oracle-quantized expert (QExpert) from the same fp32 weights."""
        if e not in self._q:
            g, u, d = self.fp32_expert(e)
            if self.L.fmt == moe.MOE_FMT_NVFP4:
                self._q[e] = offn.quantize_expert(g, u, d)
            else:
                from oracle.codebook import CBMatrix
                if self.source == "host":
                    cg = synth.codebook_weights(self.wl, self.layer, e, synth.PROJ_GATE)
                    cu = synth.codebook_weights(self.wl, self.layer, e, synth.PROJ_UP)
                else:
                    a = synth.codebook_weights_torch(self.wl, self.layer, e, e + 1, synth.PROJ_GATE, self.dev)
                    b = synth.codebook_weights_torch(self.wl, self.layer, e, e + 1, synth.PROJ_UP, self.dev)
                    cg = (a[0][0].cpu().numpy(), a[1][0].cpu().numpy())
                    cu = (b[0][0].cpu().numpy(), b[1][0].cpu().numpy())
                self._q[e] = offn.QExpert(CBMatrix(*cg), CBMatrix(*cu), offn.quantize_matrix(d))
        return self._q[e]

    def oracle_deq(self, experts):
        return {int(e): offn.dequant_expert(self.oracle_expert(int(e))) for e in np.unique(experts)}


def t2n(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_tensor(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).to(dev)


def rowwise_rel(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """max |got - ref| / max |ref| per row (last axis); 0 where the row is 0."""
    got = got.reshape(-1, got.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    den = np.abs(ref).max(axis=1)
    num = np.abs(got - ref).max(axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |v| (8 significant bits)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def assert_bf16_rounding_of(y_dev_bits: np.ndarray, y_ref: np.ndarray, slack_rel: float = 1e-5):
    """y_dev (bf16 bits) must be a round-to-nearest of a value within
    slack_rel * rowmax of the exact y_ref: |y_dev - y_ref| <= half a bf16 ulp
    of y_ref plus the fp32 accumulation slack."""
    import synth
    y = synth.bf16_bits_to_f32(np.asarray(y_dev_bits).view(np.uint16)).astype(np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    slack = slack_rel * np.abs(y_ref).max(axis=-1, keepdims=True)
    err = np.abs(y - y_ref)
    bound = bf16_half_ulp(y_ref) * (1 + 1e-6) + slack
    assert np.all(err <= bound), float((err - bound).max())
    return float((err / np.maximum(np.abs(y_ref).max(axis=-1, keepdims=True), 1e-30)).max())


def check_fused_against_separate(f, g, xbits, residual: bool, label=""):
    """The fused decode layer (f) against the separate entry points (g) on the
    same input: ids and w bit for bit.  Where both run the same down kernel
    (T * k <= 16: the one-block-per-column-slice kernel over every pair) y is
    equal bit for bit too; above that the fused layer runs one slice block per
    token and sums each down dot in another fp32 order than the separate
    down kernel, so its y must be one bf16 rounding of the separate path's
    F = r + sum_i w_i o_i (fp32 slack 1e-5 of the row's max).  Returns how
    many y elements differ from the separate path's."""
    assert np.array_equal(f["ids"], g["ids"]), label
    assert np.array_equal(f["w"].view(np.uint32), g["w"].view(np.uint32)), label
    T, k = f["ids"].shape
    if T * k <= 16:
        assert np.array_equal(f["y"], g["y"]), ("fused y differs from the separate entry points", label)
        return 0
    from oracle import ffn as offn
    y_ref = offn.combine(g["out"], g["w"], xbits if residual else None)
    assert_bf16_rounding_of(f["y"], y_ref)
    return int(np.count_nonzero(f["y"] != g["y"]))


_cases = {}


def case(name, source, fmt=moe.MOE_FMT_NVFP4):
    key = (name, source, fmt)
    if key not in _cases:
        say("building layer", name, source)
        _cases[key] = LayerCase(synth.WORKLOADS[name], 0, source, fmt)
    return _cases[key]


# Sentinels written into every output buffer (and the workspace) before a
# call: a row, tile or block a kernel skipped keeps its sentinel, which no
# correct output holds (NaN floats, bf16 NaN 0xFFFF, an id outside any
# layer's range, E4M3 scale byte 0xFF, which the quantizers never produce).
SENT_ID = 0x7EADBEEF
SENT_BF16 = -1                       # int16 view of 0xFFFF


def fill_sentinels(b: dict, dbg: dict | None = None):
    nan = float("nan")
    for key in ("w", "x_ts", "out", "logits"):
        if key in b:
            b[key].fill_(nan)
    if "ids" in b:
        b["ids"].fill_(SENT_ID)
    for key in ("x_codes", "x_scales", "ws"):
        if key in b:
            b[key].fill_(0xFF)
    if "y" in b:
        b["y"].fill_(SENT_BF16)
    if dbg:
        dbg["h"].fill_(nan)
        dbg["h_ts"].fill_(nan)
        dbg["h_codes"].fill_(0xFF)
        dbg["h_scales"].fill_(0xFF)


def assert_no_sentinels(g: dict, E: int):
    """Every output element was written (g: host copies from run_layer)."""
    ids = g["ids"]
    assert not np.any(ids == SENT_ID), "ids not written"
    assert not np.isnan(g["w"]).any(), "router weights not written"
    assert not np.isnan(g["out"]).any(), "expert output rows not written"
    assert not np.any(g["y"].view(np.uint16) == 0xFFFF), "y not written"
    if "dbg_h" in g:
        assert not np.isnan(g["dbg_h"]).any(), "debug h not written"
        assert not np.isnan(g["dbg_h_ts"]).any(), "debug h^ tensor scales not written"
        assert not np.any(g["dbg_h_scales"] == 0xFF), "debug h^ block scales not written"
        bad = ~((ids >= 0) & (ids < E)).reshape(-1)
        if bad.any():                 # pairs with an id outside [0, E): zero rows
            assert not g["out"].reshape(-1, g["out"].shape[-1])[bad].any()
            assert not g["dbg_h"][bad].any() and not g["dbg_h_codes"][bad].any()
            assert not g["dbg_h_scales"][bad].any() and not g["dbg_h_ts"][bad].any()


def run_layer(c: LayerCase, xbits: np.ndarray, residual=False, prefill=False, ids_override=None, debug=True):
    """One layer on the device; debug: also request the debug copies of h and
    h^ (without them some paths take shortcuts, e.g. the 256-row GEMM coding
    h^ itself under static h scales)."""
    T = xbits.shape[0]
    L = c.L
    b = L.alloc(T, prefill=prefill)
    x = bf16_tensor(xbits, DEV)
    dbg = dict(h=torch.empty((T * L.k, L.I), dtype=torch.float32, device=DEV),
               h_codes=torch.empty((T * L.k, L.I // 2), dtype=torch.uint8, device=DEV),
               h_scales=torch.empty((T * L.k, L.I // 16), dtype=torch.uint8, device=DEV),
               h_ts=torch.empty(T * L.k, dtype=torch.float32, device=DEV)) if debug else None
    fill_sentinels(b, dbg)
    if ids_override is None:
        L.forward(x, b, residual=residual, dbg=dbg)
    else:
        moe.moe_router_topk(x, L.W_r, L.bias, T, L.d, b["ids"], b["w"], b["logits"])
        b["ids"].copy_(torch.from_numpy(ids_override).to(DEV))
        moe.moe_quantize_act(x, T, L.H, b["x_codes"], b["x_scales"], b["x_ts"])
        ffn = moe.moe_expert_ffn_prefill if prefill else moe.moe_expert_ffn_decode
        ffn(L.d, L.experts(), (b["x_codes"], b["x_scales"], b["x_ts"]), b["ids"], T, b["out"],
            b["ws"], b["ws_bytes"], dbg)
        moe.moe_combine(b["out"], b["w"], x if residual else None, T, L.k, L.H, b["y"])
    torch.cuda.synchronize()
    out = {k: t2n(v) for k, v in b.items() if isinstance(v, torch.Tensor) and k != "ws"}
    if dbg:
        out.update({"dbg_" + k: t2n(v) for k, v in dbg.items()})
    del b, dbg
    assert_no_sentinels(out, L.E)
    return out


def check_stages(c: LayerCase, xbits, g, residual=False, check_tokens=None, h_ts=None):
    """Stage-wise comparison of device outputs g (from run_layer).  h_ts:
    the static h tensor scales per expert the layer ran with, or None."""
    T, k, I = xbits.shape[0], c.L.k, c.L.I
    toks = range(T) if check_tokens is None else check_tokens
    ids = g["ids"]
    sel = np.array(list(toks))
    deq = c.oracle_deq(ids[sel])
    xq = offn.quantize_act(xbits[sel])
    # h on the device's ids
    h_ref = offn.gate_up(deq, xq, ids[sel])
    h_dev = g["dbg_h"].reshape(T, k, I)[sel]
    rel_h = rowwise_rel(h_dev, h_ref)
    assert rel_h.max() <= 1e-5, rel_h.max()
    # h^ bit-exact from the device's h
    ts_rows = None if h_ts is None else np.asarray(h_ts, np.float32)[ids[sel]].reshape(-1)
    hc, hs, hts = offn.quantize_h(h_dev, ts_rows)
    dc = g["dbg_h_codes"].reshape(T, k, I // 2)[sel].reshape(-1, I // 2)
    ds = g["dbg_h_scales"].reshape(T, k, I // 16)[sel].reshape(-1, I // 16)
    dts = g["dbg_h_ts"].reshape(T, k)[sel].reshape(-1)
    assert np.array_equal(dc, nvfp4.pack_nibbles(hc))
    assert np.array_equal(ds, hs)
    assert np.array_equal(dts.view(np.uint32), hts.astype(np.float32).view(np.uint32))
    # o from the device's h^
    o_ref = offn.down(deq, (hc, hs, hts), ids[sel])
    o_dev = g["out"][sel]
    rel_o = rowwise_rel(o_dev, o_ref)
    assert rel_o.max() <= 2e-3, rel_o.max()
    # pure oracle o (its own h^): rows whose h^ agrees must match
    hq_pure = offn.quantize_h(h_ref, ts_rows)
    o_pure = offn.down(deq, hq_pure, ids[sel])
    same = np.all(nvfp4.pack_nibbles(hq_pure[0]) == dc, axis=1) & np.all(hq_pure[1] == hs, axis=1)
    rel_p = rowwise_rel(o_dev, o_pure)
    assert np.all(rel_p[same] <= 2e-3)
    # y from the device's o and w
    y_ref = offn.combine(g["out"][sel], g["w"][sel], xbits[sel] if residual else None)
    rel_y = assert_bf16_rounding_of(g["y"][sel], y_ref)
    return dict(rel_h=rel_h.max(), rel_o=rel_o.max(), flips=float((~same).mean()), rel_y=rel_y)




def pick_experts(ids: np.ndarray, E: int, tile_rows: int) -> list:
    """Experts whose every (t, slot) row is compared in the full-size prefill
    tests: the one with the most rows (many row tiles), the ones whose last
    row tile is the shortest and the fullest ragged tile, the lowest, middle
    and highest active ids (their tiles sit in different XCDs' block ranges),
    under skewed routing a tail expert with one to three rows, and on the
    256-row tiling the largest expert that takes 32-row tiles instead."""
    counts = np.bincount(ids.reshape(-1), minlength=E)[:E]
    act = np.nonzero(counts)[0]
    chosen = {int(counts.argmax()), int(act.min()), int(act.max()), int(act[len(act) // 2])}
    rem = counts % tile_rows
    cand = act[(counts[act] > tile_rows) & (rem[act] > 0)]
    if len(cand):
        chosen.add(int(cand[np.argmin(rem[cand])]))
        chosen.add(int(cand[np.argmax(rem[cand])]))
    small = act[counts[act] <= 3]
    if len(small):
        chosen.add(int(small[0]))
    if tile_rows == 256:
        # the 256-row tiling hands experts below 128 rows to 32-row tiles:
        # the largest such expert (several of them, a ragged last one)
        tail = act[(counts[act] < 128) & (counts[act] > 32)]
        if len(tail):
            chosen.add(int(tail[np.argmax(counts[tail])]))
    return sorted(chosen)


def check_pairs(c: LayerCase, xbits, g, pairs, h_ts=None):
    """Stage-wise comparison on the (t, slot) pairs with flat index
    t * k + slot in `pairs` (every pair must have a valid id): h against the
    oracle on the device's ids (row-wise <= 1e-5), h^ bit-exact from the
    device's h, o against the oracle's down projection of the device's h^
    (row-wise <= 2e-3), and against the pure oracle on rows whose h^ agrees."""
    k = c.L.k
    pairs = np.asarray(pairs, dtype=np.int64)
    e_sel = g["ids"].reshape(-1)[pairs]
    assert np.all((e_sel >= 0) & (e_sel < c.wl.E))
    toks = pairs // k
    deq = c.oracle_deq(e_sel)
    ids1 = e_sel.reshape(-1, 1)
    xq = offn.quantize_act(xbits[toks])                       # one x^ row per pair
    h_ref = offn.gate_up(deq, xq, ids1)[:, 0]
    h_dev = g["dbg_h"][pairs]
    rel_h = rowwise_rel(h_dev, h_ref)
    assert rel_h.max() <= 1e-5, rel_h.max()
    ts_rows = None if h_ts is None else np.asarray(h_ts, np.float32)[e_sel]
    hc, hs, hts = offn.quantize_h(h_dev, ts_rows)
    dc, ds, dts = g["dbg_h_codes"][pairs], g["dbg_h_scales"][pairs], g["dbg_h_ts"][pairs]
    assert np.array_equal(dc, nvfp4.pack_nibbles(hc))
    assert np.array_equal(ds, hs)
    assert np.array_equal(dts.view(np.uint32), hts.astype(np.float32).view(np.uint32))
    o_ref = offn.down(deq, (hc, hs, hts), ids1)[:, 0]
    o_dev = g["out"].reshape(-1, c.L.H)[pairs]
    rel_o = rowwise_rel(o_dev, o_ref)
    assert rel_o.max() <= 2e-3, rel_o.max()
    hq_pure = offn.quantize_h(h_ref, ts_rows)
    o_pure = offn.down(deq, hq_pure, ids1)[:, 0]
    same = np.all(nvfp4.pack_nibbles(hq_pure[0]) == dc, axis=1) & np.all(hq_pure[1] == hs, axis=1)
    rel_p = rowwise_rel(o_dev, o_pure)
    assert np.all(rel_p[same] <= 2e-3)
    return dict(pairs=len(pairs), rel_h=float(rel_h.max()), rel_o=float(rel_o.max()),
                flips=float((~same).mean()))


def check_y_all(g, xbits, residual: bool, chunk: int = 2048) -> float:
    """Every token's y against the oracle combine of the device's o and w:
    one bf16 rounding of the fp32 slot-order sum."""
    T = g["y"].shape[0]
    worst = 0.0
    for t0 in range(0, T, chunk):
        sl = slice(t0, min(T, t0 + chunk))
        y_ref = offn.combine(g["out"][sl], g["w"][sl], xbits[sl] if residual else None)
        worst = max(worst, assert_bf16_rounding_of(g["y"][sl], y_ref))
    return worst
