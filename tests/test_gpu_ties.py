"""GPU parity at exact rounding ties of the NVFP4 quantizer, with block
scales that are not powers of two: element quotients exactly halfway between
two E2M1 magnitudes and block-scale ratios exactly halfway between two E4M3
values, for the activation quantizer (moe_quantize_act and the fused decode
layer's copy), the weight quantizer and the h^ quantizers of every FFN path
(the decode kernels at one and three tokens, the 32-, 128- and 256-row
grouped GEMMs; dynamic and static h scales).  Bit-exact against the oracle;
each test also counts the exact ties it hit."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import synth
import quantized_moe_routed_router_amd as moe
from oracle import ffn as offn, nvfp4
from tests import ties
from tests.gpu_helpers import say, t2n, bf16_tensor, run_layer, check_pairs, check_y_all
from tests.test_gpu_quant import _check_act

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_act_quant_exact_ties():
    v = ties.act_tie_rows(40, 2560, seed=41)
    xbits = synth.f32_to_bf16_bits(v)
    _, s, ts = offn.quantize_act(xbits)
    el, sc = ties.count_ties(v, s, ts)
    say("act quant ties: element", el, "scale", sc)
    assert el >= 5000 and sc >= 300
    _check_act(xbits)


def test_weight_quant_exact_ties():
    for seed, (rows, cols) in ((42, (64, 256)), (43, (160, 640)), (44, (32, 2560))):
        W = ties.weight_tie_matrix(rows, cols, seed)
        oc, os_, ots = nvfp4.quantize(W, per_row=False)
        el, sc = ties.count_ties(W, os_, ots)
        assert el >= 2000 and sc >= 100, (el, sc)
        Wd = torch.from_numpy(W[None]).to(DEV)
        codes = torch.empty((1, rows, cols // 2), dtype=torch.uint8, device=DEV)
        scales = torch.empty((1, rows, cols // 16), dtype=torch.uint8, device=DEV)
        ts = torch.empty(1, dtype=torch.float32, device=DEV)
        moe.moe_quantize_weights(Wd, 1, rows, cols, codes, scales, ts)
        torch.cuda.synchronize()
        assert np.array_equal(t2n(codes)[0], nvfp4.pack_nibbles(oc))
        assert np.array_equal(t2n(scales)[0], os_)
        assert np.float32(t2n(ts)[0]).view(np.uint32) == np.float32(ots).view(np.uint32)
        say("weight quant ties", rows, cols, "element", el, "scale", sc)


class TieCase:
    """A tiny layer (H 256, E 16, k 2) whose h rows are 64 N exactly, built
    from the fp32 weights of tests.ties.tie_layer; the oracle quantizes the
    same fp32 weights."""

    def __init__(self, I: int, mode: str, seed: int):
        H, E, k = 256, 16, 2
        self.wl = SimpleNamespace(E=E, H=H, I=I, k=k)
        self.N = ties.h_pattern(I, mode, seed)
        self.gate, self.up, self.down, self.xrow = ties.tie_layer(H, I, E, self.N, seed + 1)
        self.L = moe.Layer(E, H, I, k, device=DEV)
        r = np.random.default_rng(seed + 2)
        self.L.set_router(torch.from_numpy((r.standard_normal((E, H)) * 0.05).astype(np.float32)).to(DEV))
        self.L.load_experts_fp32(0, torch.from_numpy(self.gate).to(DEV), torch.from_numpy(self.up).to(DEV),
                                 torch.from_numpy(self.down).to(DEV))
        self.h_ts = np.full(E, 6.0, np.float32) if mode == "static" else None
        self.L.set_static_h_scales(None if self.h_ts is None else torch.from_numpy(self.h_ts).to(DEV))
        torch.cuda.synchronize()
        self._deq = {}

    def oracle_deq(self, experts):
        for e in np.unique(experts):
            e = int(e)
            if e not in self._deq:
                self._deq[e] = offn.dequant_expert(offn.quantize_expert(self.gate[e], self.up[e], self.down[e]))
        return {int(e): self._deq[int(e)] for e in np.unique(experts)}


@pytest.mark.parametrize("I", [128, 256])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_h_quant_exact_ties(I, mode):
    """h = 64 N exactly on the device, then h^ bit-exact with the oracle on
    every path; the tie counts are asserted so the test cannot drift off the
    ties.  Paths: decode one token (dynamic: the down kernel quantizes; static:
    the gate/up kernel), decode three tokens (the h^ kernel), prefill 4 and 300
    tokens (32-row tiles; split K at 4) and 800 tokens (128-row tiles at I 128,
    256-row tiles at I 256); the fused layer equals the separate entry points."""
    c = TieCase(I, mode, seed=60 + I)
    k, E = c.wl.k, c.wl.E
    h_exact = (64 * c.N).astype(np.float32)
    r = np.random.default_rng(7)
    for T, prefill in ((1, False), (3, False), (4, True), (300, True), (800, True)):
        x = synth.f32_to_bf16_bits(np.tile(c.xrow, (T, 1)))
        ids = np.stack([r.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        if prefill:
            expect = 32 if T <= 300 else (256 if I == 256 else 128)
            assert moe.moe_ffn_prefill_tile_rows(c.L.d, T) == expect
        g = run_layer(c, x, prefill=prefill, residual=True, ids_override=ids)
        assert np.array_equal(g["dbg_h"], np.broadcast_to(h_exact, g["dbg_h"].shape)), "h is not 64 N"
        hs = g["dbg_h_scales"][:1]
        el, sc = ties.count_ties(g["dbg_h"][:1], hs, g["dbg_h_ts"][:1])
        assert el >= 40 and (mode == "dynamic" or sc >= 2), (el, sc)
        n = T * k if T <= 4 else 64
        st = check_pairs(c, x, g, np.arange(n), h_ts=c.h_ts)
        check_y_all(g, x, residual=True)
        say("h ties", mode, "I", I, "T", T, "prefill" if prefill else "decode", "ties", el, sc, st)
        if T in (1, 3):
            fb = c.L.alloc_fused(T)
            fb["ws"].fill_(0xFF)
            # the fused layer routes by itself: compare it with the separate
            # entry points on its own ids
            c.L.forward_fused(bf16_tensor(x, DEV), fb, residual=True)
            torch.cuda.synchronize()
            g2 = run_layer(c, x, residual=True, ids_override=t2n(fb["ids"]))
            assert np.array_equal(t2n(fb["y"]), g2["y"])


def test_fused_layer_act_ties():
    """The fused decode layer quantizes x with its own block routine: on tie
    rows it gives the same ids, weights and y as the separate entry points
    (which use moe_quantize_act, checked bit-exact above)."""
    from tests.gpu_helpers import case
    c = case("tiny", "host")
    x = synth.f32_to_bf16_bits(ties.act_tie_rows(4, 256, seed=45))
    for T in (1, 4):
        fb = c.L.alloc_fused(T)
        fb["ws"].fill_(0xFF)
        c.L.forward_fused(bf16_tensor(x[:T], DEV), fb, residual=True)
        torch.cuda.synchronize()
        g = run_layer(c, x[:T], residual=True)
        assert np.array_equal(t2n(fb["ids"]), g["ids"])
        assert np.array_equal(t2n(fb["w"]).view(np.uint32), g["w"].view(np.uint32))
        assert np.array_equal(t2n(fb["y"]), g["y"])
