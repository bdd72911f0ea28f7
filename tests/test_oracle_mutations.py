"""Planted mistakes in the oracle (CPU only): each mutant changes one step of
an oracle function (its source copied, one expression replaced, patched in
for the test's duration) and one of the oracle's pins must then fail.  This
is the evidence that the pins would catch such a mistake: a wrong divisor, a
tie broken the wrong way, a rounding order, a dropped sign, a swapped operand,
a reversed bit, nibble, group or row order, a wrong tie-break, softmax or bias
sign, an unstable sort, a wrong table value, an ignored static scale, a
dropped residual, a wrong RMS.  Nothing here touches the GPU."""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import codebook, ffn, formats, nvfp4, permute, router, stack
from tests import (test_oracle_codebook as pc, test_oracle_ffn as pf, test_oracle_formats as pfo,
                   test_oracle_nvfp4 as pn, test_oracle_permute as pp, test_oracle_router as pr,
                   test_oracle_stack as ps)
import synth


def _mutant(monkeypatch, module, name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, name)))
    assert old in src, (name, old)
    g = dict(module.__dict__)
    exec(compile(src.replace(old, new, 1), f"<mutant of {module.__name__}.{name}>", "exec"), g)
    monkeypatch.setattr(module, name, g[name])


def _tiny():
    wl = synth.WORKLOADS["tiny"]
    x = synth.activations(wl)
    W_r = synth.router_weights(wl)
    experts = {e: ffn.quantize_expert(*synth.expert_weights(wl, 0, e)) for e in range(wl.E)}
    return wl, x, W_r, experts, ffn.layer(x, W_r, None, experts, wl.k)


MUTANTS = [
    # (id, module, function, old, new, pin)
    ("tensor-scale divisor", nvfp4, "quantize",
     "amax / TS_DIVISOR", "amax / np.float32(2687.0)",
     lambda: pn.test_quantizer_matches_exact_brute_force(True)),
    ("scale ratio rounding order", nvfp4, "quantize",
     "ratio = (ab / six_ts[:, None]).astype(np.float32)",
     "ratio = ((ab / np.float32(6.0)) / ts_rows[:, None]).astype(np.float32)",
     pn.test_scale_rounding_order_cases),
    ("element quotient as v * (1/d)", nvfp4, "quantize",
     "q = (blocks / d[:, :, None]).astype(np.float32)",
     "q = (blocks * (np.float32(1.0) / d)[:, :, None]).astype(np.float32)",
     pn.test_element_rounding_near_e2m1_midpoints),
    ("sign of -0 dropped", nvfp4, "quantize",
     "sign = np.signbit(blocks).astype(np.int64)", "sign = (blocks < 0).astype(np.int64)",
     pn.test_round_trip_of_representable_values),
    ("ties to the odd code", formats, "round_to_grid_even",
     "(hi_c % 2 == 0)", "(hi_c % 2 == 1)",
     pn.test_closed_form_ties_in_scale_and_codes),
    ("E4M3 subnormal exponent", formats, "e4m3_decode",
     "m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7",
     pfo.test_e4m3_table_all_256_codes_vs_bitfields_and_torch),
    ("nibble order", nvfp4, "pack_nibbles",
     "(c[:, 0::2] | (c[:, 1::2] << 4))", "(c[:, 1::2] | (c[:, 0::2] << 4))",
     pn.test_nibble_order),
    ("router ties to the higher id", router, "topk",
     "np.lexsort((e_idx, -l), axis=1)", "np.lexsort((-e_idx, -l), axis=1)",
     pr.test_constant_logits_ties_to_lower_ids),
    ("softmax exponent sign", router, "topk",
     "z = np.exp(sel - sel[:, :1])", "z = np.exp(sel[:, :1] - sel)",
     pr.test_renormalised_topk_equals_full_softmax_restricted),
    ("SiLU sign", ffn, "silu",
     "z / (1.0 + np.exp(-z))", "z / (1.0 + np.exp(z))",
     pf.test_silu_closed_form),
    ("gate and up swapped", ffn, "gate_up",
     "h[rows] = silu(g) * u", "h[rows] = silu(u) * g",
     lambda: pf.test_dense_layer_exact_brute_force(_tiny())),
    ("combine without the router weights", ffn, "combine",
     'y = np.einsum("tk,tkh->th", w, o)', "y = o.sum(axis=1)",
     pf.test_layer_combines_in_fp64_and_rounds_once),
    ("unstable permutation", permute, "permute",
     'perm = np.argsort(flat, kind="stable").astype(np.int32)',
     'perm = (flat.size - 1 - np.argsort(flat[::-1], kind="stable")[::-1]).astype(np.int32)',
     lambda: pp.test_permute_vs_loop(37, 3, 8, 1)),
    ("codebook index bit order", codebook, "pack_indices",
     'bitorder="little"', 'bitorder="big"',
     pc.test_pack_round_trip_and_bit_order),
    ("codebook groups in reverse order", codebook, "dequantize",
     "g = np.arange(K) // GROUP", "g = (K // GROUP - 1) - np.arange(K) // GROUP",
     pc.test_dequant_is_table_lookup),
    ("E2M1 magnitude 1.5 read as 1.25", formats, "e2m1_decode",
     "mag = E2M1_MAGNITUDES[c & 7]", "mag = np.where((c & 7) == 3, 1.25, E2M1_MAGNITUDES[c & 7])",
     pfo.test_e2m1_table_all_16_codes),
    ("static tensor scale ignored", nvfp4, "quantize",
     "if ts_given is not None:", "if False:",
     pn.test_static_tensor_scale_brute_force),
    ("router bias subtracted", router, "logits",
     "l = l + np.asarray(bias", "l = l - np.asarray(bias",
     pr.test_bias_shifts_logits),
    ("combine without the residual", ffn, "combine",
     "y = y + bf16_bits_to_f64(residual_bits)", "y = y + 0.0 * bf16_bits_to_f64(residual_bits)",
     pf.test_zero_input_gives_residual),
    ("down projection rows reversed", ffn, "down",
     "o[rows] = hd[rows] @ Wd.T", "o[rows] = hd[rows] @ Wd[::-1].T",
     lambda: pf.test_dense_layer_exact_brute_force(_tiny())),
    ("stack RMS from the mean absolute value", stack, "rms_norm",
     "ms = np.mean(x * x, axis=-1, keepdims=True)", "ms = np.mean(np.abs(x), axis=-1, keepdims=True) ** 2",
     ps.test_output_rms_and_power_of_two_invariance),
]


@pytest.mark.parametrize("mid", [m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, mid):
    _, module, name, old, new, pin = next(m for m in MUTANTS if m[0] == mid)
    pin()                                           # passes on the oracle as written
    _mutant(monkeypatch, module, name, old, new)
    with pytest.raises(AssertionError):
        pin()
