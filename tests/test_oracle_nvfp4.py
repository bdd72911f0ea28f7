"""Pins for oracle.nvfp4: the NVFP4 quantizer against an exact-rational brute
force, closed-form invariants and the integer special case of the W4A4 dot."""
import numpy as np
import pytest

from oracle import nvfp4, formats
from tests import brute


def _rows(seed, R, K):
    r = np.random.default_rng(seed)
    v = r.standard_normal((R, K)).astype(np.float32)
    v[0, :16] = 0.0                                   # an all-zero block
    v[0, 16:32] = -0.0                                # negative zeros
    if R > 1:
        v[1] *= 1e-3                                  # small row
        v[1, 5] = 7.5                                 # one outlier
    if R > 2:
        v[2, :] = 0.37                                # all equal
    if R > 3:
        v[3, 40] = 1e-30                              # tiny with large amax
        v[3, 41] = -1e-30
    if R > 4:
        v[4, -1] = -9.0                               # row max in the last element
    return v


@pytest.mark.parametrize("per_row", [True, False])
def test_quantizer_matches_exact_brute_force(per_row):
    v = _rows(10, 6, 64)
    codes, scales, ts = nvfp4.quantize(v, per_row=per_row)
    bc, bs, bts = brute.quantize_rows(v, per_row=per_row)
    assert np.array_equal(codes, bc)
    assert np.array_equal(scales, bs)
    ts_list = list(ts) if per_row else [ts] * v.shape[0]
    for a, b in zip(ts_list, bts):
        assert float(a) == float(b)


def test_quantizer_brute_force_wide_dynamic_range():
    r = np.random.default_rng(11)
    v = (r.standard_normal((4, 128)) * np.exp2(r.integers(-20, 20, (4, 128)))).astype(np.float32)
    for per_row in (True, False):
        codes, scales, _ = nvfp4.quantize(v, per_row=per_row)
        bc, bs, _ = brute.quantize_rows(v, per_row=per_row)
        assert np.array_equal(codes, bc) and np.array_equal(scales, bs)


def test_quantizer_brute_force_weight_matrix():
    """A whole gate matrix of the tiny layer (one tensor scale)."""
    import synth
    wl = synth.WORKLOADS["tiny"]
    gate, _, _ = synth.expert_weights(wl, 0, 3)
    sub = gate[:24]                        # brute force is slow: 24 rows x 256
    # per-matrix scope of the full matrix: inject the full amax into the rows
    codes, scales, ts = nvfp4.quantize(gate, per_row=False)
    bc, bs, bts = brute.quantize_rows(np.concatenate([sub, gate[np.abs(gate).max(1).argmax()][None]]), per_row=False)
    assert float(bts[0]) == float(ts)
    assert np.array_equal(codes[:24], bc[:24]) and np.array_equal(scales[:24], bs[:24])


def test_round_trip_of_representable_values():
    r = np.random.default_rng(12)
    R, K = 8, 256
    codes = r.integers(0, 16, (R, K)).astype(np.uint8)
    scales = r.integers(1, 0x7F, (R, K // 16)).astype(np.uint8)
    ts = np.float32(0.015625)                       # power of two: products exact
    # choose block scales and codes so every block's max |value| sets its
    # scale exactly: element 0 of each block has magnitude 6 (code 7)
    codes[:, ::16] = 7
    scales[0, 0] = 0x7E                             # one element at 6*448*ts = amax
    v = nvfp4.dequantize(codes, scales, ts).astype(np.float32)
    c2, s2, ts2 = nvfp4.quantize(v, per_row=False)
    assert ts2 == ts
    assert np.array_equal(s2, scales)
    # -0 elements (code 8) keep their sign bit; +0 stays 0
    assert np.array_equal(c2, codes)


def test_zero_input():
    c, s, ts = nvfp4.quantize(np.zeros((3, 64), np.float32), per_row=True)
    assert not c.any() and not s.any() and not np.any(ts)
    c, s, ts = nvfp4.quantize(np.zeros((3, 64), np.float32), per_row=False)
    assert not c.any() and not s.any() and ts == 0


@pytest.mark.parametrize("j", [-8, -1, 1, 5])
def test_power_of_two_scaling(j):
    v = np.random.default_rng(13).standard_normal((5, 128)).astype(np.float32)
    c1, s1, t1 = nvfp4.quantize(v, per_row=True)
    c2, s2, t2 = nvfp4.quantize((v * np.float32(2.0 ** j)).astype(np.float32), per_row=True)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert np.array_equal(t2, (t1 * np.float32(2.0 ** j)).astype(np.float32))


def test_sign_symmetry():
    v = np.random.default_rng(14).standard_normal((5, 128)).astype(np.float32)
    c1, s1, t1 = nvfp4.quantize(v, per_row=True)
    c2, s2, t2 = nvfp4.quantize(-v, per_row=True)
    assert np.array_equal(s1, s2) and np.array_equal(t1, t2)
    assert np.array_equal(c2, c1 ^ 8)


def test_block_scale_covers_block_max():
    """Every block's largest element encodes at magnitude 4 or 6 (codes 6/7)
    unless the block scale saturated or underflowed."""
    v = np.random.default_rng(15).standard_normal((16, 256)).astype(np.float32)
    c, s, ts = nvfp4.quantize(v, per_row=True)
    blocks = np.abs(v).reshape(16, 16, 16)
    arg = blocks.argmax(-1)
    top = np.take_along_axis(c.reshape(16, 16, 16), arg[..., None], -1)[..., 0] & 7
    assert np.all(np.isin(top, [6, 7]))
    # dequantized error bounded by half an E2M1 step at the top of the grid
    d = nvfp4.dequantize(c, s, ts)
    err = np.abs(d - v).reshape(16, 16, 16).max(-1)
    assert np.all(err <= blocks.max(-1) * 0.2 + 1e-6)


def test_nibble_order():
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 8]], np.uint8)
    p = nvfp4.pack_nibbles(codes)
    assert list(p[0]) == [0x21, 0x43, 0x65, 0x87]
    assert np.array_equal(nvfp4.unpack_nibbles(p), codes)


def test_w4a4_dot_integer_special_case():
    """All block scales 1.0 (0x38) and tensor scales 1: the dot is exactly a
    quarter of the integer dot of A = 2*e2m1."""
    r = np.random.default_rng(16)
    N, K = 32, 512
    cw = r.integers(0, 16, (N, K)).astype(np.uint8)
    cx = r.integers(0, 16, (3, K)).astype(np.uint8)
    ones_w = np.full((N, K // 16), 0x38, np.uint8)
    ones_x = np.full((3, K // 16), 0x38, np.uint8)
    W = nvfp4.dequantize(cw, ones_w, np.float32(1))
    X = nvfp4.dequantize(cx, ones_x, np.float32(1))
    A = {c: int(round(2 * formats.e2m1_decode(np.array([c]))[0])) for c in range(16)}
    Aw = np.vectorize(A.get)(cw).astype(np.int64)
    Ax = np.vectorize(A.get)(cx).astype(np.int64)
    assert np.array_equal(X @ W.T, (Ax @ Aw.T) / 4.0)


def test_expert_bytes():
    assert nvfp4.expert_bytes(2560, 640) == 2_764_800
    assert nvfp4.expert_bytes(256, 128) == 55_296


def test_closed_form_ties_in_scale_and_codes():
    """Exact ties, built by hand from the definition.  amax = 168 gives
    ts = 168/2688 = 2^-4 and 6*ts = 0.375 (both exact).
    Block 1: max 0.375 * 1.1875 -> ratio 1.1875, the midpoint of E4M3 1.125
    (0x39) and 1.25 (0x3A): ties to the even code 0x3A.
    Block 2: max 0.375 -> scale 1.0 (0x38), d = 2^-4; elements at the E2M1
    midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 (times d) round to the even
    codes 0, 2, 2, 4, 4, 6, 6; 6.5*d saturates to code 7 ... but 6.5*d > block
    max is impossible, so the block max itself (6*d) gives code 7."""
    d = 2.0 ** -4
    v = np.zeros((1, 48), np.float32)
    v[0, 0] = 168.0
    v[0, 16] = 0.375 * 1.1875
    v[0, 32:40] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]) * d
    v[0, 40] = -0.25 * d
    codes, scales, ts = nvfp4.quantize(v, per_row=True)
    assert ts[0] == np.float32(2.0 ** -4)
    assert scales[0, 1] == 0x3A
    assert scales[0, 2] == 0x38
    assert list(codes[0, 32:41]) == [0, 2, 2, 4, 4, 6, 6, 7, 8]


def test_scale_rounding_order_cases():
    """Blocks where the order of the scale arithmetic decides the E4M3 code:
    ab / (6*ts) with 6*ts rounded first differs from (ab/6)/ts.  The cases are
    found by a seeded search in plain fp32 (torch's E4M3 conversion picks the
    codes) and then checked against the exact-rational brute force."""
    import torch
    r = np.random.default_rng(17)
    n = 200_000
    amax = np.exp2(r.uniform(-6, 6, n)).astype(np.float32)
    ts = (amax / np.float32(2688)).astype(np.float32)
    # aim ab at E4M3 midpoints m (codes 0x20..0x6F) so the ratio lands within
    # a few fp32 ulps of a tie
    grid = torch.arange(0x20, 0x71, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = (grid[:-1] + grid[1:]) / 2
    m = mids[r.integers(0, len(mids), n)]
    ab = (m * (np.float32(6) * ts)).astype(np.float32)
    ab = (ab.view(np.int32) + r.integers(-3, 4, n).astype(np.int32)).view(np.float32)
    ab = np.minimum(ab, amax)
    r1 = (ab / (np.float32(6) * ts)).astype(np.float32)
    r2 = ((ab / np.float32(6)) / ts).astype(np.float32)
    c1 = torch.from_numpy(np.minimum(r1, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    c2 = torch.from_numpy(np.minimum(r2, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    idx = np.nonzero(c1 != c2)[0][:12]
    assert len(idx) >= 4
    v = np.zeros((len(idx), 32), np.float32)
    v[:, 0] = amax[idx]
    v[:, 16] = ab[idx]
    codes, scales, _ = nvfp4.quantize(v, per_row=True)
    bc, bs, _ = brute.quantize_rows(v, per_row=True)
    assert np.array_equal(scales, bs) and np.array_equal(codes, bc)


def test_element_rounding_near_e2m1_midpoints():
    """Elements aimed within a few fp32 ulps of E2M1 midpoints times the
    block's d, with d carrying many significant bits, so that the rounding of
    v / d decides the code; checked against the exact brute force."""
    r = np.random.default_rng(18)
    rows = []
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for _ in range(24):
        amax = np.float32(np.exp2(r.uniform(-4, 4)))
        ts = np.float32(amax / np.float32(2688))
        row = np.zeros(32, np.float32)
        row[0] = amax
        # block 1: its max sets scale sb; d = E4M3(sb) * ts (fp32)
        bmax = np.float32(amax * np.float32(r.uniform(0.05, 0.9)))
        row[16] = bmax
        ratio = np.float32(bmax / np.float32(np.float32(6) * ts))
        sb = torch_e4m3(ratio)
        d = np.float32(np.float32(e4m3_val(sb)) * ts)
        m = mids[r.integers(0, len(mids), 15)]
        el = (m * d).astype(np.float32)
        el = (el.view(np.int32) + r.integers(-2, 3, 15).astype(np.int32)).view(np.float32)
        row[17:32] = np.minimum(el, bmax) * np.where(r.random(15) < 0.5, -1, 1).astype(np.float32)
        rows.append(row)
    v = np.stack(rows)
    codes, scales, _ = nvfp4.quantize(v, per_row=True)
    bc, bs, _ = brute.quantize_rows(v, per_row=True)
    assert np.array_equal(scales, bs) and np.array_equal(codes, bc)


def torch_e4m3(x):
    import torch
    return int(torch.tensor([float(min(x, 448))]).to(torch.float8_e4m3fn).view(torch.uint8)[0])


def e4m3_val(c):
    import torch
    return float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


def test_static_tensor_scale_brute_force():
    """Static (calibrated) per-row tensor scales: equal to the brute force for
    scales below (saturating blocks), at and above each row's own amax/2688."""
    v = _rows(12, 6, 64)
    own = nvfp4.quantize(v, per_row=True)[2]
    for f in (0.05, 1.0, 3.7):
        ts = (own * np.float32(f)).astype(np.float32)
        ts[0] = np.float32(0.01)                      # a row whose own ts is small
        codes, scales, ts_out = nvfp4.quantize(v, per_row=True, ts_given=ts)
        bc, bs, _ = brute.quantize_rows(v, per_row=True, ts_given=ts)
        assert np.array_equal(codes, bc) and np.array_equal(scales, bs)
        assert np.array_equal(ts_out.view(np.uint32), ts.view(np.uint32))


def test_static_tensor_scale_equals_dynamic_at_own_scale():
    v = _rows(13, 5, 128)
    c0, s0, t0 = nvfp4.quantize(v, per_row=True)
    c1, s1, t1 = nvfp4.quantize(v, per_row=True, ts_given=t0)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


def test_static_tensor_scale_worked_block():
    """One block [1, 0, ..., 0] with ts = 1/448 (fp32): 1 / (6 ts) = 74.67 rounds
    to the E4M3 value 72 (exponent 6, mantissa 1/8: code 0x69), d = 72 ts =
    0.1607..., 1 / d = 6.22 rounds to the E2M1 value 6 (code 7).  Saturation:
    a value 1e6 with the same ts takes block scale 448 (0x7E) and code 7."""
    v = np.zeros((2, 16), np.float32)
    v[0, 0] = 1.0
    v[1, 3] = -1e6
    ts = np.full(2, np.float32(1.0) / np.float32(448.0), np.float32)
    codes, scales, _ = nvfp4.quantize(v, per_row=True, ts_given=ts)
    assert scales[0, 0] == 0x69 and codes[0, 0] == 7 and not codes[0, 1:].any()
    assert scales[1, 0] == 0x7E and codes[1, 3] == 0x8 | 7
