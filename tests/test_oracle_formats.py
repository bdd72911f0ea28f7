"""Pins for oracle.formats: E2M1 / E4M3 tables and encoders, bf16 rounding.

Checked against the bit-field definitions (tests/brute.py), torch's own
float8_e4m3fn and bfloat16 conversions, and exhaustive nearest-code search.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import brute


def test_e2m1_table_all_16_codes():
    vals = F.e2m1_decode(np.arange(16))
    for c in range(16):
        assert Fraction(float(vals[c])) == brute.e2m1_value(c)
    assert list(vals[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(vals[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert np.signbit(vals[8])


def test_e4m3_table_all_256_codes_vs_bitfields_and_torch():
    vals = F.e4m3_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            assert np.isnan(vals[c]) and np.isnan(ref[c])
            continue
        assert Fraction(float(vals[c])) == brute.e4m3_value(c)
        assert vals[c] == ref[c]
    assert vals[0x38] == 1.0 and vals[0x7E] == 448.0 and vals[0x01] == 2.0 ** -9
    assert vals[0x08] == 2.0 ** -6 and vals[0x07] == 7 * 2.0 ** -9
    assert np.all(np.diff(F.E4M3_GRID) > 0)          # codes 0..0x7E increasing


def test_e2m1_encode_interval_table():
    # Intervals of round-to-nearest-even on {0,.5,1,1.5,2,3,4,6}, saturating.
    table = [((0.0, True), (0.25, True), 0), ((0.25, False), (0.75, False), 1),
             ((0.75, True), (1.25, True), 2), ((1.25, False), (1.75, False), 3),
             ((1.75, True), (2.5, True), 4), ((2.5, False), (3.5, False), 5),
             ((3.5, True), (5.0, True), 6), ((5.0, False), (1e30, True), 7)]
    for (lo, lo_in), (hi, hi_in), code in table:
        pts = [lo, hi, np.nextafter(np.float32(lo), np.float32(np.inf)),
               np.nextafter(np.float32(hi), np.float32(0)), (lo + min(hi, 100)) / 2]
        for p in pts:
            p = np.float32(p)
            inside = (p > lo or (p == lo and lo_in)) and (p < hi or (p == hi and hi_in))
            if inside:
                assert F.e2m1_encode_magnitude(p) == code, (p, code)
    # exhaustive agreement with nearest-even enumeration on random fp32
    r = np.random.default_rng(1)
    xs = np.concatenate([r.uniform(0, 8, 3000), r.uniform(0, 1, 1000)]).astype(np.float32)
    got = F.e2m1_encode_magnitude(xs)
    for x, g in zip(xs, got):
        assert g == brute.e2m1_encode(Fraction(float(x)))


def test_e4m3_encode_round_trip_midpoints_saturation():
    codes = np.arange(0x7F)
    assert np.array_equal(F.e4m3_encode_nonneg(F.e4m3_decode(codes)), codes)
    grid = F.E4M3_GRID
    mids = (grid[:-1] + grid[1:]) / 2                   # exact in fp32
    got = F.e4m3_encode_nonneg(mids.astype(np.float32))
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    assert F.e4m3_encode_nonneg(np.float32(448.0)) == 0x7E
    assert F.e4m3_encode_nonneg(np.float32(1e9)) == 0x7E
    assert F.e4m3_encode_nonneg(np.float32(2.0 ** -10)) == 0      # tie 0 / 2^-9
    assert F.e4m3_encode_nonneg(np.float32(2.0 ** -10 * 1.0001)) == 1


def test_e4m3_encode_matches_torch_below_448():
    r = np.random.default_rng(2)
    xs = np.concatenate([
        np.exp2(r.uniform(-12, np.log2(448), 20000)),
        r.uniform(0, 2.0 ** -6, 5000),
        (F.E4M3_GRID[:-1] + F.E4M3_GRID[1:]) / 2,
    ]).astype(np.float32)
    xs = xs[xs <= 448]
    mine = F.e4m3_encode_nonneg(xs)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref.astype(np.int64))


def test_e4m3_encode_vs_enumeration():
    r = np.random.default_rng(3)
    xs = np.exp2(r.uniform(-11, 9.5, 600)).astype(np.float32)
    got = F.e4m3_encode_nonneg(xs)
    for x, g in zip(xs, got):
        assert g == brute.e4m3_encode(Fraction(float(x)))


def test_bf16_helpers_vs_torch():
    r = np.random.default_rng(4)
    a = (r.standard_normal(20000) * np.exp2(r.uniform(-30, 30, 20000)))
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # values that are already fp32 round once
    assert np.array_equal(F.f64_to_bf16_bits(a.astype(np.float32).astype(np.float64)), ref)
    # fp64 values: compare against exact rounding computed with Fractions
    for v in a[:300]:
        bits = int(F.f64_to_bf16_bits(np.array([v]))[0])
        got = Fraction(float(F.bf16_bits_to_f64(np.array([bits], np.uint16))[0]))
        q = Fraction(float(v))
        # neighbours on the bf16 grid
        b_lo = bits - 1 if bits & 0x7FFF else bits
        cand = [int(b) for b in (b_lo, bits, bits + 1)]
        dists = [abs(Fraction(float(F.bf16_bits_to_f64(np.array([c], np.uint16))[0])) - q) for c in cand]
        assert abs(got - q) == min(dists)
    assert np.array_equal(F.bf16_bits_to_f64(np.array([0x3F80, 0xC000], np.uint16)), [1.0, -2.0])
