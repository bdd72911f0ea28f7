"""Exact-arithmetic brute force used to pin the oracle (tests only).

Independent of ``oracle/``: formats are decoded from their bit fields, every
rounding is done on exact rationals (``fractions.Fraction``) with an explicit
round-to-nearest-even onto the fp32 grid, encoders enumerate every code and
pick the nearest, dot products are exact integer sums, and SiLU / softmax use
60-digit ``decimal`` arithmetic.
"""
from __future__ import annotations

import decimal
from fractions import Fraction

import numpy as np

_CTX = decimal.Context(prec=60)


# ---------------------------------------------------------------- fp32 grid

def round_f32(q: Fraction) -> Fraction:
    """Nearest fp32 value to q (ties to even significand), subnormals kept.
    Overflow is not expected in these tests."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    p, d = a.numerator, a.denominator
    e = p.bit_length() - d.bit_length()          # 2^e <= a < 2^(e+2)
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    # quantum 2^(e-23): scaled = a / quantum
    sh = e - 23
    if sh >= 0:
        num, den = p, d << sh
    else:
        num, den = p << (-sh), d
    r, rem = divmod(num, den)
    twice = 2 * rem
    if twice > den or (twice == den and (r & 1)):
        r += 1
    val = Fraction(r) * (Fraction(2) ** sh)
    return sign * val


def f32(x) -> Fraction:
    return Fraction(float(np.float32(x)))


# ---------------------------------------------------------------- formats

def e2m1_value(c: int) -> Fraction:
    """From the bit fields: s | e(2) | m(1), bias 1, e = 0 subnormal."""
    s = -1 if (c >> 3) & 1 else 1
    e = (c >> 1) & 3
    m = c & 1
    if e == 0:
        v = Fraction(m, 2)                       # m * 2^(1-1) * 1/2
    else:
        v = Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return s * v


def e4m3_value(c: int) -> Fraction:
    """From the bit fields: s | e(4) | m(3), bias 7, e = 0 subnormal; 0x7F NaN."""
    assert (c & 0x7F) != 0x7F
    s = -1 if (c >> 7) & 1 else 1
    e = (c >> 3) & 15
    m = c & 7
    if e == 0:
        v = Fraction(m, 8) * Fraction(2) ** -6
    else:
        v = Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
    return s * v


E2M1_POS = [(c, e2m1_value(c)) for c in range(8)]
E4M3_POS = [(c, e4m3_value(c)) for c in range(0x7F)]


def _nearest_even(a: Fraction, table):
    best = None
    for c, v in table:
        dist = abs(v - a)
        if best is None or dist < best[1] or (dist == best[1] and c % 2 == 0):
            best = (c, dist)
    return best[0]


def e2m1_encode(a: Fraction) -> int:
    if a > 6:
        return 7
    return _nearest_even(a, E2M1_POS)


def e4m3_encode(a: Fraction) -> int:
    if a > 448:
        return 0x7E
    return _nearest_even(a, E4M3_POS)


# ---------------------------------------------------------------- quantizer

def quantize_rows(v: np.ndarray, per_row: bool, ts_given=None):
    """NVFP4 quantization of fp32 rows in exact rationals, each operation
    rounded to fp32 as it happens.  ts_given: static per-row tensor scales
    (fp32 values) used instead of amax / 2688.  Returns (codes, scales,
    ts-list)."""
    v = np.asarray(v, dtype=np.float32)
    R, K = v.shape
    F = [[Fraction(float(x)) for x in row] for row in v]
    neg = np.signbit(v)
    if per_row:
        amaxes = [max(abs(x) for x in row) for row in F]
    else:
        m = max(abs(x) for row in F for x in row)
        amaxes = [m] * R
    codes = np.zeros((R, K), np.uint8)
    scales = np.zeros((R, K // 16), np.uint8)
    tss = []
    for r in range(R):
        if ts_given is not None:
            ts = Fraction(float(np.float32(ts_given[r])))
        else:
            ts = round_f32(amaxes[r] / 2688) if amaxes[r] != 0 else Fraction(0)
        tss.append(ts)
        six = round_f32(6 * ts)
        for b in range(K // 16):
            blk = F[r][16 * b:16 * b + 16]
            if ts == 0:
                sb = 0
            else:
                ab = max(abs(x) for x in blk)
                sb = e4m3_encode(round_f32(ab / six))
            scales[r, b] = sb
            d = round_f32(e4m3_value(sb) * ts)
            for j, x in enumerate(blk):
                if d == 0:
                    codes[r, 16 * b + j] = 0
                    continue
                q = round_f32(x / d)
                mag = e2m1_encode(abs(q))
                codes[r, 16 * b + j] = (8 if neg[r, 16 * b + j] else 0) | mag
    return codes, scales, tss


# ---------------------------------------------------------------- exact dots

def int_parts(codes, scales):
    """A = 2*e2m1 (integers), S = E4M3 * 2^9 (integers) per element."""
    codes = np.asarray(codes)
    A = np.array([int(2 * e2m1_value(c)) for c in range(16)], dtype=np.int64)[codes]
    Sv = np.array([int(e4m3_value(c) * 512) if (c & 0x7F) != 0x7F else 0
                   for c in range(256)], dtype=np.int64)
    S = np.repeat(Sv[np.asarray(scales)], 16, axis=-1)
    return A, S


def exact_matvec(Wc, Ws, Wts, Xc, Xs, Xts):
    """Exact W^ x^ for every row of W and every row of X:
    returns Fraction matrix [X rows][W rows]."""
    Aw, Sw = int_parts(Wc, Ws)
    Ax, Sx = int_parts(Xc, Xs)
    IW = Aw * Sw                                 # value = IW * ts / 1024
    IX = Ax * Sx
    P = IX @ IW.T                                # exact int64 (|P| < 2^62 here)
    out = []
    for i in range(P.shape[0]):
        xts = Xts[i] if isinstance(Xts, (list, tuple)) else Fraction(float(Xts[i]))
        out.append([Fraction(int(P[i, j])) * xts * Fraction(Wts) / (1024 * 1024)
                    for j in range(P.shape[1])])
    return out


def dec(q: Fraction) -> decimal.Decimal:
    return _CTX.divide(decimal.Decimal(q.numerator), decimal.Decimal(q.denominator))


def silu_exact(z: Fraction) -> decimal.Decimal:
    zd = dec(z)
    return _CTX.divide(zd, _CTX.add(decimal.Decimal(1), _CTX.exp(-zd)))


def dec_to_fraction(d: decimal.Decimal) -> Fraction:
    return Fraction(d)
