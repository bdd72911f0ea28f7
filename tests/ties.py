"""Inputs that put the NVFP4 quantizer's rounding decisions exactly on ties,
at block scales d that are not powers of two.

Two kinds of tie exist in the quantizer (every step fp32, round to nearest
even): an element whose quotient v / d lies exactly halfway between two E2M1
magnitudes (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5), and a block whose scale
ratio max|v_b| / (6 ts) lies exactly halfway between two E4M3 values.  For
such inputs a division that is off by one unit in the last place, or a
rounding that breaks ties the wrong way, changes a code.

The rows here are built so the ties are exact in fp32 (and, for activations,
in bf16): the tensor scale ts is chosen with few significant bits (so that
d = E4M3(sb) * ts and m * d stay exact), and the block maxima are placed at
6 * d (so the block scale is exactly the intended E4M3 value) or at
mu * 6 * ts for an E4M3 midpoint mu.  Nothing here evaluates the quantizer;
tests count the ties with the oracle's own scales.

Also the tiny layer whose h rows hit exact ties (tie_layer): x, gate and up
weights chosen so that every gate output is 32 (SiLU(32) rounds to 32 in
fp32) and every up output an exact multiple of 2, making h = 64 * N for
integers N set row element by row element.
"""
from __future__ import annotations

import numpy as np

E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def e4m3_values() -> np.ndarray:
    """Values of the non-negative E4M3 codes 0x00 .. 0x7E (bit fields)."""
    c = np.arange(0x7F)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))


def bf16_exact(v) -> np.ndarray:
    """True where the fp32 value is exactly representable in bf16."""
    u = np.asarray(v, np.float32).view(np.uint32)
    return (u & 0xFFFF) == 0


def _f32(x):
    return np.float32(x)


def _elem_block(ab, d, signs, rng):
    """A 16-element block: ab first, then the 7 midpoints * d with signs and
    the same with the opposite signs, then -ab (all exact)."""
    ties = (E2M1_MIDS * np.float64(d)).astype(np.float32)
    blk = np.concatenate([[ab], ties * signs, -ties * signs, [-ab]]).astype(np.float32)
    return blk[rng.permutation(16)]


def act_tie_rows(n_rows: int, H: int, seed: int) -> np.ndarray:
    """fp32 rows, every element bf16-exact, with exact element and scale
    ties at tensor scales ts = c * 2^j (c = 3, 5, 7, 9, 11: not powers of two)."""
    rng = np.random.default_rng(seed)
    vals = e4m3_values()
    mids = (vals[1:] + vals[:-1]) / 2
    rows = []
    for r in range(n_rows):
        c = [3, 5, 7, 9, 11][r % 5]
        j = int(rng.integers(-24, 4))
        ts = _f32(c * 2.0 ** j)
        amax = _f32(2688 * np.float64(ts))
        six_ts = _f32(6) * ts
        row = np.zeros(H, np.float32)
        row[0] = amax
        # candidate block scales S: d = S ts, 6 d and all m d exact in bf16
        good_s = []
        for S in vals[1:]:
            d = _f32(np.float32(S) * ts)
            ab = _f32(6) * d
            if ab > amax or not bf16_exact(ab) or _f32(ab / six_ts) != np.float32(S):
                continue
            if not np.all(bf16_exact((E2M1_MIDS * np.float64(d)).astype(np.float32))):
                continue
            if np.any((E2M1_MIDS * np.float64(d)).astype(np.float32) != E2M1_MIDS * np.float64(d)):
                continue
            good_s.append((ab, d))
        good_mu = []
        for mu in mids:
            ab = _f32(np.float64(mu) * np.float64(six_ts))
            if ab == 0 or ab > amax or not bf16_exact(ab) or np.float64(ab) != mu * np.float64(six_ts):
                continue
            if np.float64(_f32(ab / six_ts)) != mu:
                continue
            good_mu.append(ab)
        for b in range(1, H // 16):
            if b % 2 == 1 and good_s:
                ab, d = good_s[int(rng.integers(len(good_s)))]
                signs = np.where(rng.random(7) < 0.5, -1.0, 1.0).astype(np.float32)
                row[16 * b:16 * b + 16] = _elem_block(ab, d, signs, rng)
            elif good_mu:
                ab = good_mu[int(rng.integers(len(good_mu)))]
                rest = (rng.uniform(-1, 1, 15) * ab).astype(np.float32)
                rest = _to_bf16_f32(rest)
                rest = np.clip(rest, -ab, ab)
                blk = np.concatenate([[ab], rest]).astype(np.float32)
                row[16 * b:16 * b + 16] = blk[rng.permutation(16)]
        rows.append(row)
    out = np.stack(rows)
    assert np.all(bf16_exact(out))
    return out


def _to_bf16_f32(v):
    """Round fp32 values to bf16 (nearest even), returned as fp32."""
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def weight_tie_matrix(rows: int, cols: int, seed: int) -> np.ndarray:
    """An fp32 weight matrix (one tensor scale) whose tensor scale ts has 16
    random significant bits; its blocks alternate between element ties at
    d = S ts (20 significant bits) and scale ties at mu * 6 ts."""
    rng = np.random.default_rng(seed)
    vals = e4m3_values()
    mids = (vals[1:] + vals[:-1]) / 2
    mant = 1 + rng.integers(0, 1 << 15) / float(1 << 15)
    ts = _f32(mant * 2.0 ** int(rng.integers(-14, -8)))
    amax = _f32(2688 * np.float64(ts))
    assert np.float64(amax) == 2688 * np.float64(ts)
    six_ts = _f32(6) * ts
    W = np.zeros((rows, cols), np.float32)
    W[0, 0] = amax
    for r in range(rows):
        for b in range(cols // 16):
            if r == 0 and b == 0:
                continue
            if (r + b) % 2 == 0:
                S = vals[int(rng.integers(40, 0x7E))]
                d = _f32(np.float32(S) * ts)
                ab = _f32(6) * d
                ties = E2M1_MIDS * np.float64(d)
                if ab > amax or np.any(ties.astype(np.float32) != ties) or _f32(ab / six_ts) != np.float32(S):
                    continue
                signs = np.where(rng.random(7) < 0.5, -1.0, 1.0).astype(np.float32)
                W[r, 16 * b:16 * b + 16] = _elem_block(ab, d, signs, rng)
            else:
                mu = mids[int(rng.integers(40, len(mids)))]
                ab = _f32(np.float64(mu) * np.float64(six_ts))
                if ab > amax or np.float64(ab) != mu * np.float64(six_ts) or np.float64(_f32(ab / six_ts)) != mu:
                    continue
                blk = np.concatenate([[ab], (rng.uniform(-1, 1, 15) * ab).astype(np.float32)])
                W[r, 16 * b:16 * b + 16] = blk[rng.permutation(16)]
    return W


def count_ties(v: np.ndarray, scales: np.ndarray, ts) -> tuple:
    """(element ties, scale ties) of rows v [R, K] given the quantizer's block
    scale codes [R, K/16] and tensor scale(s): elements with |v| / d exactly
    an E2M1 midpoint, blocks with max|v_b| / (6 ts) exactly an E4M3 midpoint
    (both decided in fp64, where these quotients are exact)."""
    v = np.asarray(v, np.float64)
    R, K = v.shape
    vals = e4m3_values()
    mids = (vals[1:] + vals[:-1]) / 2
    ts = np.broadcast_to(np.asarray(ts, np.float64).reshape(-1, 1), (R, 1))
    d = (vals[scales].astype(np.float32) * ts.astype(np.float32)).astype(np.float32).astype(np.float64)
    q = np.abs(v.reshape(R, K // 16, 16)) / np.where(d == 0, np.inf, d)[:, :, None]
    elem = int(np.isin(q, E2M1_MIDS).sum())
    six_ts = (np.float32(6) * ts.astype(np.float32)).astype(np.float64)
    ab = np.abs(v.reshape(R, K // 16, 16)).max(axis=2)
    ratio = ab / np.where(six_ts == 0, np.inf, six_ts)
    scale = int(np.isin(ratio, mids).sum())
    return elem, scale


# ---------------------------------------------------------------- h ties
U = 64.0                      # h = U * N on the tie layer


def _up_terms(n: int) -> list:
    """Fifteen values 2a (a an E2M1 value) summing to n (|n| <= 167)."""
    assert abs(n) <= 167
    sgn = 1 if n >= 0 else -1
    r = abs(n)
    terms = []
    while r >= 12:
        terms.append(12)
        r -= 12
    tail = {0: [], 1: [1], 2: [2], 3: [3], 4: [4], 5: [4, 1], 6: [6], 7: [6, 1], 8: [8], 9: [8, 1],
            10: [8, 2], 11: [8, 3]}[r]
    terms += tail
    assert len(terms) <= 15
    return [sgn * t for t in terms]


def h_pattern(I: int, mode: str, seed: int) -> np.ndarray:
    """Integers N [I] (h = 64 N) for one h row.
    dynamic: the row amax is 126 * 64, so ts = 3; blocks with max 72 (block
    scale 256, d = 12 * 64: ties at N = 12 m) and max 36 (block scale 128,
    d = 6 * 64: ties at 15, 21, 30), and general blocks.
    static (ts = 6 given): blocks with max 72 (scale 128, d = 12 * 64: the
    same element ties) and scale-ratio ties: max 153 gives 272 (between E4M3
    256 and 288: to even, 256) and max 171 gives 304 (between 288 and 320: to
    even, 320)."""
    rng = np.random.default_rng(seed)
    N = np.full(I, 18, np.int64)
    mids12 = (12 * E2M1_MIDS).astype(np.int64)           # 3, 9, 15, 21, 30, 42, 60
    for b in range(I // 16):
        sl = slice(16 * b, 16 * b + 16)
        kind = b % 4
        if mode == "dynamic" and b == 0:
            blk = np.concatenate([[126], rng.integers(-120, 121, 15)])
        elif kind in (0, 1):
            s = np.where(rng.random(7) < 0.5, -1, 1)
            blk = np.concatenate([[72], mids12 * s, -mids12 * s, [-72]])
        elif mode == "dynamic" and kind == 2:
            blk = np.array([36, 15, -15, 21, -21, 30, -30, 14, 16, 20, 22, 29, 31, -35, 7, -8])
        elif mode == "dynamic":
            blk = rng.integers(-126, 127, 16)
        else:
            top = 153 if kind == 2 else 171
            blk = np.concatenate([[top], rng.integers(-140, 141, 15)])
        N[sl] = blk[rng.permutation(16)]
    return N


def tie_layer(H: int, I: int, E: int, N: np.ndarray, seed: int):
    """fp32 expert weights gate, up [E, I, H], down [E, H, I] and one bf16
    activation row (fp32 values) such that every expert's h row is 64 * N:
    x = [2688, 0 x 15] then blocks [6, 4 x 15]: its tensor scale is 1 and x^
    reproduces these values; gate and up matrices have tensor scale 2^-8
    (an element 10.5 = 2688 * 2^-8 where x is 0) and block scale 256, so the
    gate row [.., 6 (position 16), -1 (17), ..] gives g = 6 * 6 - 4 = 32 and
    the up row [6, a_1 .. a_15] at positions 16..31 gives u = 36 + 4 sum a;
    h = SiLU(32) u = 32 u = 64 (18 + 2 sum a).  Down weights are random."""
    assert H >= 32 and H % 16 == 0
    x = np.zeros(H, np.float32)
    x[0] = 2688.0
    for b in range(1, H // 16):
        x[16 * b] = 6.0
        x[16 * b + 1:16 * b + 16] = 4.0
    gate = np.zeros((E, I, H), np.float32)
    up = np.zeros((E, I, H), np.float32)
    gate[:, :, 16] = 6.0
    gate[:, :, 17] = -1.0
    gate[:, 0, 1] = 10.5
    up[:, :, 16] = 6.0
    up[:, 0, 1] = 10.5
    for n in range(I):
        terms = _up_terms(int(N[n]) - 18)
        up[:, n, 17:17 + len(terms)] = np.asarray(terms, np.float32) / 2
    rng = np.random.default_rng(seed)
    down = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    return gate, up, down, x
