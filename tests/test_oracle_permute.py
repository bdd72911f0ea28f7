"""Pins for oracle.permute against a plain loop counting sort."""
import numpy as np
import pytest

from oracle import permute


def _loop(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    perm = []
    for e in range(E):
        for i, v in enumerate(flat):
            if v == e:
                perm.append(i)
    inv = [0] * len(flat)
    for j, i in enumerate(perm):
        inv[i] = j
    return counts, offsets, perm, inv


@pytest.mark.parametrize("T,k,E,seed", [(4, 2, 16, 0), (37, 3, 8, 1), (1, 10, 512, 2), (0, 2, 4, 3), (50, 1, 1, 4)])
def test_permute_vs_loop(T, k, E, seed):
    r = np.random.default_rng(seed)
    ids = r.integers(0, E, (T, k)) if T else np.zeros((0, k), int)
    c, o, p, inv = permute.permute(ids, E)
    lc, lo, lp, li = _loop(ids, E)
    assert list(c) == lc and list(o) == lo and list(p) == lp and list(inv) == li


def test_permute_invariants_skewed():
    r = np.random.default_rng(5)
    ids = np.minimum(r.zipf(1.5, (500, 10)) - 1, 63)
    c, o, p, inv = permute.permute(ids, 64)
    assert c.sum() == ids.size and o[-1] == ids.size
    assert np.array_equal(np.sort(p), np.arange(ids.size))
    flat = ids.reshape(-1)
    assert np.all(np.diff(flat[p]) >= 0)
    for e in range(64):
        seg = p[o[e]:o[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    assert np.array_equal(p[inv], np.arange(ids.size))
