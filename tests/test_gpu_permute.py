"""GPU parity: token-by-expert counting sort, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import quantized_moe_routed_router_amd as moe
from oracle import permute as operm
from tests.gpu_helpers import say, t2n

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_permute(ids: np.ndarray, E: int):
    T, k = ids.shape
    N = T * k
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(max(N, 1), dtype=torch.int32, device=DEV)
    inv = torch.empty(max(N, 1), dtype=torch.int32, device=DEV)
    wsb = moe.moe_permute_workspace_bytes(T, k, E)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    idt = torch.from_numpy(np.ascontiguousarray(ids, np.int32).reshape(-1) if N else np.zeros(1, np.int32)).to(DEV)
    moe.moe_permute(idt, T, k, E, counts, offsets, perm, inv, ws, wsb)
    torch.cuda.synchronize()
    return t2n(counts), t2n(offsets), t2n(perm)[:N], t2n(inv)[:N]


@pytest.mark.parametrize("T,k,E,kind", [(4, 2, 16, "uniform"), (1, 10, 512, "uniform"),
                                        (8192, 10, 512, "zipf"), (1000, 3, 7, "uniform"),
                                        (3000, 10, 512, "one"), (65536, 10, 512, "uniform"),
                                        (333, 1, 1, "uniform")])
def test_permute_bit_exact(T, k, E, kind):
    say("permute", T, k, E, kind)
    r = np.random.default_rng(T + k + E)
    if kind == "uniform":
        ids = np.stack([r.permutation(E)[:k] for _ in range(T)]) if T * k <= 200_000 else \
            r.integers(0, E, (T, k))
    elif kind == "zipf":
        ids = np.minimum(r.zipf(1.1, (T, k)) - 1, E - 1)
    else:
        ids = np.full((T, k), 17)
    ids = ids.astype(np.int32)
    c, o, p, inv = run_permute(ids, E)
    oc, oo, op, oinv = operm.permute(ids, E)
    assert np.array_equal(c, oc) and np.array_equal(o, oo)
    assert np.array_equal(p, op) and np.array_equal(inv, oinv)


def test_permute_empty():
    c, o, p, inv = run_permute(np.zeros((0, 4), np.int32), 32)
    assert not c.any() and not o.any()


def test_permute_invalid_ids_trail():
    ids = np.array([[3, -1], [7, 3], [40, 0]], np.int32)
    c, o, p, inv = run_permute(ids, 8)
    assert list(c) == [1, 0, 0, 2, 0, 0, 0, 1]
    assert o[-1] == 4                      # entries with valid ids
    assert list(p[:4]) == [5, 0, 3, 2]     # (expert, flat index) order
    assert sorted(p[4:]) == [1, 4]
    assert np.array_equal(p[inv], np.arange(6))
