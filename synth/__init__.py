"""Seeded synthetic inputs for the routed-expert NVFP4 MoE layer.

This module is shared by the CPU oracle and by the HIP path.  It only *draws*
inputs (activations, router weights, router bias, fp32 expert weights,
codebooks and codebook indices) and converts fp32 to bf16 bit patterns; it
holds none of the method's arithmetic (no quantizer, router, FFN or combine).

Workload shapes follow the engine the pages describe: the release-post page
("capy-flash v0.7.1: a 125B MoE on 64 GB of RAM ...", section "What shipped")
gives 48 layers x 512 routed experts with gate/up and down projections; the
hidden size, expert width, top-k and value distributions are the stated
synthetic workloads (see WORKLOADS).

Every tensor has its own seed derived from (workload seed, layer, expert,
projection), so any single expert can be regenerated on the host without
drawing the others.  Large workloads draw their expert weights on the device
with torch's Philox generator instead (``expert_weights_torch``); those values
differ from the host draws of the same expert, so a test that mixes the two
copies the device draws back to the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# Projection ids used in seeds.
PROJ_GATE, PROJ_UP, PROJ_DOWN = 0, 1, 2
FMT_NVFP4, FMT_CB3G128 = 0, 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int                 # hidden size
    I: int                 # expert intermediate size
    E: int                 # routed experts per layer
    k: int                 # experts per token
    T: int                 # tokens per step
    layers: int = 1
    router_std: float = 0.02
    expert_std: float = 0.02
    outlier_rate: float = 0.0   # fraction of activation elements scaled
    outlier_mult: float = 1.0
    zipf_s: float = 0.0         # router bias -s*ln(rank_e); 0 = no bias
    seed: int = 0
    gate_up_fmt: int = FMT_NVFP4
    residual: bool = False

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Layer-0 activation second moment with 1% of elements scaled by 20:
# E[x^2] = 0.99 * 1 + 0.01 * 400 = 4.99.  A router std of 1/sqrt(H * E[x^2])
# makes each logit ~N(0, 1) ("logits N(0,1)-scaled" for the 48-layer stack).
_STACK_ROUTER_STD = 1.0 / math.sqrt(2560 * 4.99)
# The first layer's input RMS, sqrt(E[x^2]): the scale every later layer's
# input is brought back to in the 48-layer stack.
STACK_INPUT_RMS = math.sqrt(4.99)

WORKLOADS = {
    # Tiny single layer, small enough for exact brute force.
    "tiny": Workload("tiny", H=256, I=128, E=16, k=2, T=4,
                     router_std=0.05, expert_std=0.02, seed=0),
    # Flash-Next-shaped decode layer, one token.
    "decode": Workload("decode", H=2560, I=640, E=512, k=10, T=1,
                       outlier_rate=0.01, outlier_mult=20.0, seed=1),
    # Same layer, eight tokens.
    "decode_b8": Workload("decode_b8", H=2560, I=640, E=512, k=10, T=8,
                          outlier_rate=0.01, outlier_mult=20.0, seed=1),
    # 48 stacked decode layers with residual add.
    "stack48": Workload("stack48", H=2560, I=640, E=512, k=10, T=1, layers=48,
                        router_std=_STACK_ROUTER_STD, outlier_rate=0.01,
                        outlier_mult=20.0, seed=2, residual=True),
    # Degenerate routing on the tiny shapes: one expert per token, and every
    # expert for every token (k = E = 16: the most pairs one token can have).
    "tiny_k1": Workload("tiny_k1", H=256, I=128, E=16, k=1, T=4,
                        router_std=0.05, expert_std=0.02, seed=7),
    "tiny_all": Workload("tiny_all", H=256, I=128, E=16, k=16, T=4,
                         router_std=0.05, expert_std=0.02, seed=8),
    # The largest expert count and top-k the library takes (E = 1024, k = 32)
    # on the tiny widths.
    "max_ek": Workload("max_ek", H=256, I=128, E=1024, k=32, T=4,
                       router_std=0.05, expert_std=0.02, seed=10),
    # Wide single layers (few experts): one token with H above 2560 takes the
    # decode path with a K-split gate/up and a separate h^ step.
    "wide4k": Workload("wide4k", H=4096, I=256, E=16, k=4, T=1, seed=5),
    "wide10k": Workload("wide10k", H=10240, I=128, E=8, k=2, T=1, seed=6),
    # Wide intermediate size (I = 1152: 72 NVFP4 blocks per h row, more than
    # one per lane of a wave) on few experts.
    "wide_i": Workload("wide_i", H=256, I=1152, E=8, k=2, T=4,
                       router_std=0.05, expert_std=0.02, seed=9),
    # 8192-token prefill with a Zipf(1.1) router bias.
    "prefill8k": Workload("prefill8k", H=2560, I=640, E=512, k=10, T=8192,
                          zipf_s=1.1, seed=3),
    # 65536-token prefill, uniform routing.
    "prefill64k": Workload("prefill64k", H=2560, I=640, E=512, k=10, T=65536,
                           seed=4),
    # Same, gate/up in the 3-bit group-128 fp16-codebook format.
    "prefill64k_cb": Workload("prefill64k_cb", H=2560, I=640, E=512, k=10,
                              T=65536, seed=4, gate_up_fmt=FMT_CB3G128),
}


# --------------------------------------------------------------------------
# bf16 bit patterns (input encoding only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.
    Inputs are finite."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    return ((bits + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# host draws (numpy PCG64, one stream per tensor)
# --------------------------------------------------------------------------

def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(v) for v in key])


def activations(wl: Workload, T: Optional[int] = None, stream: int = 0) -> np.ndarray:
    """bf16 bits [T, H]: N(0,1); with outliers, each element independently
    (probability outlier_rate) multiplied by outlier_mult before rounding."""
    T = wl.T if T is None else T
    g = _rng(wl.seed, 0xA11, stream)
    x = g.standard_normal((T, wl.H), dtype=np.float32)
    if wl.outlier_rate > 0:
        mask = g.random((T, wl.H)) < wl.outlier_rate
        x = np.where(mask, x * np.float32(wl.outlier_mult), x).astype(np.float32)
    return f32_to_bf16_bits(x)


def router_weights(wl: Workload, layer: int = 0) -> np.ndarray:
    """fp32 [E, H] ~ N(0, router_std)."""
    g = _rng(wl.seed, 0xB0, layer)
    return (g.standard_normal((wl.E, wl.H), dtype=np.float32)
            * np.float32(wl.router_std)).astype(np.float32)


def router_bias(wl: Workload, layer: int = 0) -> Optional[np.ndarray]:
    """fp32 [E] or None.  Zipf(s) popularity: expert e gets the rank r_e of a
    seeded permutation of 1..E and bias -s*ln(r_e), so exp(bias) is
    proportional to r_e^-s (the normalising constant cancels in softmax)."""
    if wl.zipf_s == 0:
        return None
    g = _rng(wl.seed, 0xB1, layer)
    rank = g.permutation(wl.E) + 1
    return (-wl.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)


def expert_weights(wl: Workload, layer: int, expert: int):
    """(gate [I,H], up [I,H], down [H,I]) fp32 ~ N(0, expert_std), host draw."""
    out = []
    for proj, shape in ((PROJ_GATE, (wl.I, wl.H)), (PROJ_UP, (wl.I, wl.H)),
                        (PROJ_DOWN, (wl.H, wl.I))):
        g = _rng(wl.seed, 0xC0, layer, expert, proj)
        out.append((g.standard_normal(shape, dtype=np.float32)
                    * np.float32(wl.expert_std)).astype(np.float32))
    return tuple(out)


def static_h_scales(wl: Workload, layer: int = 0) -> np.ndarray:
    """Calibrated-style static h tensor scales, one per expert (fp32 [E]):
    a base of the order of a row's amax / 2688 at this workload's weight and
    activation spread (g and u ~ expert_std * sqrt(H * E[x^2]), a row amax of
    about 6 of their product) times a seeded factor in [0.5, 2], so some
    rows saturate and some quantize coarsely."""
    x2 = (1.0 - wl.outlier_rate) + wl.outlier_rate * wl.outlier_mult ** 2
    s = wl.expert_std * math.sqrt(wl.H * x2)
    base = 6.0 * s * s / 2688.0
    g = _rng(wl.seed, 0x5C, layer)
    return (base * g.uniform(0.5, 2.0, wl.E)).astype(np.float32)


def codebook_weights(wl: Workload, layer: int, expert: int, proj: int):
    """3-bit group-128 codebook weights for one gate or up matrix [I, H].

    Returns (codebooks fp16 [I, H/128, 8], indices uint8 [I, H] in 0..7).
    Each group's 8 entries are 8 N(0, expert_std) draws sorted ascending and
    rounded to fp16; each weight's index is drawn uniformly, so every weight
    is marginally N(0, expert_std) up to fp16 rounding."""
    assert proj in (PROJ_GATE, PROJ_UP)
    g = _rng(wl.seed, 0xCB, layer, expert, proj)
    groups = wl.H // 128
    cb = np.sort(g.standard_normal((wl.I, groups, 8)) * wl.expert_std, axis=-1)
    idx = g.integers(0, 8, size=(wl.I, wl.H), dtype=np.uint8)
    return cb.astype(np.float16), idx


# --------------------------------------------------------------------------
# device draws (torch Philox) for workloads too large for host memory
# --------------------------------------------------------------------------

def _torch_gen(device, *key: int):
    import torch
    h = 0x9E3779B97F4A7C15
    for v in key:
        h = ((h ^ (int(v) & 0xFFFFFFFFFFFF)) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    gen = torch.Generator(device=device)
    gen.manual_seed(h & 0x7FFFFFFFFFFFFFFF)
    return gen


def expert_weights_torch(wl: Workload, layer: int, e0: int, e1: int, device):
    """fp32 device tensors gate [n,I,H], up [n,I,H], down [n,H,I] for experts
    e0..e1-1, drawn with torch's generator on `device` (one stream per
    (layer, expert, projection))."""
    import torch
    n = e1 - e0
    gate = torch.empty((n, wl.I, wl.H), dtype=torch.float32, device=device)
    up = torch.empty_like(gate)
    down = torch.empty((n, wl.H, wl.I), dtype=torch.float32, device=device)
    for j in range(n):
        e = e0 + j
        for proj, t in ((PROJ_GATE, gate), (PROJ_UP, up), (PROJ_DOWN, down)):
            gen = _torch_gen(device, wl.seed, 0xC0, layer, e, proj)
            t[j].normal_(0.0, wl.expert_std, generator=gen)
    return gate, up, down


def codebook_weights_torch(wl: Workload, layer: int, e0: int, e1: int, proj: int, device):
    """Device version of codebook_weights for experts e0..e1-1:
    (codebooks fp16 [n, I, H/128, 8], indices uint8 [n, I, H])."""
    import torch
    n = e1 - e0
    groups = wl.H // 128
    cbs = torch.empty((n, wl.I, groups, 8), dtype=torch.float16, device=device)
    idx = torch.empty((n, wl.I, wl.H), dtype=torch.uint8, device=device)
    for j in range(n):
        gen = _torch_gen(device, wl.seed, 0xCB, layer, e0 + j, proj)
        v = torch.empty((wl.I, groups, 8), dtype=torch.float32, device=device)
        v.normal_(0.0, wl.expert_std, generator=gen)
        cbs[j] = torch.sort(v, dim=-1).values.to(torch.float16)
        idx[j] = torch.randint(0, 8, (wl.I, wl.H), generator=gen, device=device,
                               dtype=torch.int64).to(torch.uint8)
    return cbs, idx


def router_weights_torch(wl: Workload, layer: int, device):
    import torch
    gen = _torch_gen(device, wl.seed, 0xB0, layer)
    w = torch.empty((wl.E, wl.H), dtype=torch.float32, device=device)
    w.normal_(0.0, wl.router_std, generator=gen)
    return w


def activations_torch(wl: Workload, T: int, stream: int, device):
    """bf16 [T, H] device tensor, same recipe as `activations`."""
    import torch
    gen = _torch_gen(device, wl.seed, 0xA11, stream)
    x = torch.empty((T, wl.H), dtype=torch.float32, device=device)
    x.normal_(0.0, 1.0, generator=gen)
    if wl.outlier_rate > 0:
        m = torch.rand((T, wl.H), generator=gen, device=device) < wl.outlier_rate
        x = torch.where(m, x * wl.outlier_mult, x)
    return x.to(torch.bfloat16)
