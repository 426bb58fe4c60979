"""Seeded synthetic device tensors for the full-size launches.

The workloads too large to draw on the host -- the decode batch through 32
layer pools, the Llama-3-8B-shaped stack (40 GiB of resident adapters), the
FLUX-sized merge -- are drawn directly in device memory with a seeded torch
generator.  ``bench.py`` and the GPU parity tests both build them through the
functions here, so the tests check exactly the launches the benchmark times.
Like the rest of ``workloads``, this module only draws random numbers and lays
them out; it performs none of the LoRA arithmetic.

Distributions as in ``workloads``: A, B ~ N(0, 0.02), x, y ~ N(0, 1), drawn in
float32 and rounded to bf16; batches from the numpy generators of
``workloads`` (Zipf(1.1) adapter choice over a seeded permutation of the pool).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, List, Tuple

import numpy as np

from . import LLAMA3_8B_LAYERS, LLAMA3_8B_PROJ, SEEDS, Batch, batch_c2, batch_c4


def _torch():
    import torch
    return torch


def randn_pool(gen, n, r, d_in, d_out, dev, std=0.02):
    """A resident bf16 pool A [n][r][d_in], B [n][d_out][r]."""
    torch = _torch()
    A = (torch.randn((n, r, d_in), generator=gen, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)
    B = (torch.randn((n, d_out, r), generator=gen, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)
    return A, B


def randn_act(gen, T, d, dev):
    """Activations [T][d], bf16."""
    torch = _torch()
    return torch.randn((T, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)


def batch_tensors(b: Batch, dev):
    """(idx, seg_off or None, scale or None) of a batch as device tensors."""
    torch = _torch()
    idx = torch.from_numpy(np.ascontiguousarray(b.idx, dtype=np.int32)).to(dev)
    seg = None if b.seg_off is None else torch.from_numpy(np.ascontiguousarray(b.seg_off, dtype=np.int32)).to(dev)
    sc = None if b.scale is None else torch.from_numpy(np.ascontiguousarray(b.scale, dtype=np.float32)).to(dev)
    return idx, seg, sc


@dataclasses.dataclass
class DecodeStack:
    """One 64-token decode batch family through `layers` independent q_proj pools."""
    pools: List[Tuple]      # [(A, B)] per layer
    xs: List                # [T][d] per layer
    ys: List                # [T][d] per layer
    batches: List[Batch]    # n_batches seeded batches (a step cycles through them)
    n: int
    r: int
    d: int


def decode_stack(dev, layers=32, n=1000, r=16, d=4096, T=64, n_batches=16, seed=SEEDS["C2"],
                 make_batch: Callable = batch_c2) -> DecodeStack:
    """The decode workload of the Llama-3-8B q_proj shape: pools of n rank-r
    adapters per layer, batches of T one-token requests (make_batch(rng, n))."""
    torch = _torch()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    pools = [randn_pool(gen, n, r, d, d, dev) for _ in range(layers)]
    xs = [randn_act(gen, T, d, dev) for _ in range(layers)]
    ys = [randn_act(gen, T, d, dev) for _ in range(layers)]
    batches = [make_batch(np.random.default_rng([seed, j]), n) for j in range(n_batches)]
    return DecodeStack(pools, xs, ys, batches, n, r, d)


@dataclasses.dataclass
class LayerProj:
    layer: int
    name: str
    A: object
    B: object
    x: object
    y: object


@dataclasses.dataclass
class C4Stack:
    """The Llama-3-8B-shaped stack: every (layer, projection) with its own pool,
    x and y, grouped by projection shape in the order shapes first appear
    (q,o 4096->4096 | k,v 4096->1024 | gate,up 4096->14336 | down 14336->4096)."""
    batch: Batch
    groups: List[Tuple[int, int, List[LayerProj]]]   # (d_in, d_out, projections of that shape)
    n: int
    r: int


def c4_stack(dev, seed=SEEDS["C4"], n=256, r=32, layers=LLAMA3_8B_LAYERS) -> C4Stack:
    torch = _torch()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    batch = batch_c4(np.random.default_rng(seed), n)
    T = batch.T
    by_shape = {}
    for li in range(layers):
        for name, d_in, d_out in LLAMA3_8B_PROJ:
            A, B = randn_pool(gen, n, r, d_in, d_out, dev)
            x, y = randn_act(gen, T, d_in, dev), randn_act(gen, T, d_out, dev)
            by_shape.setdefault((d_in, d_out), []).append(LayerProj(li, name, A, B, x, y))
    groups = [(d_in, d_out, projs) for (d_in, d_out), projs in by_shape.items()]
    return C4Stack(batch, groups, n, r)


@dataclasses.dataclass
class C4SharedX:
    """The Llama-3-8B-shaped stack with the model's own input sharing: per layer,
    q / k / v read one x and gate / up another (o and down have their own)."""
    batch: Batch
    layers: List[Tuple[dict, dict]]   # per layer: ({proj: x}, {proj: (A, B, y)})
    dims: dict                        # proj -> (d_in, d_out)
    n: int
    r: int


def c4_shared_x(dev, seed=SEEDS["C4"], n=256, r=32, layers=LLAMA3_8B_LAYERS) -> C4SharedX:
    torch = _torch()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 1)
    batch = batch_c4(np.random.default_rng(seed), n)
    T = batch.T
    dims = {name: (d_in, d_out) for name, d_in, d_out in LLAMA3_8B_PROJ}
    per_layer = []
    for _ in range(layers):
        x_attn, x_o, x_mlp, x_down = (randn_act(gen, T, dims[k][0], dev) for k in ("q", "o", "gate", "down"))
        proj = {}
        for name, (d_in, d_out) in dims.items():
            A, B = randn_pool(gen, n, r, d_in, d_out, dev)
            proj[name] = (A, B, randn_act(gen, T, d_out, dev))
        per_layer.append(({"q": x_attn, "k": x_attn, "v": x_attn, "o": x_o, "gate": x_mlp, "up": x_mlp,
                           "down": x_down}, proj))
    return C4SharedX(batch, per_layer, dims, n, r)


def flux_merge(dev, r=64, layers=57, per_layer=4, d=3072, seed=106):
    """One rank-r adapter for every attention projection of a FLUX-sized model
    (layers x per_layer weights of d x d, bf16): [(A [1][r][d], B [1][d][r], W [d][d])]."""
    torch = _torch()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    mats = []
    for _ in range(layers * per_layer):
        A, B = randn_pool(gen, 1, r, d, d, dev)
        W = (torch.randn((d, d), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        mats.append((A, B, W))
    return mats
