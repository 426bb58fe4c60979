"""Algorithmic work of one unmerged multi-LoRA call: bytes and FLOPs.

These counts define what a launch *must* move and compute; they are what the
benchmark divides by measured time.  They follow the cost model of "Serving
several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
alongside": the alongside form costs two multiply-add FLOPs per element of
each of the two low-rank products, an adapter holds the elements of A and B,
and merging (or unmerging) reads and writes every affected weight once.  Here
A is r x d_in and B is d_out x r.  The tests rebuild the page's printed FLUX
table (tests/golden/lora_costs_flux.txt) from these functions.
"""
from __future__ import annotations

from typing import Iterable


def lora_flops(slot_tokens: int, r: int, d_in: int, d_out: int) -> int:
    """FLOPs of the unmerged delta: 2 multiply-add FLOPs per MAC, r*d_in MACs for
    the shrink and d_out*r for the expand, per (token, applied adapter)."""
    return 2 * slot_tokens * (d_in * r + r * d_out)


def adapter_bytes(r: int, d_in: int, d_out: int, elem: int) -> int:
    """Bytes of one adapter: A (r x d_in) plus B (d_out x r)."""
    return r * (d_in + d_out) * elem


def call_bytes(touched_tokens: int, distinct_adapters: int, r: int, d_in: int, d_out: int, elem: int) -> int:
    """Algorithmic HBM bytes of one fused call: every touched row of x read once,
    every touched row of y read and written once, every adapter used read once."""
    return touched_tokens * (d_in + 2 * d_out) * elem + distinct_adapters * adapter_bytes(r, d_in, d_out, elem)


def sliced_call_bytes(touched_tokens: int, distinct_adapters: int, r: int, d_in: int, d_outs, elem: int) -> int:
    """Algorithmic HBM bytes of one group of projections that read one x: x read
    once for the group, each projection's y read and written once, each used
    adapter of each projection read once."""
    return (touched_tokens * (d_in + 2 * sum(d_outs)) * elem
            + distinct_adapters * sum(adapter_bytes(r, d_in, d, elem) for d in d_outs))


def batch_work(seg_bounds: Iterable, idx, n_adapters: int):
    """(touched tokens, slot-tokens, distinct adapters) of a batch.
    seg_bounds: [(start, end)] per request; idx: [S][K] with -1 = empty."""
    touched = slot_tokens = 0
    used = set()
    for s, (lo, hi) in enumerate(seg_bounds):
        L = max(0, hi - lo)
        valid = [int(i) for i in idx[s] if 0 <= int(i) < n_adapters]
        if L and valid:
            touched += L
            slot_tokens += L * len(valid)
            used.update(valid)
    return touched, slot_tokens, len(used)


def merge_bytes(n_weights: int, d_out: int, d_in: int, elem: int) -> int:
    """Weight traffic of merging (or unmerging) adapters into n_weights weights of
    d_out x d_in: each weight is read once and written once."""
    return 2 * n_weights * d_out * d_in * elem
