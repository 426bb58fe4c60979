#!/usr/bin/env python3
"""Benchmark of the unmerged multi-LoRA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME[,NAME]] [--no-cpu-baseline]

One JSON line on stdout.  The headline workload ("C2x32") is the decode
batch of the Llama-3-8B q_proj configuration -- 64 requests x 1 token,
adapters drawn Zipf(1.1) from a pool of 1000 resident rank-16 adapters per
layer, 4096 -> 4096, bf16 -- taken through the q_proj LoRA of all 32 layers:
one step = one plan build (device scheduler) + one multi-problem fused
launch over the 32 layer pools.  Every step uses a different batch (cycled
from 16 seeded batches) so that adapter reuse across steps is what Zipf
popularity gives, not a replay of one batch.

`value` is LoRA-delta tokens/s (tokens through all 32 layers per second).
`roofline` is for the dominant kernel (the fused apply kernel): algorithmic
bytes per launch / its average duration from HIP events recorded around it
on its stream, against the 8 TB/s HBM peak.  `variants` holds the same
measurements for the other workloads (tiny fp32, single-layer decode, long
prefill, the full Llama-3-8B-shaped stack, the diffusion multi-adapter
cases).  `cpu_baseline` times the fp64 oracle on a bounded sample of the
headline workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from rank_sgmv_bgmv_amd import accounting  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0

# HBM traffic of the headline kernel per launch, from two rocprofv3 --pmc runs
# of `bench.py --only decode32` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
# each scaled by what the same counter reads for a plain copy of known size
# (`bench.py --copy-calibration`: 256 MiB read + 256 MiB written per launch
# reads FETCH_SIZE 131084 KiB and WRITE_SIZE 262144 KiB, so x2.0 and x1.0).
# Valid only for the kernel sources they were taken on: reported as null once
# those sources change.
TRAFFIC_SOURCES = ["rank_sgmv_bgmv_amd/csrc/lora_valu.hip", "rank_sgmv_bgmv_amd/csrc/lora_device.hpp",
                   "rank_sgmv_bgmv_amd/csrc/lora_internal.hpp"]
MEASURED_TRAFFIC = {"sources_sha256_16": "f2b142c4cc45f5b0", "fetch_kib": 180004.5, "write_kib": 16384.0,
                    "fetch_scale": 2.0, "write_scale": 1.0}


def measured_traffic_bytes():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    m = MEASURED_TRAFFIC
    if h.hexdigest()[:16] != m["sources_sha256_16"]:
        return None
    return m["fetch_kib"] * 1024 * m["fetch_scale"] + m["write_kib"] * 1024 * m["write_scale"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ helpers --
def torch_mod():
    import torch
    return torch


def dev_bf16(a, dev):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def dev_tensor(a, dtype, dev):
    torch = torch_mod()
    if dtype == W.BF16:
        return dev_bf16(a, dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def dev_batch(b: W.Batch, dev):
    torch = torch_mod()
    import rank_sgmv_bgmv_amd as L
    idx = torch.from_numpy(np.ascontiguousarray(b.idx, dtype=np.int32)).to(dev)
    seg = None if b.seg_off is None else torch.from_numpy(np.ascontiguousarray(b.seg_off, dtype=np.int32)).to(dev)
    sc = None if b.scale is None else torch.from_numpy(np.ascontiguousarray(b.scale, dtype=np.float32)).to(dev)
    return L.Batch(b.T, idx, seg, sc)


def randn_pool(gen, n, r, d_in, d_out, dev, std=0.02):
    """A resident bf16 pool drawn on the device (torch generator, seeded)."""
    torch = torch_mod()
    A = (torch.randn((n, r, d_in), generator=gen, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)
    B = (torch.randn((n, d_out, r), generator=gen, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)
    return A, B


def randn_act(gen, T, d, dev):
    torch = torch_mod()
    return torch.randn((T, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)


class Timer:
    """Times K steps between two synchronizations; HIP events around the
    dominant kernel's launches give its average duration."""

    def __init__(self, steps):
        torch = torch_mod()
        self.steps = steps
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]

    def run(self, step, warmup):
        torch = torch_mod()
        for i in range(warmup):
            step(i, None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(self.steps):
            step(i, self.ev[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        k_ms = [a.elapsed_time(b) for a, b in self.ev]
        return wall, float(np.mean(k_ms)), k_ms


def result(name, wall, steps, tokens, bytes_step, flops_step, k_ms_avg, k_bytes, k_flops, launches, extra=None):
    ms = wall / steps * 1e3
    d = {
        "workload": name,
        "ms_per_step": round(ms, 5),
        "tokens_per_s": tokens / (ms * 1e-3),
        "algorithmic_GBps_step": bytes_step / (ms * 1e-3) / 1e9,
        "algorithmic_TFLOPs_step": flops_step / (ms * 1e-3) / 1e12,
        "apply_kernel_us": round(k_ms_avg * 1e3, 3),
        "apply_launches_per_step": launches,
        "apply_bytes_per_launch": k_bytes,
        "apply_GBps": k_bytes / (k_ms_avg * 1e-3) / 1e9,
        "apply_frac_hbm": k_bytes / (k_ms_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "apply_TFLOPs": k_flops / (k_ms_avg * 1e-3) / 1e12,
    }
    if extra:
        d.update(extra)
    return d


# ---------------------------------------------------------------- workloads --
def bench_decode_layers(dev, steps, warmup, layers=32, n=1000, n_batches=16, seed=W.SEEDS["C2"],
                        make_batch=W.batch_c2, name="decode q_proj"):
    """C2 batch through `layers` q_proj pools: plan + one multi-problem launch per step."""
    torch = torch_mod()
    import rank_sgmv_bgmv_amd as L
    r, d = 16, 4096
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    pools = [randn_pool(gen, n, r, d, d, dev) for _ in range(layers)]
    xs = [randn_act(gen, 64, d, dev) for _ in range(layers)]
    ys = [randn_act(gen, 64, d, dev) for _ in range(layers)]
    batches = [make_batch(np.random.default_rng([seed, j]), n) for j in range(n_batches)]
    dbs = [dev_batch(b, dev) for b in batches]
    plan = L.new_workspace(dbs[0], n, dev)
    shape = L.Pool(pools[0][0], pools[0][1])
    table, aligned = L.problems_table([(A, B, x, y) for (A, B), x, y in zip(pools, xs, ys)], dev)
    assert aligned

    def step(i, ev):
        db = dbs[i % n_batches]
        L.lora_plan_build(db, n, plan)
        if ev: ev[0].record()
        L.lora_apply_multi(shape, db, plan, table, aligned)
        if ev: ev[1].record()

    tm = Timer(steps)
    wall, k_ms, _ = tm.run(step, warmup)
    used = [batches[i % n_batches] for i in range(steps)]
    distinct = np.mean([len(np.unique(b.idx[b.idx >= 0])) for b in used])
    slot_tokens = np.mean([int((b.idx >= 0).sum()) for b in used])
    k_bytes = layers * accounting.call_bytes(64, distinct, r, d, d, 2)
    k_flops = layers * accounting.lora_flops(slot_tokens, r, d, d)
    res = result(f"{name} x{layers} layers", wall, steps, 64, k_bytes, k_flops, k_ms, k_bytes, k_flops, 1,
                 {"distinct_adapters_per_layer": float(distinct), "layers": layers})
    return res, (pools, batches, xs, ys)


def bench_single(case: W.Case, dev, steps, warmup, name):
    """One adapted layer: plan + fused apply per step (lora_apply builds the plan)."""
    import rank_sgmv_bgmv_amd as L
    A, B = dev_tensor(case.pool.A, case.dtype, dev), dev_tensor(case.pool.B, case.dtype, dev)
    pool = L.Pool(A, B)
    db = dev_batch(case.batch, dev)
    x = dev_tensor(case.x, case.dtype, dev)
    y = dev_tensor(case.y, case.dtype, dev)
    plan = L.new_workspace(db, case.pool.n, dev)

    def step(i, ev):
        L.lora_plan_build(db, case.pool.n, plan)
        if ev: ev[0].record()
        L.lora_apply_planned(pool, db, plan, x, y)
        if ev: ev[1].record()

    wall, k_ms, _ = Timer(steps).run(step, warmup)
    eb = 2 if case.dtype == W.BF16 else 4
    p = case.pool
    touched, slot_tokens, distinct = accounting.batch_work(case.batch.seg_bounds(), case.batch.idx, p.n)
    k_bytes = accounting.call_bytes(touched, distinct, p.r, p.d_in, p.d_out, eb)
    k_flops = accounting.lora_flops(slot_tokens, p.r, p.d_in, p.d_out)
    return result(name, wall, steps, touched, k_bytes, k_flops, k_ms, k_bytes, k_flops, 1,
                  {"tokens": touched, "distinct_adapters": distinct})


def bench_c4_stack(dev, steps, warmup, seed=W.SEEDS["C4"]):
    """Full Llama-3-8B-shaped stack: 32 layers x 7 projections, r=32, 256 adapters per
    projection; mixed 4 x 512 prefill + 256 decode tokens.  One plan per step, then
    one multi-problem launch per projection shape (q,o | k,v | gate,up | down)."""
    torch = torch_mod()
    import rank_sgmv_bgmv_amd as L
    r, n, layers = 32, 256, W.LLAMA3_8B_LAYERS
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    batch = W.batch_c4(np.random.default_rng(seed), n)
    db = dev_batch(batch, dev)
    T = batch.T
    groups = {}
    for li in range(layers):
        for name, d_in, d_out in W.LLAMA3_8B_PROJ:
            A, B = randn_pool(gen, n, r, d_in, d_out, dev)
            x, y = randn_act(gen, T, d_in, dev), randn_act(gen, T, d_out, dev)
            groups.setdefault((d_in, d_out), []).append((A, B, x, y))
    launches = []
    for (d_in, d_out), probs in groups.items():
        table, aligned = L.problems_table(probs, dev)
        launches.append((L.Pool(probs[0][0], probs[0][1]), table, aligned, probs, d_in, d_out))
    plan = L.new_workspace(db, n, dev)
    torch.cuda.synchronize()

    def step(i, ev):
        L.lora_plan_build(db, n, plan)
        if ev: ev[0].record()
        for shape, table, aligned, _, _, _ in launches:
            L.lora_apply_multi(shape, db, plan, table, aligned)
        if ev: ev[1].record()

    wall, k_ms, _ = Timer(steps).run(step, warmup)
    touched, slot_tokens, distinct = accounting.batch_work(batch.seg_bounds(), batch.idx, n)
    byts = flops = 0
    for _, _, _, probs, d_in, d_out in launches:
        byts += len(probs) * accounting.call_bytes(touched, distinct, r, d_in, d_out, 2)
        flops += len(probs) * accounting.lora_flops(slot_tokens, r, d_in, d_out)
    return result("llama3-8b stack 32x7 mixed", wall, steps, touched, byts, flops, k_ms, byts, flops, len(launches),
                  {"distinct_adapters": distinct, "note": "apply_* covers the 4 multi-problem launches together"})


def bench_c4_shared_x(dev, steps, warmup, seed=W.SEEDS["C4"], modes=("multi", "sliced")):
    """The Llama-3-8B-shaped stack with the model's own input sharing: per layer,
    query / key / value read one x and gate / up read another.  Timed two ways
    on the same data: one multi-problem launch per projection shape (q,o | k,v |
    gate,up | down: a shared x is fetched once per projection) and the sliced
    launches (q/k/v | o | gate/up | down: a tile of x is fetched once per group).
    Bytes: the minimum, with each shared x read once."""
    torch = torch_mod()
    import rank_sgmv_bgmv_amd as L
    r, n, layers = 32, 256, W.LLAMA3_8B_LAYERS
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 1)
    batch = W.batch_c4(np.random.default_rng(seed), n)
    db = dev_batch(batch, dev)
    T = batch.T
    dims = {name: (d_in, d_out) for name, d_in, d_out in W.LLAMA3_8B_PROJ}
    per_layer = []
    for _ in range(layers):
        x_attn, x_o, x_mlp, x_down = (randn_act(gen, T, dims[k][0], dev) for k in ("q", "o", "gate", "down"))
        proj = {}
        for name, (d_in, d_out) in dims.items():
            A, B = randn_pool(gen, n, r, d_in, d_out, dev)
            proj[name] = (A, B, randn_act(gen, T, d_out, dev))
        per_layer.append(({"q": x_attn, "k": x_attn, "v": x_attn, "o": x_o, "gate": x_mlp, "up": x_mlp,
                           "down": x_down}, proj))
    shape_groups = [("q", "o"), ("k", "v"), ("gate", "up"), ("down",)]
    multi = []
    for names in shape_groups:
        probs = [(proj[k][0], proj[k][1], xs[k], proj[k][2]) for xs, proj in per_layer for k in names]
        table, aligned = L.problems_table(probs, dev)
        multi.append((L.Pool(probs[0][0], probs[0][1]), table, aligned))
    slice_groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    sliced = []
    for names in slice_groups:
        groups = [(xs[names[0]], [proj[k] for k in names]) for xs, proj in per_layer]
        table, d_outs, aligned = L.sliced_table(groups, dev)
        sliced.append((L.Pool(groups[0][1][0][0], groups[0][1][0][1]), table, d_outs, aligned))
    plan = L.new_workspace(db, n, dev)
    torch.cuda.synchronize()

    def step_multi(i, ev):
        L.lora_plan_build(db, n, plan)
        if ev: ev[0].record()
        for shape, table, aligned in multi:
            L.lora_apply_multi(shape, db, plan, table, aligned)
        if ev: ev[1].record()

    def step_sliced(i, ev):
        L.lora_plan_build(db, n, plan)
        if ev: ev[0].record()
        for shape, table, d_outs, aligned in sliced:
            L.lora_apply_sliced(shape, db, plan, table, d_outs, aligned)
        if ev: ev[1].record()

    ms_multi = ms_sliced = wall = float("nan")
    if "multi" in modes:
        wall, ms_multi, _ = Timer(steps).run(step_multi, warmup)
    if "sliced" in modes:
        wall, ms_sliced, _ = Timer(steps).run(step_sliced, warmup)
    touched, slot_tokens, distinct = accounting.batch_work(batch.seg_bounds(), batch.idx, n)
    byts = layers * sum(accounting.sliced_call_bytes(touched, distinct, r, dims[names[0]][0],
                                                     [dims[k][1] for k in names], 2) for names in slice_groups)
    flops = layers * sum(accounting.lora_flops(slot_tokens, r, d_in, d_out) for d_in, d_out in dims.values())
    k_ms = ms_sliced if "sliced" in modes else ms_multi
    res = result("llama3-8b stack 32x7 mixed, shared x", wall, steps, touched, byts, flops, k_ms, byts, flops,
                 len(sliced), {"distinct_adapters": distinct})
    res.update({"apply_us_per_shape_multi": round(ms_multi * 1e3, 3), "apply_us_sliced": round(ms_sliced * 1e3, 3),
                "speedup_sliced": ms_multi / ms_sliced,
                "note": "apply_* covers the 4 sliced launches; bytes count each shared x once"})
    return res


def bench_merge_flux(dev, steps, warmup, r=64, layers=57, per_layer=4, d=3072):
    """Merge one rank-r adapter into every attention projection of a FLUX-sized
    model (57 layers x 4 projections of 3072 x 3072, bf16) with one
    lora_merge_multi launch: the page's merge cost model, one read and one write
    of the affected weights.  Alternate steps merge (alpha 1) and unmerge
    (alpha -1), so the weights stay bounded."""
    torch = torch_mod()
    import rank_sgmv_bgmv_amd as L
    gen = torch.Generator(device=dev)
    gen.manual_seed(106)
    mats = []
    for _ in range(layers * per_layer):
        A, B = randn_pool(gen, 1, r, d, d, dev)
        Wm = (torch.randn((d, d), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        mats.append((A, B, Wm))
    table, aligned = L.merge_table(mats, dev)
    assert aligned
    shape = L.Pool(mats[0][0], mats[0][1])
    torch.cuda.synchronize()

    def step(i, ev):
        alpha = 1.0 if i % 2 == 0 else -1.0
        if ev: ev[0].record()
        L.lora_merge_multi(shape, [0], table, aligned, None, alpha)
        if ev: ev[1].record()

    wall, k_ms, _ = Timer(steps).run(step, warmup)
    n = layers * per_layer
    weight_bytes = n * d * d * 2
    k_bytes = 2 * weight_bytes + n * accounting.adapter_bytes(r, d, d, 2)
    flops = n * 2 * d * d * r
    _, page_ms, _ = accounting.lora_costs(d, layers, per_layer, r, 4608)
    return {"workload": f"merge r{r} into {n} projections of {d}x{d} bf16 (FLUX-sized)",
            "ms_per_step": round(wall / steps * 1e3, 5), "merge_ms": round(k_ms, 4),
            "launches_per_step": 1, "bytes_per_step": k_bytes, "GBps": k_bytes / (k_ms * 1e-3) / 1e9,
            "frac_hbm": k_bytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "TFLOPs": flops / (k_ms * 1e-3) / 1e12,
            "roof_ms_at_8TBps": round(k_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
            "page_model_ms_at_3350GBps": round(page_ms, 3)}


def bench_decode_ranks(dev, steps, warmup, layers=8, n=1000, r=64, d=4096, seed=W.SEEDS["C2"]):
    """Decode over pools stored at rank 64 whose adapters have ranks 8, 16, 32
    or 64 (a quarter each): with the pool's rank array (only each adapter's
    own rows and columns are read) and without it (the zero padding is read)."""
    torch = torch_mod()
    import rank_sgmv_bgmv_amd as L
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 7)
    ranks_np = np.random.default_rng(seed).choice([8, 16, 32, 64], size=n).astype(np.int32)
    ranks = torch.from_numpy(ranks_np).to(dev)
    pools = []
    for _ in range(layers):
        A, B = randn_pool(gen, n, r, d, d, dev)
        mask = torch.arange(r, device=dev)[None, :] < ranks[:, None]  # [n][r]
        A.mul_(mask[:, :, None].to(A.dtype))
        B.mul_(mask[:, None, :].to(B.dtype))
        pools.append((A, B))
    xs = [randn_act(gen, 64, d, dev) for _ in range(layers)]
    ys = [randn_act(gen, 64, d, dev) for _ in range(layers)]
    batches = [W.batch_c2(np.random.default_rng([seed, j]), n) for j in range(16)]
    dbs = [dev_batch(b, dev) for b in batches]
    plan = L.new_workspace(dbs[0], n, dev)
    table, aligned = L.problems_table([(A, B, x, y) for (A, B), x, y in zip(pools, xs, ys)], dev)
    out = {}
    for name, shape in (("with_ranks", L.Pool(pools[0][0], pools[0][1], ranks)),
                        ("padded", L.Pool(pools[0][0], pools[0][1]))):
        def step(i, ev, shape=shape):
            db = dbs[i % 16]
            L.lora_plan_build(db, n, plan)
            if ev: ev[0].record()
            L.lora_apply_multi(shape, db, plan, table, aligned)
            if ev: ev[1].record()
        _, k_ms, _ = Timer(steps).run(step, warmup)
        out[name] = k_ms
    used = [batches[i % 16] for i in range(steps)]
    # algorithmic bytes: x, y and each distinct adapter's own rank
    byts = []
    for b in used:
        ids = np.unique(b.idx[b.idx >= 0])
        byts.append(layers * (64 * 3 * d * 2 + sum(int(ranks_np[i]) * 2 * d * 2 for i in ids)))
    k_bytes = float(np.mean(byts))
    return {"workload": f"decode x{layers} layers, rank-64 pools of adapters with ranks 8/16/32/64",
            "apply_us_with_ranks": round(out["with_ranks"] * 1e3, 3), "apply_us_padded": round(out["padded"] * 1e3, 3),
            "bytes_per_launch_own_ranks": k_bytes,
            "GBps_with_ranks": k_bytes / (out["with_ranks"] * 1e-3) / 1e9,
            "speedup_from_ranks": out["padded"] / out["with_ranks"]}


def bench_pool_load(dev, reps=5, n_slots=64, r=64, d=4096, apply_reps=40):
    """Pool slot management: 64 rank-64 adapters (4096 x 4096, bf16, 1 MiB each)
    copied from page-locked host memory into pool slots with lora_pool_load on a
    second stream, alone and while the compute stream runs decode applies (the
    64-token Zipf batch through one 1000-adapter q_proj pool) on other memory."""
    torch = torch_mod()
    import rank_sgmv_bgmv_amd as L
    gen = torch.Generator(device=dev)
    gen.manual_seed(107)
    A = torch.zeros((n_slots, r, d), dtype=torch.bfloat16, device=dev)
    B = torch.zeros((n_slots, d, r), dtype=torch.bfloat16, device=dev)
    dst = L.Pool(A, B)
    hA = torch.randn((n_slots, r, d), dtype=torch.float32).to(torch.bfloat16).pin_memory()
    hB = torch.randn((n_slots, d, r), dtype=torch.float32).to(torch.bfloat16).pin_memory()
    load_bytes = n_slots * accounting.adapter_bytes(r, d, d, 2)
    # the compute job
    cA, cB = randn_pool(gen, 1000, 16, d, d, dev)
    pool = L.Pool(cA, cB)
    b = W.batch_c2(np.random.default_rng(W.SEEDS["C2"]), 1000)
    db = dev_batch(b, dev)
    x, y = randn_act(gen, 64, d, dev), randn_act(gen, 64, d, dev)
    plan = L.new_workspace(db, 1000, dev)
    L.lora_plan_build(db, 1000, plan)
    copy = torch.cuda.Stream(device=dev)  # default priority
    compute = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def loads():
        e0, e1 = ev(), ev()
        e0.record(copy)
        for i in range(n_slots):
            L.lora_pool_load(dst, i, hA[i], hB[i], stream=copy)
        e1.record(copy)
        return e0, e1

    def applies():
        e0, e1 = ev(), ev()
        e0.record(compute)
        for _ in range(apply_reps):
            L.lora_apply_planned(pool, db, plan, x, y)
        e1.record(compute)
        return e0, e1

    res = {"loads_alone": [], "applies_alone": [], "loads_overlapped": [], "applies_overlapped": []}
    for rep in range(reps + 1):
        torch.cuda.synchronize()
        la = loads(); torch.cuda.synchronize()
        aa = applies(); torch.cuda.synchronize()
        lo = loads(); ao = applies(); torch.cuda.synchronize()
        if rep == 0:
            continue  # warm-up
        res["loads_alone"].append(la[0].elapsed_time(la[1]))
        res["applies_alone"].append(aa[0].elapsed_time(aa[1]))
        res["loads_overlapped"].append(lo[0].elapsed_time(lo[1]))
        res["applies_overlapped"].append(ao[0].elapsed_time(ao[1]))
    m = {k: float(np.median(v)) for k, v in res.items()}
    return {"workload": f"load {n_slots} rank-{r} {d}x{d} bf16 adapters from pinned memory into pool slots",
            "bytes": load_bytes, "loads_ms": round(m["loads_alone"], 4),
            "load_GBps": load_bytes / (m["loads_alone"] * 1e-3) / 1e9,
            "ms_per_0.1GB": round(m["loads_alone"] * 0.1e9 / load_bytes, 3),
            "page_ms_per_0.1GB_at_25GBps": 4.0,
            "applies_ms_alone": round(m["applies_alone"], 4),
            "applies_ms_with_loads": round(m["applies_overlapped"], 4),
            "loads_ms_with_applies": round(m["loads_overlapped"], 4),
            "apply_launches": apply_reps}


# -------------------------------------------------------------- cpu baseline --
def cpu_baseline_decode(state, layers_sample=8, min_seconds=12.0):
    """The fp64 oracle on the host for the headline workload: one 64-token
    batch through `layers_sample` distinct layers (only the adapters the batch
    touches are copied to the host; the oracle's work does not depend on the
    others), cycled until `min_seconds` of wall time have passed, scaled to
    tokens/s through 32 layers."""
    import oracle
    torch = torch_mod()
    pools, batches, xs, ys = state
    b = batches[0]
    used = np.unique(b.idx)
    remap = {int(a): i for i, a in enumerate(used)}
    idx = np.vectorize(lambda a: remap[int(a)])(b.idx).astype(np.int32)
    host = []
    for li in range(layers_sample):
        A, B = pools[li]
        sel = torch.from_numpy(used.astype(np.int64)).to(A.device)
        host.append((A.index_select(0, sel).view(torch.int16).cpu().numpy().view(np.uint16),
                     B.index_select(0, sel).view(torch.int16).cpu().numpy().view(np.uint16),
                     xs[li].view(torch.int16).cpu().numpy().view(np.uint16),
                     ys[li].view(torch.int16).cpu().numpy().view(np.uint16)))
    orc = oracle.load()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    calls = 0
    t0 = time.perf_counter()
    while True:
        for A, B, x, y in host:
            orc.apply(W.BF16, A, B, x, y, T=64, S=64, K=1, seg_off=None, idx=idx, nthreads=cores)
        calls += len(host)
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    per_layer = dt / calls
    return {"value": 64 / (per_layer * 32), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one 64-token batch through {layers_sample} of the 32 layers, cycled for {calls} layer calls "
                      f"({dt:.1f} s wall, {cores} threads); tokens/s scaled to 32 layers"}


def copy_calibration(dev, mib=256, reps=5):
    """A plain device copy of known size: each launch reads and writes `mib` MiB.
    Profiled with the FETCH_SIZE / WRITE_SIZE counters it gives the factor that
    turns those counters into HBM bytes for the LoRA kernels."""
    torch = torch_mod()
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": n, "copy_bytes_written": n, "launches": reps}


# --------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="", help="comma list of: decode32,c1,c2,c3,c4,c4x,c5,merge,stacked,ranks,poolload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (the reference kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; requests would shard across GPUs "
                                   "with no exchange, and no multi-GPU path is implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    torch = torch_mod()
    dev = "cuda:0"
    if args.copy_calibration:
        print(json.dumps(copy_calibration(dev)))
        return
    import rank_sgmv_bgmv_amd as L
    L.lib()
    only = set(s for s in args.only.split(",") if s)
    want = lambda k: not only or k in only  # noqa: E731

    variants = {}
    head = state = None
    if want("decode32"):
        log("decode32 ...")
        head, state = bench_decode_layers(dev, args.steps, args.warmup)
    if want("c1"):
        log("c1 ...")
        variants["C1_tiny_fp32"] = bench_single(W.case_c1(), dev, args.steps, args.warmup, "C1 tiny fp32")
    if want("c2"):
        log("c2 ...")
        variants["C2_decode_1layer"] = bench_single(W.case_c2(), dev, args.steps, args.warmup, "C2 decode q_proj 1 layer")
    if want("c3"):
        log("c3 ...")
        variants["C3_prefill_r64"] = bench_single(W.case_c3(), dev, args.steps, args.warmup, "C3 prefill r64")
    if want("c5"):
        for d, r in [(1280, 64), (1280, 128), (640, 64), (640, 128)]:
            log(f"c5 d{d} r{r} ...")
            variants[f"C5_d{d}_r{r}"] = bench_single(W.case_c5(d, r), dev, args.steps, args.warmup,
                                                     f"C5 diffusion d{d} r{r}")
    if want("merge"):
        log("merge ...")
        torch.cuda.empty_cache()
        variants["merge_flux_r64"] = bench_merge_flux(dev, max(6, args.steps // 5), max(2, args.warmup // 5))
    if want("c4x"):
        log("c4 shared x ...")
        torch.cuda.empty_cache()
        modes = tuple(m for m in ("multi", "sliced") if os.environ.get("LORA_BENCH_C4X_MODE", m) == m)
        variants["C4_llama3_8b_shared_x"] = bench_c4_shared_x(dev, max(3, args.steps // 4), max(1, args.warmup // 2),
                                                              modes=modes)
    if want("stacked"):
        log("decode stacked ...")
        torch.cuda.empty_cache()
        variants["decode_stacked_x32"], _ = bench_decode_layers(
            dev, args.steps, args.warmup, make_batch=W.batch_decode_stacked,
            name="decode q_proj, 30% of requests stacking 2-3 adapters,")
    if want("ranks"):
        log("ranks ...")
        torch.cuda.empty_cache()
        variants["decode_mixed_ranks"] = bench_decode_ranks(dev, args.steps, args.warmup)
    if want("poolload"):
        log("pool load ...")
        variants["pool_load_pinned"] = bench_pool_load(dev)
    if want("c4"):
        log("c4 ...")
        torch.cuda.empty_cache()
        variants["C4_llama3_stack"] = bench_c4_stack(dev, max(5, args.steps // 5), max(2, args.warmup // 5))

    cpu = None
    if head is not None and not args.no_cpu_baseline:
        log("cpu baseline ...")
        cpu = cpu_baseline_decode(state)

    if head is None:  # a partial run: report the first variant as the line
        name, head = next(iter(variants.items()))
    line = {
        "metric": "LoRA-delta tokens/s + achieved HBM GB/s (% of peak), decode & prefill SGMV",
        "value": head.get("tokens_per_s"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.get("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init adapters)",
        "config": {"workload": head["workload"] + ": 64 requests x 1 token, Zipf(1.1) over 1000 resident rank-16 "
                                                  "adapters per layer, 4096->4096 bf16, plan + one fused multi-layer "
                                                  "launch per step", "global_batch": 64, "seq_len": 1,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": head.get("apply_GBps", head.get("GBps")), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": (head.get("apply_GBps", head.get("GBps")) or 0.0) / HBM_PEAK_GBS,
                     "traffic": measured_traffic_bytes() if head is not None and "decode" in head["workload"] else None,
                     "kernel": "valu_kernel<bf16, vec, fused> (shrink + expand of every decode tile, one launch for all 32 layers)",
                     "bytes_per_launch": head.get("apply_bytes_per_launch"), "avg_launch_us": head.get("apply_kernel_us")},
        "cpu_baseline": cpu,
        "headline": head,
        "variants": variants,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
