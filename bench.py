#!/usr/bin/env python3
"""Benchmark of the unmerged multi-LoRA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME[,NAME]] [--no-cpu-baseline]

One JSON line on stdout.  The headline workload ("decode q_proj x32 layers")
is the decode batch of the Llama-3-8B q_proj configuration -- 64 requests x 1
token, adapters drawn Zipf(1.1) from a pool of 1000 resident rank-16 adapters
per layer, 4096 -> 4096, bf16 -- taken through the q_proj LoRA of all 32
layers: one step = one plan build (the device scheduler) + one multi-problem
fused launch over the 32 layer pools.  Every step uses a different batch
(cycled from 16 seeded batches).

Timing protocol.  Before every timed step a 1 GiB buffer is read (untimed), so
that neither the L2 caches nor the 256 MB memory-side cache hold anything the
step reads: the step's bytes come from HBM.  HIP events recorded on the
launching stream bracket the plan build and the apply launch of every step;
each record gives the median, p10 and p90 over the steps, and the mean that
the roofline uses.  The same workloads run back to back without the flush are
reported under "warm".  `value` (tokens/s) is 64 tokens over the median
flushed step time (plan + apply).

`roofline` is for the dominant kernel (the fused VALU apply kernel of the
headline): algorithmic bytes per launch over its mean flushed launch time,
against the 8 TB/s HBM peak.  `variants` holds the other workloads (tiny fp32,
one decode layer, long prefill, the Llama-3-8B-shaped stack three ways, the
diffusion multi-adapter cases, merge, ...).  `calibration` holds a 1 GiB copy,
a 1 GiB read and an empty-kernel floor measured in the same run.
`cpu_baseline` times the fp64 oracle on bounded samples on the host cores.
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
import workloads.device as WD  # noqa: E402
from rank_sgmv_bgmv_amd import accounting  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FLUSH_BYTES = 1 << 30

# HBM traffic of the headline kernel per launch, from two rocprofv3 --pmc runs
# of `bench.py --only decode32` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch,
# caches flushed before every step as in the timed runs),
# each scaled by what the same counter reads for a plain copy of known size
# (`bench.py --copy-calibration`: 256 MiB read + 256 MiB written per launch
# reads FETCH_SIZE 131084 KiB and WRITE_SIZE 262144 KiB, so x2.0 and x1.0).
# Valid only for the kernel sources they were taken on: reported as null once
# those sources change.
TRAFFIC_SOURCES = ["rank_sgmv_bgmv_amd/csrc/lora_valu.hip", "rank_sgmv_bgmv_amd/csrc/lora_device.hpp",
                   "rank_sgmv_bgmv_amd/csrc/lora_internal.hpp"]
MEASURED_TRAFFIC = {"sources_sha256_16": "aa7701ba82f8fa85", "fetch_kib": 181167.5, "write_kib": 16384.0,
                    "fetch_scale": 2.0, "write_scale": 1.0}


def sources_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic_bytes():
    m = MEASURED_TRAFFIC
    if sources_hash(TRAFFIC_SOURCES) != m["sources_sha256_16"]:
        return None
    return m["fetch_kib"] * 1024 * m["fetch_scale"] + m["write_kib"] * 1024 * m["write_scale"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ helpers --
def torch_mod():
    import torch
    return torch


def dev_tensor(a, dtype, dev):
    torch = torch_mod()
    if dtype == W.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def dev_batch(b: W.Batch, dev):
    import rank_sgmv_bgmv_amd as L
    idx, seg, sc = WD.batch_tensors(b, dev)
    return L.Batch(b.T, idx, seg, sc)


class Flusher:
    """Reads a 1 GiB device buffer: afterwards the L2 caches and the memory-side
    cache hold that buffer's (clean) lines and nothing a timed step reads."""

    def __init__(self, dev):
        torch = torch_mod()
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.sum()


def stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"median_us": round(float(np.median(a)) * 1e3, 3), "p10_us": round(float(np.percentile(a, 10)) * 1e3, 3),
            "p90_us": round(float(np.percentile(a, 90)) * 1e3, 3), "mean_us": round(float(a.mean()) * 1e3, 3)}


class Timer:
    """K timed steps.  A step is given an `ev(name)` callback that records a HIP
    event on the current stream; the per-step durations between consecutive
    marks are collected.  With a flusher, the caches are flushed before every
    step (outside the events)."""

    def __init__(self, steps, flusher=None):
        self.steps = steps
        self.flusher = flusher

    def run(self, step, warmup):
        torch = torch_mod()
        for i in range(warmup):
            if self.flusher:
                self.flusher()
            step(i, lambda name: None)
        torch.cuda.synchronize()
        marks = []
        t0 = time.perf_counter()
        for i in range(self.steps):
            if self.flusher:
                self.flusher()
            m = []

            def ev(name, m=m):
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                m.append((name, e))
            step(i, ev)
            marks.append(m)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        spans = {}
        for m in marks:
            for (n0, e0), (n1, e1) in zip(m, m[1:]):
                spans.setdefault(f"{n0}->{n1}", []).append(e0.elapsed_time(e1))
            spans.setdefault("step", []).append(m[0][1].elapsed_time(m[-1][1]))
        return wall, spans


def record(name, steps, tokens, k_bytes, k_flops, spans, apply_key, flushed, extra=None):
    """One workload's record: per-step and apply-launch statistics; GB/s and
    TFLOP/s are algorithmic work over the mean apply time (the roofline figure)
    and over the median."""
    apply_ms = spans[apply_key]
    step_ms = spans["step"]
    mean_apply = float(np.mean(apply_ms))
    med_step = float(np.median(step_ms))
    d = {
        "workload": name,
        "flushed": flushed,
        "steps": steps,
        "ms_per_step": round(med_step, 5),
        "tokens_per_s": tokens / (med_step * 1e-3),
        "step": stats(step_ms),
        "apply": stats(apply_ms),
        "apply_bytes_per_launch": k_bytes,
        "apply_flops_per_launch": k_flops,
        "apply_GBps": k_bytes / (mean_apply * 1e-3) / 1e9,
        "apply_frac_hbm": k_bytes / (mean_apply * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "apply_GBps_median": k_bytes / (float(np.median(apply_ms)) * 1e-3) / 1e9,
        "apply_TFLOPs": k_flops / (mean_apply * 1e-3) / 1e12,
    }
    if extra:
        d.update(extra)
    return d


# ---------------------------------------------------------------- workloads --
def bench_decode_layers(dev, steps, warmup, flusher, layers=32, stack=None, make_batch=W.batch_c2,
                        name="decode q_proj"):
    """The decode batch through `layers` q_proj pools: plan + one multi-problem launch per step."""
    import rank_sgmv_bgmv_amd as L
    st = stack or WD.decode_stack(dev, layers=layers, make_batch=make_batch)
    n, r, d = st.n, st.r, st.d
    dbs = [dev_batch(b, dev) for b in st.batches]
    plan = L.new_workspace(dbs[0], n, dev)
    shape = L.Pool(*st.pools[0])
    table, aligned = L.problems_table([(A, B, x, y) for (A, B), x, y in zip(st.pools, st.xs, st.ys)], dev)
    assert aligned

    def step(i, ev):
        db = dbs[i % len(dbs)]
        ev("start")
        L.lora_plan_build(db, n, plan)
        ev("plan")
        L.lora_apply_multi(shape, db, plan, table, aligned)
        ev("apply")

    _, spans = Timer(steps, flusher).run(step, warmup)
    used = [st.batches[i % len(st.batches)] for i in range(steps)]
    distinct = np.mean([len(np.unique(b.idx[b.idx >= 0])) for b in used])
    slot_tokens = np.mean([int((b.idx >= 0).sum()) for b in used])
    k_bytes = layers * accounting.call_bytes(64, distinct, r, d, d, 2)
    k_flops = layers * accounting.lora_flops(slot_tokens, r, d, d)
    res = record(f"{name} x{layers} layers", steps, 64, k_bytes, k_flops, spans, "plan->apply", flusher is not None,
                 {"distinct_adapters_per_layer": float(distinct), "layers": layers,
                  "plan_us": stats(spans["start->plan"])})
    return res, st


def bench_single(case: W.Case, dev, steps, warmup, flusher, name):
    """One adapted layer: plan + fused apply per step."""
    import rank_sgmv_bgmv_amd as L
    A, B = dev_tensor(case.pool.A, case.dtype, dev), dev_tensor(case.pool.B, case.dtype, dev)
    pool = L.Pool(A, B)
    db = dev_batch(case.batch, dev)
    x = dev_tensor(case.x, case.dtype, dev)
    y = dev_tensor(case.y, case.dtype, dev)
    plan = L.new_workspace(db, case.pool.n, dev)

    def step(i, ev):
        ev("start")
        L.lora_plan_build(db, case.pool.n, plan)
        ev("plan")
        L.lora_apply_planned(pool, db, plan, x, y)
        ev("apply")

    _, spans = Timer(steps, flusher).run(step, warmup)
    eb = 2 if case.dtype == W.BF16 else 4
    p = case.pool
    touched, slot_tokens, distinct = accounting.batch_work(case.batch.seg_bounds(), case.batch.idx, p.n)
    k_bytes = accounting.call_bytes(touched, distinct, p.r, p.d_in, p.d_out, eb)
    k_flops = accounting.lora_flops(slot_tokens, p.r, p.d_in, p.d_out)
    res = record(name, steps, touched, k_bytes, k_flops, spans, "plan->apply", flusher is not None,
                 {"tokens": touched, "distinct_adapters": distinct})
    if case.dtype == W.BF16 and p.r >= 64:
        res["apply_frac_mfma_peak"] = res["apply_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS
    return res


def bench_c4_stack(dev, steps, warmup, flusher):
    """Full Llama-3-8B-shaped stack: 32 layers x 7 projections, r=32, 256 adapters per
    projection; mixed 4 x 512 prefill + 256 decode tokens.  One plan per step, then the
    224 projections three ways: one multi-problem launch per projection shape (4
    launches), one lora_apply_planned call per projection (224 launches), and those
    224 calls captured once in a HIP graph and replayed."""
    torch = torch_mod()
    import rank_sgmv_bgmv_amd as L
    st = WD.c4_stack(dev)
    n, r = st.n, st.r
    db = dev_batch(st.batch, dev)
    launches, calls = [], []
    for d_in, d_out, projs in st.groups:
        table, aligned = L.problems_table([(p.A, p.B, p.x, p.y) for p in projs], dev)
        launches.append((L.Pool(projs[0].A, projs[0].B), table, aligned))
        calls += [(L.Pool(p.A, p.B), p.x, p.y) for p in projs]
    plan = L.new_workspace(db, n, dev)
    torch.cuda.synchronize()

    def step_multi(i, ev):
        ev("start")
        L.lora_plan_build(db, n, plan)
        ev("plan")
        for shape, table, aligned in launches:
            L.lora_apply_multi(shape, db, plan, table, aligned)
        ev("apply")

    def step_calls(i, ev):
        ev("start")
        L.lora_plan_build(db, n, plan)
        ev("plan")
        for pool, x, y in calls:
            L.lora_apply_planned(pool, db, plan, x, y)
        ev("apply")

    # the 224 calls captured once (every call's kernels on the capturing stream)
    L.lora_plan_build(db, n, plan)
    for pool, x, y in calls:  # first launches (per-kernel attributes) outside the capture
        L.lora_apply_planned(pool, db, plan, x, y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for pool, x, y in calls:
                L.lora_apply_planned(pool, db, plan, x, y)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()

    def step_graph(i, ev):
        ev("start")
        L.lora_plan_build(db, n, plan)
        ev("plan")
        graph.replay()
        ev("apply")

    touched, slot_tokens, distinct = accounting.batch_work(st.batch.seg_bounds(), st.batch.idx, n)
    byts = flops = 0
    for d_in, d_out, projs in st.groups:
        byts += len(projs) * accounting.call_bytes(touched, distinct, r, d_in, d_out, 2)
        flops += len(projs) * accounting.lora_flops(slot_tokens, r, d_in, d_out)
    out = {}
    for key, fn, what in (("multi", step_multi, "4 multi-problem launches"),
                          ("calls", step_calls, "224 lora_apply_planned calls"),
                          ("graph", step_graph, "224 calls replayed from a HIP graph")):
        _, spans = Timer(steps, flusher).run(fn, warmup)
        out[key] = record(f"llama3-8b stack 32x7 mixed, {what}", steps, touched, byts, flops, spans,
                          "plan->apply", flusher is not None, {"distinct_adapters": distinct})
    res = dict(out["multi"])
    res["note"] = "apply_* covers the whole stack (4 multi-problem launches)"
    res["as_224_calls"] = {k: out["calls"][k] for k in ("apply", "apply_GBps", "apply_frac_hbm")}
    res["as_graph_of_224_calls"] = {k: out["graph"][k] for k in ("apply", "apply_GBps", "apply_frac_hbm")}
    del graph
    return res


def bench_c4_shared_x(dev, steps, warmup, flusher, modes=("multi", "sliced")):
    """The Llama-3-8B-shaped stack with the model's own input sharing, timed two
    ways on the same data: one multi-problem launch per projection shape (q,o |
    k,v | gate,up | down: a shared x is fetched once per projection) and the
    sliced launches (q/k/v | o | gate/up | down).  Bytes: the minimum, with each
    shared x read once."""
    import rank_sgmv_bgmv_amd as L
    st = WD.c4_shared_x(dev)
    n, r, dims = st.n, st.r, st.dims
    db = dev_batch(st.batch, dev)
    shape_groups = [("q", "o"), ("k", "v"), ("gate", "up"), ("down",)]
    multi = []
    for names in shape_groups:
        probs = [(proj[k][0], proj[k][1], xs[k], proj[k][2]) for xs, proj in st.layers for k in names]
        table, aligned = L.problems_table(probs, dev)
        multi.append((L.Pool(probs[0][0], probs[0][1]), table, aligned))
    slice_groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    sliced = []
    for names in slice_groups:
        groups = [(xs[names[0]], [proj[k] for k in names]) for xs, proj in st.layers]
        table, d_outs, aligned = L.sliced_table(groups, dev)
        sliced.append((L.Pool(groups[0][1][0][0], groups[0][1][0][1]), table, d_outs, aligned))
    plan = L.new_workspace(db, n, dev)

    def step_multi(i, ev):
        ev("start")
        L.lora_plan_build(db, n, plan)
        ev("plan")
        for shape, table, aligned in multi:
            L.lora_apply_multi(shape, db, plan, table, aligned)
        ev("apply")

    def step_sliced(i, ev):
        ev("start")
        L.lora_plan_build(db, n, plan)
        ev("plan")
        for shape, table, d_outs, aligned in sliced:
            L.lora_apply_sliced(shape, db, plan, table, d_outs, aligned)
        ev("apply")

    touched, slot_tokens, distinct = accounting.batch_work(st.batch.seg_bounds(), st.batch.idx, n)
    byts = W.LLAMA3_8B_LAYERS * sum(accounting.sliced_call_bytes(touched, distinct, r, dims[names[0]][0],
                                                                 [dims[k][1] for k in names], 2)
                                    for names in slice_groups)
    flops = W.LLAMA3_8B_LAYERS * sum(accounting.lora_flops(slot_tokens, r, d_in, d_out)
                                     for d_in, d_out in dims.values())
    recs = {}
    for key, fn in (("multi", step_multi), ("sliced", step_sliced)):
        if key in modes:
            _, spans = Timer(steps, flusher).run(fn, warmup)
            recs[key] = record(f"llama3-8b stack 32x7 mixed, shared x, {key}", steps, touched, byts, flops, spans,
                               "plan->apply", flusher is not None, {"distinct_adapters": distinct})
    res = dict(recs.get("sliced") or recs["multi"])
    if "multi" in recs and "sliced" in recs:
        res["apply_us_per_shape_multi"] = recs["multi"]["apply"]["median_us"]
        res["apply_us_sliced"] = recs["sliced"]["apply"]["median_us"]
        res["speedup_sliced"] = recs["multi"]["apply"]["median_us"] / recs["sliced"]["apply"]["median_us"]
    res["note"] = "apply_* covers the 4 sliced launches; bytes count each shared x once"
    return res


def bench_merge_flux(dev, steps, warmup, flusher, r=64, layers=57, per_layer=4, d=3072):
    """Merge one rank-r adapter into every attention projection of a FLUX-sized
    model (57 layers x 4 projections of 3072 x 3072, bf16) with one
    lora_merge_multi launch.  Alternate steps merge (alpha 1) and unmerge
    (alpha -1), so the weights stay bounded."""
    import rank_sgmv_bgmv_amd as L
    mats = WD.flux_merge(dev, r=r, layers=layers, per_layer=per_layer, d=d)
    table, aligned = L.merge_table(mats, dev)
    assert aligned
    shape = L.Pool(mats[0][0], mats[0][1])

    def step(i, ev):
        ev("start")
        L.lora_merge_multi(shape, [0], table, aligned, None, 1.0 if i % 2 == 0 else -1.0)
        ev("merge")

    _, spans = Timer(steps, flusher).run(step, warmup)
    n_mats = layers * per_layer
    k_bytes = accounting.merge_bytes(n_mats, d, d, 2) + n_mats * accounting.adapter_bytes(r, d, d, 2)
    flops = n_mats * 2 * d * d * r
    k_ms = float(np.mean(spans["step"]))
    return {"workload": f"merge r{r} into {n_mats} projections of {d}x{d} bf16 (FLUX-sized)",
            "flushed": flusher is not None, "merge": stats(spans["step"]),
            "launches_per_step": 1, "bytes_per_step": k_bytes, "GBps": k_bytes / (k_ms * 1e-3) / 1e9,
            "frac_hbm": k_bytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "TFLOPs": flops / (k_ms * 1e-3) / 1e12,
            "roof_ms_at_8TBps": round(k_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
            "page_model_ms_at_3350GBps": round(accounting.merge_bytes(n_mats, d, d, 2) / 3350e9 * 1e3, 3)}


def bench_decode_ranks(dev, steps, warmup, flusher, layers=8, n=1000, r=64, d=4096, seed=W.SEEDS["C2"]):
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
        A, B = WD.randn_pool(gen, n, r, d, d, dev)
        mask = torch.arange(r, device=dev)[None, :] < ranks[:, None]  # [n][r]
        A.mul_(mask[:, :, None].to(A.dtype))
        B.mul_(mask[:, None, :].to(B.dtype))
        pools.append((A, B))
    xs = [WD.randn_act(gen, 64, d, dev) for _ in range(layers)]
    ys = [WD.randn_act(gen, 64, d, dev) for _ in range(layers)]
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
            ev("start")
            L.lora_apply_multi(shape, db, plan, table, aligned)
            ev("apply")
        _, spans = Timer(steps, flusher).run(step, warmup)
        out[name] = float(np.mean(spans["step"]))
    used = [batches[i % 16] for i in range(steps)]
    byts = []
    for b in used:
        ids = np.unique(b.idx[b.idx >= 0])
        byts.append(layers * (64 * 3 * d * 2 + sum(int(ranks_np[i]) * 2 * d * 2 for i in ids)))
    k_bytes = float(np.mean(byts))
    return {"workload": f"decode x{layers} layers, rank-64 pools of adapters with ranks 8/16/32/64",
            "flushed": flusher is not None,
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
    cA, cB = WD.randn_pool(gen, 1000, 16, d, d, dev)
    pool = L.Pool(cA, cB)
    db = dev_batch(W.batch_c2(np.random.default_rng(W.SEEDS["C2"]), 1000), dev)
    x, y = WD.randn_act(gen, 64, d, dev), WD.randn_act(gen, 64, d, dev)
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


# ------------------------------------------------------------- calibration --
def calibration(dev, reps=20):
    """Same-run reference points: a 1 GiB device copy (read + write), a 1 GiB read
    (a sum), each with the caches flushed first, and the empty-kernel floor (HIP
    events around a one-element fill)."""
    torch = torch_mod()
    flush = Flusher(dev)
    n = FLUSH_BYTES
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    tiny = torch.empty(1, dtype=torch.float32, device=dev)

    def timed(fn, flushed):
        out = []
        for i in range(reps + 2):
            if flushed:
                flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                out.append(e0.elapsed_time(e1))
        return float(np.median(out))

    copy_ms = timed(lambda: dst.copy_(src), True)
    read_ms = timed(lambda: src.sum(), True)
    floor_ms = timed(lambda: tiny.fill_(0.0), False)
    del src, dst
    # The decode headline's adapter stream without its arithmetic
    # (lora_calib_gather_read, include/lora_calib.h): 2688 blocks of 128 KB
    # (one rank-16 4096-wide A or B each, about as many as the 32-layer launch
    # reads) at distinct random block-aligned places of a 4 GiB pool, read (a)
    # one block per workgroup, (b) two per workgroup with a barrier between
    # them and an 8 KB slice read and written back, as a decode work item
    # reads A, then B, and updates one row of y.
    import rank_sgmv_bgmv_amd as L
    blk, n_blk, pool_bytes = 128 << 10, 2688, 4 << 30
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    pick = np.random.default_rng(7).choice(pool_bytes // blk, size=n_blk, replace=False)
    off = torch.from_numpy(pick.astype(np.int64) * blk).to(dev)
    assert int(off.max()) + blk <= pool_bytes
    sink = torch.empty(n_blk, dtype=torch.int32, device=dev)
    rmw = torch.zeros(n_blk // 2 * 8192, dtype=torch.uint8, device=dev)
    one_ms = timed(lambda: L.lora_calib_gather_read(pool, off, 1, blk, sink), True)
    pair_ms = timed(lambda: L.lora_calib_gather_read(pool, off, 2, blk, sink, rmw=rmw, rmw_bytes=8192), True)
    # the same with at most two workgroups per compute unit, as the decode kernel runs
    pair2_ms = timed(lambda: L.lora_calib_gather_read(pool, off, 2, blk, sink, rmw=rmw, rmw_bytes=8192,
                                                      lds_bytes=65536), True)
    del pool, rmw
    pair_bytes = n_blk * blk + 2 * (n_blk // 2) * 8192
    # The 4096-wide rank-64 prefill batch of 32 requests over 8 adapters
    # (16997 rows in 392 tiles of up to 48) as 392 full 48-row tiles, with no
    # arithmetic (lora_calib_tile_stream): x read and y read and written back
    # in the MFMA kernel's stage order with the tile's A and B beside each
    # stage, the same without A and B, and whole rows at a time.
    n_tiles, t_rows, t_rb = 392, 48, 8192
    tx = torch.zeros(n_tiles * t_rows * t_rb, dtype=torch.uint8, device=dev)
    ty = torch.zeros_like(tx)
    tad = torch.zeros(8 * (t_rb // 512 * 32768 + t_rb // 256 * 16384), dtype=torch.uint8, device=dev)
    tsink = torch.empty(n_tiles, dtype=torch.int32, device=dev)
    tiles_ms = {k: timed(lambda o=o, a=a: L.lora_calib_tile_stream(tx, ty, t_rows, t_rb, tsink, order=o, adapters=a,
                                                                   n_adapters=8 if a is not None else 0), True)
                for k, o, a in (("stage_order_with_A_B", 0, tad), ("stage_order", 0, None), ("row_order", 1, None))}
    del tx, ty, tad
    tile_bytes = 3 * n_tiles * t_rows * t_rb
    return {"copy_1GiB_GBps": 2 * n / (copy_ms * 1e-3) / 1e9, "read_1GiB_GBps": n / (read_ms * 1e-3) / 1e9,
            "gather_read": {"what": f"{n_blk} blocks of 128 KB at random places of a 4 GiB pool, one workgroup each",
                            "bytes": n_blk * blk, "us": round(one_ms * 1e3, 3),
                            "GBps": n_blk * blk / (one_ms * 1e-3) / 1e9},
            "decode_skeleton": {"what": f"{n_blk // 2} workgroups, each reading two of those blocks with a barrier "
                                        "between them and reading and writing back 8 KB (a decode work item's "
                                        "A, B and y row, no arithmetic)",
                                "bytes": pair_bytes, "us": round(pair_ms * 1e3, 3),
                                "GBps": pair_bytes / (pair_ms * 1e-3) / 1e9,
                                "two_per_cu_us": round(pair2_ms * 1e3, 3),
                                "two_per_cu_GBps": pair_bytes / (pair2_ms * 1e-3) / 1e9},
            "prefill_tile_skeleton": {"what": f"{n_tiles} tiles of {t_rows} rows of x (read) and y (read and "
                                              f"written back), {t_rb} bytes a row, no arithmetic; "
                                              "stage_order_with_A_B also reads its tile's adapter's A and B "
                                              "(1 MB, 8 adapters) a stage at a time",
                                      "bytes": tile_bytes,
                                      **{f"{k}_us": round(v * 1e3, 3) for k, v in tiles_ms.items()},
                                      **{f"{k}_GBps": tile_bytes / (v * 1e-3) / 1e9 for k, v in tiles_ms.items()}},
            "empty_kernel_floor_us": round(floor_ms * 1e3, 3),
            "note": "torch copy_ and sum, and the library's gather-read probe, each after a cache flush; medians "
                    "of HIP-event times"}


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


# -------------------------------------------------------------- cpu baseline --
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _timed_calls(fn, min_seconds):
    calls = 0
    t0 = time.perf_counter()
    while True:
        fn()
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return dt / calls, calls, dt


def cpu_baseline(stack, seconds=4.0):
    """The fp64 oracle as it stands, on the host cores of this machine, single-
    threaded and on every core: (a) the headline decode -- one 64-token batch
    through one q_proj layer (only the adapters the batch touches are copied to
    the host; the oracle's work does not depend on the others), scaled to 32
    layers; (b) C3 prefill on a sample of 512 of its rows (the first and last
    row of every request and random rows), over the sample."""
    import oracle
    torch = torch_mod()
    orc = oracle.load()
    cores = host_cores()
    b = stack.batches[0]
    used = np.unique(b.idx)
    remap = {int(a): i for i, a in enumerate(used)}
    idx = np.vectorize(lambda a: remap[int(a)])(b.idx).astype(np.int32)
    A, B = stack.pools[0]
    sel = torch.from_numpy(used.astype(np.int64)).to(A.device)
    hA = A.index_select(0, sel).view(torch.int16).cpu().numpy().view(np.uint16)
    hB = B.index_select(0, sel).view(torch.int16).cpu().numpy().view(np.uint16)
    hx = stack.xs[0].view(torch.int16).cpu().numpy().view(np.uint16)
    hy = stack.ys[0].view(torch.int16).cpu().numpy().view(np.uint16)
    out = {}
    for label, nt in (("1_thread", 1), ("all_cores", cores)):
        per, calls, dt = _timed_calls(lambda: orc.apply(W.BF16, hA, hB, hx, hy, T=64, S=64, K=1, seg_off=None,
                                                        idx=idx, nthreads=nt), seconds)
        out[f"decode_{label}"] = {"tokens_per_s": 64 / (per * 32), "layer_call_ms": per * 1e3, "calls": calls,
                                  "threads": nt}
    c3 = W.case_c3()
    rng = np.random.default_rng(1)
    rows = set()
    for lo, hi in c3.batch.seg_bounds():
        rows.update((lo, hi - 1))
    rows.update(int(v) for v in rng.integers(0, c3.batch.T, size=512 - len(rows)))
    rows = np.array(sorted(rows), dtype=np.int32)
    for label, nt in (("1_thread", 1), ("all_cores", cores)):
        per, calls, dt = _timed_calls(lambda: orc.apply_case(c3, rows=rows, nthreads=nt), seconds)
        out[f"prefill_C3_{label}"] = {"tokens_per_s": len(rows) / per, "call_ms_for_sample": per * 1e3,
                                      "sample_rows": int(len(rows)), "calls": calls, "threads": nt}
    head = out["decode_all_cores"]
    return {"value": head["tokens_per_s"], "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": (f"headline decode: one 64-token batch through one q_proj layer ({len(used)} distinct adapters "
                       f"copied to the host), repeated for {seconds:.0f} s per thread count, tokens/s scaled to 32 "
                       f"layers; C3 prefill: {len(rows)} sampled rows of {c3.batch.T}, tokens/s over the sample; "
                       f"value = decode on all {cores} cores"),
            "detail": out}


# --------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="",
                    help="comma list of: decode32,warm,c1,c2,c3,c4,c4x,c5,merge,stacked,ranks,poolload,calib")
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
    flusher = Flusher(dev)
    K, Wm = args.steps, args.warmup

    variants = {}
    head = stack = None
    if want("decode32"):
        log("decode32 ...")
        head, stack = bench_decode_layers(dev, K, Wm, flusher)
    if want("warm"):
        log("decode32 warm ...")
        variants["decode_q_proj_x32_warm"], stack = bench_decode_layers(dev, K, Wm, None, stack=stack)
    if want("c1"):
        log("c1 ...")
        variants["C1_tiny_fp32"] = bench_single(W.case_c1(), dev, K, Wm, flusher, "C1 tiny fp32")
    if want("c2"):
        log("c2 ...")
        c2 = W.case_c2()
        variants["C2_decode_1layer"] = bench_single(c2, dev, K, Wm, flusher, "C2 decode q_proj 1 layer")
        variants["C2_decode_1layer_warm"] = bench_single(c2, dev, K, Wm, None, "C2 decode q_proj 1 layer, warm")
        del c2
    if want("c3"):
        log("c3 ...")
        variants["C3_prefill_r64"] = bench_single(W.case_c3(), dev, K, Wm, flusher, "C3 prefill r64")
    if want("c5"):
        # LORA_BENCH_C5="1280x64,640x128" narrows the sweep (a profiled run per shape)
        c5 = [(1280, 64), (1280, 128), (640, 64), (640, 128)]
        pick = os.environ.get("LORA_BENCH_C5", "")
        if pick:
            c5 = [tuple(int(v) for v in s.split("x")) for s in pick.split(",")]
        for d, r in c5:
            log(f"c5 d{d} r{r} ...")
            variants[f"C5_d{d}_r{r}"] = bench_single(W.case_c5(d, r), dev, K, Wm, flusher, f"C5 diffusion d{d} r{r}")
    if want("stacked"):
        log("decode stacked ...")
        torch.cuda.empty_cache()
        variants["decode_stacked_x32"], _ = bench_decode_layers(
            dev, K, Wm, flusher, make_batch=W.batch_decode_stacked,
            name="decode q_proj, 30% of requests stacking 2-3 adapters,")
    if want("ranks"):
        log("ranks ...")
        torch.cuda.empty_cache()
        variants["decode_mixed_ranks"] = bench_decode_ranks(dev, K, Wm, flusher)
    if want("poolload"):
        log("pool load ...")
        variants["pool_load_pinned"] = bench_pool_load(dev)
    if want("merge"):
        log("merge ...")
        torch.cuda.empty_cache()
        variants["merge_flux_r64"] = bench_merge_flux(dev, max(6, K // 5), max(2, Wm // 5), flusher)
    if want("c4x"):
        log("c4 shared x ...")
        torch.cuda.empty_cache()
        modes = tuple(m for m in ("multi", "sliced") if os.environ.get("LORA_BENCH_C4X_MODE", m) == m)
        variants["C4_llama3_8b_shared_x"] = bench_c4_shared_x(dev, max(5, K // 4), max(2, Wm // 2), flusher, modes)
    if want("c4"):
        log("c4 ...")
        torch.cuda.empty_cache()
        variants["C4_llama3_stack"] = bench_c4_stack(dev, max(5, K // 5), max(2, Wm // 5), flusher)
    calib = None
    if want("calib"):
        log("calibration ...")
        torch.cuda.empty_cache()
        calib = calibration(dev)

    cpu = None
    if stack is not None and not args.no_cpu_baseline:
        log("cpu baseline ...")
        cpu = cpu_baseline(stack)

    if head is None and not variants:  # calibration alone
        print(json.dumps({"calibration": calib}))
        return
    if head is None:  # a partial run: report the first variant as the line
        name, head = next(iter(variants.items()))
    apply = head.get("apply") or {}
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
        "data": "synthetic (seeded; random-init adapters); caches flushed before every timed step",
        "config": {"workload": head["workload"] + ": 64 requests x 1 token, Zipf(1.1) over 1000 resident rank-16 "
                                                  "adapters per layer, 4096->4096 bf16, plan + one fused multi-layer "
                                                  "launch per step", "global_batch": 64, "seq_len": 1,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": head.get("apply_GBps", head.get("GBps")), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": (head.get("apply_GBps", head.get("GBps")) or 0.0) / HBM_PEAK_GBS,
                     "traffic": measured_traffic_bytes() if "decode" in head["workload"] else None,
                     "kernel": "valu_kernel<bf16, vec, fused> (shrink + expand of every decode tile, one launch for "
                               "all 32 layers)",
                     "bytes_per_launch": head.get("apply_bytes_per_launch"), "avg_launch_us": apply.get("mean_us"),
                     "median_launch_us": apply.get("median_us"), "flushed": head.get("flushed"),
                     "same_traffic_no_arithmetic_GBps": (calib or {}).get("decode_skeleton", {}).get("two_per_cu_GBps")},
        "cpu_baseline": cpu,
        "calibration": calib,
        "headline": head,
        "variants": variants,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
