"""GPU parity of the launches the benchmark times, at their full size and in
their launch configuration (the device tensors come from workloads.device, the
builders bench.py uses), against the fp64 oracle on sampled rows:

  * the Llama-3-8B-shaped stack: 4 lora_apply_multi launches of 64, 64, 64 and
    32 problems on one plan (about three VALU work items per workgroup), the
    sliced launches of the shared-x stack, the 224 per-projection calls
    captured in a HIP graph, and the 4 launches captured in one (their second
    stream included);
  * the merge of one rank-64 adapter into 228 FLUX-sized 3072 x 3072 weights
    (about 16 work items per workgroup);
  * the decode batch through 32 q_proj pools of 1000 adapters.

"Serving several LoRAs, ControlNet and IP-Adapter", "Exercises" (four
requests): one kernel covers every group, each result lands in its own row.
"""
import numpy as np
import pytest
import torch

import oracle
import rank_sgmv_bgmv_amd as L
import workloads as W
import workloads.device as WD
from _gpu import DEV, check_problem_sampled, dev_batch, from_dev, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _checked(projs, k=3):
    """First, middle and last layer of a launch's problems."""
    idx = sorted({0, len(projs) // 2, len(projs) - 1})[:k]
    return [projs[i] for i in idx]


def test_c4_stack_multi_launches_as_timed(orc):
    st = WD.c4_stack(DEV)
    db = dev_batch(st.batch)
    plan = L.new_workspace(db, st.n, DEV)
    L.lora_plan_build(db, st.n, plan)
    assert [len(p) for _, _, p in st.groups] == [64, 64, 64, 32]
    rows = sample_rows(st.batch, 48, 41)
    for d_in, d_out, projs in st.groups:
        chk = _checked(projs)
        y0 = [p.y.clone() for p in chk]
        table, aligned = L.problems_table([(p.A, p.B, p.x, p.y) for p in projs], DEV)
        assert aligned
        L.lora_apply_multi(L.Pool(projs[0].A, projs[0].B), db, plan, table, aligned)
        torch.cuda.synchronize()
        for p, y_init in zip(chk, y0):
            check_problem_sampled(orc, st.batch, p.A, p.B, p.x, y_init, p.y, rows,
                                  f"C4 layer {p.layer} {p.name} ({d_in}->{d_out})")
    assert L.lora_read_device_errors(plan) == 0
    del st, plan
    _free()


def test_c4_shared_x_sliced_launches_as_timed(orc):
    st = WD.c4_shared_x(DEV)
    db = dev_batch(st.batch)
    plan = L.new_workspace(db, st.n, DEV)
    L.lora_plan_build(db, st.n, plan)
    rows = sample_rows(st.batch, 40, 42)
    for names in [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]:
        groups = [(xs[names[0]], [proj[k] for k in names]) for xs, proj in st.layers]
        table, d_outs, aligned = L.sliced_table(groups, DEV)
        assert aligned
        chk = sorted({0, len(groups) // 2, len(groups) - 1})
        y0 = {(g, k): groups[g][1][k][2].clone() for g in chk for k in range(len(names))}
        A0, B0 = groups[0][1][0][0], groups[0][1][0][1]
        L.lora_apply_sliced(L.Pool(A0, B0), db, plan, table, d_outs, aligned)
        torch.cuda.synchronize()
        for g in chk:
            x = groups[g][0]
            for k, name in enumerate(names):
                A, B, y = groups[g][1][k]
                check_problem_sampled(orc, st.batch, A, B, x, y0[(g, k)], y, rows, f"sliced layer {g} {name}")
    del st, plan
    _free()


def test_c4_per_projection_calls_in_a_graph(orc):
    """The 224 lora_apply_planned calls of the stack as the benchmark captures
    them in one HIP graph: every replay (with eager work and synchronisations
    between them) must equal the eager calls bit for bit; one projection of each
    shape is also checked against the oracle."""
    st = WD.c4_stack(DEV)
    db = dev_batch(st.batch)
    plan = L.new_workspace(db, st.n, DEV)
    L.lora_plan_build(db, st.n, plan)
    calls = [(L.Pool(p.A, p.B), p) for _, _, projs in st.groups for p in projs]
    y0 = [p.y.clone() for _, p in calls]
    for pool, p in calls:
        L.lora_apply_planned(pool, db, plan, p.x, p.y)
    torch.cuda.synchronize()
    eager = [p.y.clone() for _, p in calls]
    rows = sample_rows(st.batch, 24, 43)
    for _, _, projs in st.groups:
        i = next(k for k, (_, p) in enumerate(calls) if p is projs[-1])
        p = projs[-1]
        check_problem_sampled(orc, st.batch, p.A, p.B, p.x, y0[i], p.y, rows, f"eager call {p.layer} {p.name}")

    def reset():
        for (_, p), y in zip(calls, y0):
            p.y.copy_(y)

    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for pool, p in calls:
                L.lora_apply_planned(pool, db, plan, p.x, p.y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        L.lora_plan_build(db, st.n, plan)  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, ((_, p), want) in enumerate(zip(calls, eager)):
            assert torch.equal(p.y.view(torch.int16), want.view(torch.int16)), f"replay {rep}, call {k}"
    del graph, st, plan, eager, y0
    _free()


def test_c4_multi_launches_in_a_graph_and_against_single_calls():
    """The stack's 4 multi-problem launches run the decode tiles' kernel on a
    second stream beside the prefill tiles' kernel.  Captured in one HIP graph
    (the fork and join are part of the capture), every replay, with eager work
    and synchronisations between them, must equal the eager launches bit for
    bit, and both must equal one lora_apply_planned call per projection (one
    stream) bit for bit on the checked projections."""
    st = WD.c4_stack(DEV)
    db = dev_batch(st.batch)
    plan = L.new_workspace(db, st.n, DEV)
    L.lora_plan_build(db, st.n, plan)
    launches, projs_all = [], []
    for _, _, projs in st.groups:
        table, aligned = L.problems_table([(p.A, p.B, p.x, p.y) for p in projs], DEV)
        launches.append((L.Pool(projs[0].A, projs[0].B), table, aligned))
        projs_all += projs
    y0 = [p.y.clone() for p in projs_all]

    def reset():
        for p, y in zip(projs_all, y0):
            p.y.copy_(y)

    def run_multi():
        for shape, table, aligned in launches:
            L.lora_apply_multi(shape, db, plan, table, aligned)

    run_multi()
    torch.cuda.synchronize()
    eager = [p.y.clone() for p in projs_all]
    chk = sorted({0, 63, 64, 127, 128, 191, 192, 223})
    reset()
    for i in chk:
        p = projs_all[i]
        L.lora_apply_planned(L.Pool(p.A, p.B), db, plan, p.x, p.y)
    torch.cuda.synchronize()
    for i in chk:
        assert torch.equal(projs_all[i].y.view(torch.int16), eager[i].view(torch.int16)), f"single call {i}"
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run_multi()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        L.lora_plan_build(db, st.n, plan)  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (p, want) in enumerate(zip(projs_all, eager)):
            assert torch.equal(p.y.view(torch.int16), want.view(torch.int16)), f"replay {rep}, problem {k}"
    del graph, st, plan, eager, y0
    _free()


def test_merge_flux_multi_as_timed(orc):
    """lora_merge_multi over the 228 FLUX-sized weights the benchmark merges
    (about 16 work items per workgroup): rows of five weights against the
    oracle, then the unmerge of the next step against the merged weights."""
    mats = WD.flux_merge(DEV)
    assert len(mats) == 228
    table, aligned = L.merge_table(mats, DEV)
    assert aligned
    shape = L.Pool(mats[0][0], mats[0][1])
    chk = [0, 57, 113, 170, 227]
    W0 = {i: mats[i][2].clone() for i in chk}
    L.lora_merge_multi(shape, [0], table, aligned, None, 1.0)
    torch.cuda.synchronize()
    merged = {i: mats[i][2].clone() for i in chk}
    for alpha, before, after in ((1.0, W0, merged), (-1.0, merged, None)):
        if alpha < 0:
            L.lora_merge_multi(shape, [0], table, aligned, None, alpha)
            torch.cuda.synchronize()
        for i in chk:
            A, B, Wd = mats[i]
            got = from_dev(Wd if after is None else after[i], W.BF16)
            Ah, Bh, Wh = from_dev(A, W.BF16), from_dev(B, W.BF16), from_dev(before[i], W.BF16)
            for lo in (0, 1531, 3064):
                ref = orc.merge(W.BF16, Ah, Bh, Wh, np.array([0], np.int32), alpha=alpha, rows=(lo, lo + 8))
                g = W.decode_f64(got[lo:lo + 8], W.BF16)
                assert np.all(np.abs(g - ref) <= 1e-2 * (1 + np.abs(ref))), (i, lo, alpha)
    del mats, table
    _free()


def test_decode_x32_as_timed(orc):
    """The headline launch as it is timed: the 64-token Zipf batches through the
    32 q_proj pools of workloads.device.decode_stack, one plan and one
    multi-problem launch each; three of the bench's batches, four layers each
    checked in full against the oracle."""
    st = WD.decode_stack(DEV)
    table, aligned = L.problems_table([(A, B, x, y) for (A, B), x, y in zip(st.pools, st.xs, st.ys)], DEV)
    assert aligned
    shape = L.Pool(*st.pools[0])
    y_init = [y.clone() for y in st.ys]
    for j in (0, 7, 15):
        for y, y0 in zip(st.ys, y_init):
            y.copy_(y0)
        b = st.batches[j]
        db = dev_batch(b)
        plan = L.new_workspace(db, st.n, DEV)
        L.lora_plan_build(db, st.n, plan)
        L.lora_apply_multi(shape, db, plan, table, aligned)
        torch.cuda.synchronize()
        rows = np.arange(64, dtype=np.int32)
        for li in (0, 11, 22, 31):
            A, B = st.pools[li]
            check_problem_sampled(orc, b, A, B, st.xs[li], y_init[li], st.ys[li], rows, f"batch {j} layer {li}")
    del st, table
    _free()
