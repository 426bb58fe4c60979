"""GPU tests of the serving-side rows: adapters loaded into pool slots from
pinned host memory (also on a second stream, overlapping applies that use
other slots), and per-step scale schedules on one plan.  Checked against the
fp64 oracle with the tolerances of tests/_gpu.py."""
import numpy as np
import pytest
import torch

import oracle
import rank_sgmv_bgmv_amd as L
import workloads as W
from _gpu import DEV, assert_parity, dev_batch, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _pinned(a: np.ndarray):
    """A page-locked host tensor holding the bf16 bit patterns of `a`."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    p = torch.empty(t.shape, dtype=torch.bfloat16, pin_memory=True)
    p.copy_(t)
    return p


def _case(seed, n, r, d_in, d_out, S, K=1, with_scale=False):
    return W.random_case(seed, dtype=W.BF16, n=n, r=r, d_in=d_in, d_out=d_out, S=S, K=K, min_len=1, max_len=40,
                         with_scale=with_scale)


def test_slots_loaded_from_pinned_memory(orc):
    case = _case(4100, n=6, r=16, d_in=256, d_out=384, S=10, K=2)
    p = case.pool
    A = torch.zeros((p.n, p.r, p.d_in), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((p.n, p.d_out, p.r), dtype=torch.bfloat16, device=DEV)
    pool = L.Pool(A, B)
    host = [(_pinned(p.A[i]), _pinned(p.B[i])) for i in range(p.n)]
    for i, (ah, bh) in enumerate(host):
        L.lora_pool_load(pool, i, ah, bh)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(A, W.BF16), p.A) and np.array_equal(from_dev(B, W.BF16), p.B)
    db = dev_batch(case.batch)
    x, y = to_dev(case.x, W.BF16), to_dev(case.y, W.BF16)
    ws = L.new_workspace(db, p.n, DEV)
    L.lora_apply(pool, db, x, y, ws)
    torch.cuda.synchronize()
    y_ref, touched, _, _ = orc.apply_case(case)
    assert_parity(case, from_dev(y, W.BF16), y_ref, touched, what="pool loaded from pinned memory")


def test_slot_loads_overlap_applies_on_other_slots(orc):
    """Slots 0-2 are resident; slots 3-5 are copied on a second stream while
    the compute stream applies batches that use slots 0-2 only; an event then
    orders a batch that uses slots 3-5 after the copies."""
    n, r, d_in, d_out = 6, 32, 512, 512
    rng = np.random.default_rng(4200)
    full = W.make_pool(rng, W.BF16, n, r, d_in, d_out)
    A = torch.zeros((n, r, d_in), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((n, d_out, r), dtype=torch.bfloat16, device=DEV)
    A[:3].copy_(to_dev(full.A[:3], W.BF16))
    B[:3].copy_(to_dev(full.B[:3], W.BF16))
    pool = L.Pool(A, B)
    host = {i: (_pinned(full.A[i]), _pinned(full.B[i])) for i in range(3, 6)}

    def batch_on(slots, seed):
        g = np.random.default_rng(seed)
        S = 12
        lengths = g.integers(1, 30, size=S)
        idx = g.choice(slots, size=(S, 1)).astype(np.int32)
        return W.Batch(int(lengths.sum()), S, 1, W.offsets_from_lengths(lengths), idx, None)

    old_b, new_b = batch_on([0, 1, 2], 1), batch_on([3, 4, 5], 2)
    xs = {k: W.encode(rng.standard_normal((b.T, d_in)), W.BF16) for k, b in (("old", old_b), ("new", new_b))}
    ys = {k: W.encode(rng.standard_normal((b.T, d_out)), W.BF16) for k, b in (("old", old_b), ("new", new_b))}
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream(device=DEV)  # default priority
    db_old, db_new = dev_batch(old_b), dev_batch(new_b)
    x_old, x_new = to_dev(xs["old"], W.BF16), to_dev(xs["new"], W.BF16)
    y_old = [to_dev(ys["old"], W.BF16) for _ in range(4)]
    y_new = to_dev(ys["new"], W.BF16)
    ws_old, ws_new = L.new_workspace(db_old, n, DEV), L.new_workspace(db_new, n, DEV)
    torch.cuda.synchronize()
    loaded = torch.cuda.Event()
    with torch.cuda.stream(copy):
        for i, (ah, bh) in host.items():
            L.lora_pool_load(pool, i, ah, bh, stream=copy)
        loaded.record(copy)
    for yo in y_old:  # runs while the copies may still be in flight
        L.lora_apply(pool, db_old, x_old, yo, ws_old)
    compute.wait_event(loaded)
    L.lora_apply(pool, db_new, x_new, y_new, ws_new)
    torch.cuda.synchronize()
    for k, b, out in [("old", old_b, from_dev(y_old[-1], W.BF16)), ("new", new_b, from_dev(y_new, W.BF16))]:
        c = W.Case(k, W.BF16, b, full, xs[k], ys[k])
        y_ref, touched, _, _ = orc.apply_case(c)
        assert_parity(c, out, y_ref, touched, what=f"{k} slots")


def test_scale_schedule_reuses_the_plan(orc):
    """"LoRA: merged or alongside", the paragraph on diffusion: a LoRA's weight
    may change with the timestep, which the unmerged form follows by swapping a
    scalar per step.  The plan depends on the offsets and indices only, so one
    plan serves every step of a schedule; each step passes its own scales."""
    case = _case(4300, n=5, r=32, d_in=256, d_out=256, S=8, K=2, with_scale=True)
    p, b = case.pool, case.batch
    A, B = to_dev(p.A, W.BF16), to_dev(p.B, W.BF16)
    pool = L.Pool(A, B)
    idx = torch.from_numpy(b.idx).to(DEV)
    seg = torch.from_numpy(b.seg_off).to(DEV)
    base = L.Batch(b.T, idx, seg, torch.from_numpy(b.scale).to(DEV))
    plan = L.new_workspace(base, p.n, DEV)
    L.lora_plan_build(base, p.n, plan)
    x = to_dev(case.x, W.BF16)
    for step, w in enumerate([1.0, 0.8, 0.5, 0.1, 0.0]):  # a decaying schedule, down to the LoRA off
        sc = (b.scale * np.float32(w)).astype(np.float32)
        batch_t = L.Batch(b.T, idx, seg, torch.from_numpy(sc).to(DEV))
        y = to_dev(case.y, W.BF16)
        L.lora_apply_planned(pool, batch_t, plan, x, y)
        torch.cuda.synchronize()
        c = W.Case(f"step{step}", W.BF16, W.Batch(b.T, b.S, b.K, b.seg_off, b.idx, sc), p, case.x, case.y)
        y_ref, touched, _, _ = orc.apply_case(c)
        assert_parity(c, from_dev(y, W.BF16), y_ref, touched, what=f"schedule step {step} (w={w})")


def test_next_plan_built_on_a_second_stream(orc):
    """A decode loop that builds the plan of step j + 1 on a second stream,
    into the other of two workspaces, while step j's launch runs over three
    layers; events order each plan before its launch and each workspace's
    reuse after the launch that read it.  Every step's outputs match the
    oracle."""
    n, r, d, layers, steps = 60, 16, 512, 3, 6
    rng = np.random.default_rng(4400)
    pool_np = [W.make_pool(rng, W.BF16, n, r, d, d, 0.02) for _ in range(layers)]
    pools = [(to_dev(p.A, W.BF16), to_dev(p.B, W.BF16)) for p in pool_np]
    shape = L.Pool(*pools[0])
    batches = [W.batch_c2(np.random.default_rng([4400, j]), n) for j in range(steps)]
    dbs = [dev_batch(b) for b in batches]
    xy = [[W.make_xy(rng, W.BF16, b.T, d, d, None, None) for _ in range(layers)] for b in batches]
    ys = [[to_dev(y, W.BF16) for _, y in s] for s in xy]
    xs = [[to_dev(x, W.BF16) for x, _ in s] for s in xy]
    tables = [L.problems_table([(A, B, x, y) for (A, B), x, y in zip(pools, xs[j], ys[j])], DEV)[0]
              for j in range(steps)]
    plans = [L.new_workspace(dbs[0], n, DEV) for _ in range(2)]
    main = torch.cuda.current_stream(DEV)
    side = torch.cuda.Stream(device=DEV)
    planned = [torch.cuda.Event() for _ in range(2)]
    consumed = [torch.cuda.Event() for _ in range(2)]

    def build(j):
        with torch.cuda.stream(side):
            side.wait_event(consumed[j % 2])
            L.lora_plan_build(dbs[j], n, plans[j % 2])
            planned[j % 2].record(side)

    build(0)
    for j in range(steps):
        main.wait_event(planned[j % 2])
        L.lora_apply_multi(shape, dbs[j], plans[j % 2], tables[j])
        consumed[j % 2].record(main)
        if j + 1 < steps:
            build(j + 1)
    torch.cuda.synchronize()
    for j, b in enumerate(batches):
        for li, p in enumerate(pool_np):
            x, y = xy[j][li]
            c = W.Case(f"step{j}_layer{li}", W.BF16, b, p, x, y)
            y_ref, touched, _, _ = orc.apply_case(c)
            assert_parity(c, from_dev(ys[j][li], W.BF16), y_ref, touched, what=f"step {j} layer {li}")
