"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case is seeded and synthetic (workloads/).  Small cases are compared on
every row; the full-size workloads on sampled rows (first and last row of
every request plus random rows), and their routing on every row with the
exact routing probe.  Tolerances are in tests/_gpu.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import rank_sgmv_bgmv_amd as L
import workloads as W
from _gpu import DevCase, assert_parity, dev_batch, from_dev, sample_rows, to_dev, DEV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _rand(seed, **kw):
    return W.random_case(seed, **kw)


# ------------------------------------------------------------------ small --
def test_c1_tiny_fp32(orc):
    case = W.case_c1()
    out = DevCase(case).apply()
    y_ref, touched, _, _ = orc.apply_case(case)
    assert touched.sum() > 0 and (~touched).sum() > 0
    assert_parity(case, out, y_ref, touched, what="C1")


GRID = {
    "bf16_decode_r16": dict(dtype=W.BF16, n=6, r=16, d_in=256, d_out=320, per_token=True, S=40),
    "bf16_mixed_r32_scale": dict(dtype=W.BF16, n=5, r=32, d_in=192, d_out=640, S=10, min_len=0, max_len=40,
                                 with_scale=True),
    "bf16_k3_r16": dict(dtype=W.BF16, n=7, r=16, d_in=128, d_out=512, S=9, K=3, min_len=1, max_len=30,
                        with_scale=True, p_empty=0.3),
    "bf16_k2_r64_chunks": dict(dtype=W.BF16, n=4, r=64, d_in=256, d_out=1024, S=6, K=2, min_len=0, max_len=100),
    "bf16_k4_r128_mfma": dict(dtype=W.BF16, n=6, r=128, d_in=128, d_out=128, S=4, K=4, min_len=20, max_len=90,
                              with_scale=True, p_empty=0.2),
    # three stacked rank-128 slots / six rank-64 slots: the MFMA kernel takes
    # its half-size stages (two workgroups per CU fit in LDS only then); d_in
    # and d_out end inside a stage
    "bf16_k3_r128_half_stages": dict(dtype=W.BF16, n=6, r=128, d_in=200, d_out=200, S=5, K=3, min_len=20,
                                     max_len=150, with_scale=True, p_empty=0.2),
    "bf16_k6_r64_half_stages": dict(dtype=W.BF16, n=8, r=64, d_in=320, d_out=192, S=4, K=6, min_len=30,
                                    max_len=120, p_empty=0.1),
    "bf16_k5_r128_valu": dict(dtype=W.BF16, n=6, r=128, d_in=64, d_out=64, S=3, K=5, min_len=10, max_len=40,
                              p_empty=0.2),
    "bf16_r256": dict(dtype=W.BF16, n=3, r=256, d_in=128, d_out=96, S=5, min_len=1, max_len=30),
    "bf16_r24": dict(dtype=W.BF16, n=4, r=24, d_in=64, d_out=136, S=8, min_len=1, max_len=40, with_scale=True),
    "bf16_scalar_odd": dict(dtype=W.BF16, n=4, r=5, d_in=37, d_out=23, S=6, K=2, min_len=0, max_len=20,
                            with_scale=True),
    "bf16_ld_padded": dict(dtype=W.BF16, n=3, r=32, d_in=128, d_out=256, ldx=136, ldy=272, S=5, min_len=0,
                           max_len=50, gaps=True),
    "bf16_ld_unaligned": dict(dtype=W.BF16, n=3, r=16, d_in=64, d_out=64, ldx=67, ldy=70, S=5, min_len=0,
                              max_len=30),
    "f32_vec_k2": dict(dtype=W.F32, n=5, r=8, d_in=64, d_out=96, per_token=True, S=33, K=2, with_scale=True),
    "f32_scalar_gaps": dict(dtype=W.F32, n=4, r=3, d_in=17, d_out=29, S=7, min_len=0, max_len=12, gaps=True),
    "f32_r64_big_groups": dict(dtype=W.F32, n=3, r=64, d_in=64, d_out=80, S=4, min_len=20, max_len=70),
    "bf16_hot_per_token_mfma": dict(dtype=W.BF16, n=3, r=16, d_in=512, d_out=1024, per_token=True, S=300),
    "bf16_partial_chunks": dict(dtype=W.BF16, n=3, r=64, d_in=200, d_out=136, S=4, min_len=30, max_len=90),
    "bf16_wide_out_chunks": dict(dtype=W.BF16, n=3, r=16, d_in=256, d_out=4096, S=2, min_len=1, max_len=3),
    "bf16_gaps_empty_slots": dict(dtype=W.BF16, n=8, r=32, d_in=96, d_out=160, S=12, K=2, min_len=0, max_len=25,
                                  gaps=True, p_empty=0.5, with_scale=True),
    # fewer than 128 rows: the VALU kernel also takes the groups of >= 17 rows
    "bf16_small_batch_long_groups": dict(dtype=W.BF16, n=2, r=16, d_in=256, d_out=512, S=3, min_len=20,
                                         max_len=40, with_scale=True),
}


@pytest.mark.parametrize("name", sorted(GRID))
def test_random_grid(orc, name):
    case = _rand(1000 + sorted(GRID).index(name), **GRID[name])
    out = DevCase(case).apply()
    y_ref, touched, _, _ = orc.apply_case(case)
    assert_parity(case, out, y_ref, touched, what=name)


# ------------------------------------------------------- exact routing probe --
def _routing_expect(orc, batch: W.Batch, n: int):
    """Oracle routing for every row (cheap: the routing does not depend on the pool)."""
    z = np.zeros((n, 1, 1), np.float32)
    _, touched, routing, _ = orc.apply(W.F32, z, z, np.zeros((batch.T, 1), np.float32),
                                       np.zeros((batch.T, 1), np.float32), T=batch.T, S=batch.S, K=batch.K,
                                       seg_off=batch.seg_off, idx=batch.idx)
    return touched, routing


def _routing_run(dtype, batch: W.Batch, n, r, d_in, d_out):
    """x = e_0, A_i[0][0] = 1, B_i[o][0] = [o == i], y = 0 on touched rows and
    sentinels elsewhere: y_out[t] is the multi-hot vector of the adapters applied."""
    td = torch.bfloat16 if dtype == W.BF16 else torch.float32
    A = torch.zeros((n, r, d_in), dtype=td, device=DEV)
    A[:, 0, 0] = 1
    B = torch.zeros((n, d_out, r), dtype=td, device=DEV)
    ar = torch.arange(n, device=DEV)
    B[ar, ar, 0] = 1
    x = torch.zeros((batch.T, d_in), dtype=td, device=DEV)
    x[:, 0] = 1
    y = torch.zeros((batch.T, d_out), dtype=td, device=DEV)
    db = dev_batch(batch)
    ws = L.new_workspace(db, n, DEV)
    return A, B, x, y, db, ws


@pytest.mark.parametrize("which", ["C1", "C2", "C3", "C4_k", "C5_d640_r64", "bf16_k3"])
def test_routing_probe_exact(orc, which):
    rng = np.random.default_rng(7)
    if which == "C1":
        c = W.case_c1(); b, n, r, d_in, d_out, dt = c.batch, 4, 8, 256, 256, W.F32
    elif which == "C2":
        b, n, r, d_in, d_out, dt = W.batch_c2(np.random.default_rng(W.SEEDS["C2"])), 1000, 16, 4096, 4096, W.BF16
    elif which == "C3":
        b, n, r, d_in, d_out, dt = W.batch_c3(np.random.default_rng(W.SEEDS["C3"])), 8, 64, 4096, 4096, W.BF16
    elif which == "C4_k":
        b, n, r, d_in, d_out, dt = W.batch_c4(np.random.default_rng(W.SEEDS["C4"])), 256, 32, 4096, 1024, W.BF16
    elif which == "C5_d640_r64":
        b, n, r, d_in, d_out, dt = W.batch_c5(np.random.default_rng(W.SEEDS["C5"])), 200, 64, 640, 640, W.BF16
    else:
        b = W.random_batch(rng, S=20, K=3, n=9, min_len=0, max_len=60, p_empty=0.4, gaps=True)
        n, r, d_in, d_out, dt = 9, 16, 64, 64, W.BF16
    touched, routing = _routing_expect(orc, b, n)
    A, B, x, y, db, ws = _routing_run(dt, b, n, r, d_in, d_out)
    # sentinel untouched rows: -0.0 everywhere
    sent = torch.tensor(~touched, device=DEV)
    y[sent] = -0.0
    L.lora_apply(L.Pool(A, B), db, x, y, ws)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()
    expect = np.zeros((b.T, d_out), np.float32)
    for k in range(b.K):
        rows = np.nonzero(routing[:, k] >= 0)[0]
        np.add.at(expect, (rows, routing[rows, k]), 1.0)
    # exact on touched rows, and untouched rows still carry -0.0
    assert np.array_equal(got[touched], expect[touched])
    if (~touched).any():
        u = got[~touched]
        assert np.all(u == 0) and np.all(np.signbit(u))


# ---------------------------------------------------- integer-exact probe --
@pytest.mark.parametrize("name", ["bf16_mixed_r32_scale", "bf16_k4_r128_mfma", "bf16_decode_r16", "bf16_r256",
                                  "f32_vec_k2", "bf16_hot_per_token_mfma"])
def test_integer_probe_bitwise(orc, name):
    base = _rand(2000 + len(name), **GRID[name])
    if base.batch.scale is not None:  # scales that keep every product exact
        g = np.random.default_rng(5)
        b = dataclasses.replace(base.batch, scale=g.choice([-2.0, 1.0, 2.0], size=base.batch.scale.shape).astype(np.float32))
        base = dataclasses.replace(base, batch=b)
    case = W.integer_probe(31, base)
    out = DevCase(case).apply()
    y_ref, touched, _, _ = orc.apply_case(case)
    want = W.encode(y_ref.astype(np.float32), case.dtype)  # exact integers -> one RNE rounding
    d_out = case.pool.d_out
    assert np.array_equal(out[touched][:, :d_out], want[touched]), name
    assert np.array_equal(out[~touched], case.y[~touched])


def test_untouched_sentinels_bitwise(orc):
    base = _rand(3001, dtype=W.BF16, n=4, r=16, d_in=64, d_out=64, S=10, K=2, min_len=0, max_len=20, gaps=True,
                 p_empty=0.5)
    _, touched, _, _ = orc.apply_case(base)
    case = W.sentinel_rows(base, np.nonzero(~touched)[0])
    out = DevCase(case).apply()
    assert np.array_equal(out[~touched].view(np.uint16), case.y[~touched].view(np.uint16))


# ------------------------------------------------------- full-size workloads --
def test_c2_decode_full(orc):
    case = W.case_c2()
    out = DevCase(case).apply()
    y_ref, touched, _, _ = orc.apply_case(case)
    assert touched.all()
    assert_parity(case, out, y_ref, touched, what="C2")


def test_c3_prefill_sampled(orc):
    case = W.case_c3()
    dc = DevCase(case)
    out = dc.apply()
    rows = sample_rows(case.batch, 64, 3)
    y_ref, touched, _, _ = orc.apply_case(case, rows=rows)
    assert_parity(case, out, y_ref, touched, rows=rows, what="C3")


def test_c3_stacked_sampled(orc):
    """C3's lengths and pools with a third of the requests stacking a second,
    scaled adapter and one request with none: the long groups take the 48-row
    prefill tiling, with tiles that span requests and tiles with two slots."""
    base = W.case_c3()
    rng = np.random.default_rng(9103)
    S = base.batch.S
    idx = np.full((S, 2), -1, np.int32)
    idx[:, 0] = base.batch.idx[:, 0]
    for s in rng.choice(S, size=S // 3, replace=False):
        idx[s, 1] = (idx[s, 0] + 1 + int(rng.integers(0, 7))) % base.pool.n
    idx[int(rng.integers(0, S)), :] = -1
    scale = rng.uniform(0.5, 1.5, (S, 2)).astype(np.float32)
    batch = W.Batch(base.batch.T, S, 2, base.batch.seg_off, idx, scale)
    case = W.Case("C3_stacked", W.BF16, batch, base.pool, base.x, base.y)
    out = DevCase(case).apply()
    rows = sample_rows(batch, 64, 4)
    y_ref, touched, _, _ = orc.apply_case(case, rows=rows)
    assert not touched.all(), "the request with no adapter must stay untouched"
    assert_parity(case, out, y_ref, touched, rows=rows, what="C3 stacked")


@pytest.mark.parametrize("d,r", [(1280, 64), (1280, 128), (640, 64), (640, 128)])
def test_c5_diffusion_sampled(orc, d, r):
    case = W.case_c5(d, r)
    out = DevCase(case).apply()
    rows = sample_rows(case.batch, 48, 5)
    y_ref, touched, _, _ = orc.apply_case(case, rows=rows)
    assert_parity(case, out, y_ref, touched, rows=rows, what=case.name)


def test_decode_x32_multi_sampled(orc):
    """The decode launch as it is timed: the 64-token Zipf batch through 32
    q_proj pools (1000 rank-16 adapters of 4096x4096 each) in one multi-problem
    launch sharing one plan.  Launched twice from the same y: the second launch
    must reproduce the first bit for bit (no row's sums depend on which
    workgroup ran it, or when).  Four layers are checked against the oracle in
    full."""
    layers, n, r, d = 32, 1000, 16, 4096
    gen = torch.Generator(device=DEV)
    gen.manual_seed(W.SEEDS["C2"])
    batch = W.batch_c2(np.random.default_rng(W.SEEDS["C2"]), n)

    def rnd(*shape, std=1.0):
        return (torch.randn(shape, generator=gen, device=DEV) * std).to(torch.bfloat16)

    pools = [(rnd(n, r, d, std=0.02), rnd(n, d, r, std=0.02)) for _ in range(layers)]
    xs = [rnd(64, d) for _ in range(layers)]
    y0 = [rnd(64, d) for _ in range(layers)]
    ys = [y.clone() for y in y0]
    db = dev_batch(batch)
    plan = L.new_workspace(db, n, DEV)
    L.lora_plan_build(db, n, plan)
    table, aligned = L.problems_table([(A, B, x, y) for (A, B), x, y in zip(pools, xs, ys)], DEV)
    assert aligned
    shape = L.Pool(*pools[0])
    L.lora_apply_multi(shape, db, plan, table, aligned)
    torch.cuda.synchronize()
    first = [y.clone() for y in ys]
    for y, y_init in zip(ys, y0):
        y.copy_(y_init)
    L.lora_apply_multi(shape, db, plan, table, aligned)
    torch.cuda.synchronize()
    for li in range(layers):
        assert torch.equal(ys[li].view(torch.int16), first[li].view(torch.int16)), f"layer {li}"
    used = np.unique(batch.idx[batch.idx >= 0])
    remap = np.full(n, -1, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    idx_small = np.where(batch.idx >= 0, remap[np.maximum(batch.idx, 0)], -1).astype(np.int32)
    sel = torch.from_numpy(used.astype(np.int64)).to(DEV)
    for li in (0, 9, 20, 31):
        A_s, B_s = from_dev(pools[li][0][sel], W.BF16), from_dev(pools[li][1][sel], W.BF16)
        pool = W.Pool(W.BF16, len(used), r, d, d, A_s, B_s)
        small = W.Batch(64, 64, 1, None, idx_small, None)
        case = W.Case(f"decode_x32_layer{li}", W.BF16, small, pool, from_dev(xs[li], W.BF16),
                      from_dev(y0[li], W.BF16))
        y_ref, touched, _, _ = orc.apply_case(case)
        assert_parity(case, from_dev(ys[li], W.BF16), y_ref, touched, what=case.name)


def test_decode_stacked_multi_sampled(orc):
    """The stacked decode launch as it is timed: 64 one-token requests, 30% of
    them stacking 2-3 Zipf adapters, rank-16 4096 x 4096 pools of 1000
    adapters, several layers in one multi-problem launch; two layers checked
    in full against the oracle (on the adapters the batch uses)."""
    layers, n, r, d = 4, 1000, 16, 4096
    gen = torch.Generator(device=DEV)
    gen.manual_seed(W.SEEDS["C2"] + 11)
    batch = W.batch_decode_stacked(np.random.default_rng([W.SEEDS["C2"], 0]), n)

    def rnd(*shape, std=1.0):
        return (torch.randn(shape, generator=gen, device=DEV) * std).to(torch.bfloat16)

    pools = [(rnd(n, r, d, std=0.02), rnd(n, d, r, std=0.02)) for _ in range(layers)]
    xs = [rnd(64, d) for _ in range(layers)]
    y0 = [rnd(64, d) for _ in range(layers)]
    ys = [y.clone() for y in y0]
    db = dev_batch(batch)
    plan = L.new_workspace(db, n, DEV)
    L.lora_plan_build(db, n, plan)
    table, aligned = L.problems_table([(A, B, x, y) for (A, B), x, y in zip(pools, xs, ys)], DEV)
    assert aligned
    L.lora_apply_multi(L.Pool(*pools[0]), db, plan, table, aligned)
    torch.cuda.synchronize()
    used = np.unique(batch.idx[batch.idx >= 0])
    remap = np.full(n, -1, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    idx_small = np.where(batch.idx >= 0, remap[np.maximum(batch.idx, 0)], -1).astype(np.int32)
    sel = torch.from_numpy(used.astype(np.int64)).to(DEV)
    for li in (0, layers - 1):
        A_s, B_s = from_dev(pools[li][0][sel], W.BF16), from_dev(pools[li][1][sel], W.BF16)
        pool = W.Pool(W.BF16, len(used), r, d, d, A_s, B_s)
        small = W.Batch(64, 64, batch.K, None, idx_small, None)
        case = W.Case(f"decode_stacked_layer{li}", W.BF16, small, pool, from_dev(xs[li], W.BF16),
                      from_dev(y0[li], W.BF16))
        y_ref, touched, _, _ = orc.apply_case(case)
        assert_parity(case, from_dev(ys[li], W.BF16), y_ref, touched, what=case.name)


def _c4_layer(layer_seed=0):
    """One layer of the Llama-3-8B-shaped stack: the batch (shared) and 7 projection cases."""
    rng = np.random.default_rng(W.SEEDS["C4"])
    batch = W.batch_c4(rng)
    cases = []
    for pi, (name, d_in, d_out) in enumerate(W.LLAMA3_8B_PROJ):
        g = np.random.default_rng([W.SEEDS["C4"], layer_seed, pi])
        pool = W.make_pool(g, W.BF16, 256, 32, d_in, d_out)
        x, y = W.make_xy(g, W.BF16, batch.T, d_in, d_out)
        cases.append(W.Case(f"C4_{name}", W.BF16, batch, pool, x, y))
    return batch, cases


def test_c4_layer_sampled_and_multi(orc):
    batch, cases = _c4_layer()
    db = dev_batch(batch)
    plan = L.new_workspace(db, 256, DEV)
    L.lora_plan_build(db, 256, plan)
    rows = sample_rows(batch, 40, 9)
    outs = {}
    for case in cases:
        dc = DevCase(case)
        L.lora_apply_planned(dc.pool, db, plan, dc.x, dc.y)
        torch.cuda.synchronize()
        out = from_dev(dc.y_full, W.BF16)
        outs[case.name] = out
        y_ref, touched, _, _ = orc.apply_case(case, rows=rows)
        assert_parity(case, out, y_ref, touched, rows=rows, what=case.name)
    # q and o share a shape: one multi-problem launch equals two planned calls bit for bit
    dq, do = DevCase(cases[0]), DevCase(cases[3])
    table, aligned = L.problems_table([(dq.A, dq.B, dq.x, dq.y), (do.A, do.B, do.x, do.y)], DEV)
    assert aligned
    L.lora_apply_multi(dq.pool, db, plan, table, aligned)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dq.y_full, W.BF16), outs["C4_q"])
    assert np.array_equal(from_dev(do.y_full, W.BF16), outs["C4_o"])


# ------------------------------------------------------------- split API --
@pytest.mark.parametrize("name", ["bf16_k3_r16", "bf16_k4_r128_mfma", "f32_vec_k2", "bf16_scalar_odd",
                                  "bf16_hot_per_token_mfma"])
def test_shrink_expand(orc, name):
    case = _rand(4000 + len(name), **GRID[name])
    dc = DevCase(case)
    p, b = case.pool, case.batch
    KR = b.K * p.r
    ldv = KR + 4
    sentinel = -12345.0
    v = torch.full((b.T, ldv), sentinel, dtype=torch.float32, device=DEV)
    L.lora_shrink(dc.pool, dc.batch, dc.x, v[:, :KR], dc.ws)
    torch.cuda.synchronize()
    vg = v.cpu().numpy()
    v_ref, touched = orc.shrink_case(case)
    assert np.all(vg[~touched] == sentinel) and np.all(vg[:, KR:] == sentinel)
    tol = 1e-4 if case.dtype == W.BF16 else 1e-5
    err = np.abs(vg[touched, :KR] - v_ref[touched])
    assert np.all(err <= tol * (1 + np.abs(v_ref[touched]))), np.max(err)
    # expand with the oracle's own intermediate (rounded to fp32) as the shared input
    v_in = np.full((b.T, ldv), 0.0, np.float32)
    v_in[:, :KR] = v_ref.astype(np.float32)
    vt = torch.from_numpy(v_in).to(DEV)
    L.lora_expand(dc.pool, dc.batch, vt[:, :KR], dc.y, dc.ws)
    torch.cuda.synchronize()
    out = from_dev(dc.y_full, case.dtype)
    y_ref, touched2 = orc.expand(case.dtype, p.B, v_in[:, :KR], case.y, T=b.T, S=b.S, K=b.K, seg_off=b.seg_off,
                                 idx=b.idx)
    assert np.array_equal(touched, touched2)
    assert_parity(case, out, y_ref, touched2, what=name + " expand")
    # expand(shrink(x)) is the fused result, within tolerance of the oracle
    dc.reset_y()
    L.lora_expand(dc.pool, dc.batch, v[:, :KR], dc.y, dc.ws)
    torch.cuda.synchronize()
    y_ref3, t3, _, _ = orc.apply_case(case)
    assert_parity(case, from_dev(dc.y_full, case.dtype), y_ref3, t3, what=name + " compose")


# --------------------------------------------------- plans and properties --
def test_planned_equals_oneshot_and_deterministic(orc):
    case = _rand(5001, **GRID["bf16_mixed_r32_scale"])
    dc = DevCase(case)
    out1 = dc.apply()
    dc.reset_y()
    out2 = dc.apply()
    assert np.array_equal(out1, out2)
    dc.reset_y()
    plan = L.new_workspace(dc.batch, case.pool.n, DEV)
    L.lora_plan_build(dc.batch, case.pool.n, plan)
    L.lora_apply_planned(dc.pool, dc.batch, plan, dc.x, dc.y)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dc.y_full, case.dtype), out1)


def test_permutation_equivariance_bitwise(orc):
    case = _rand(5002, **GRID["bf16_mixed_r32_scale"])
    b = case.batch
    perm = np.random.default_rng(1).permutation(b.S)
    bounds = b.seg_bounds()
    rows = np.concatenate([np.arange(*bounds[s]) for s in perm]).astype(np.int64)
    lengths = [bounds[s][1] - bounds[s][0] for s in perm]
    b2 = W.Batch(len(rows), b.S, b.K, W.offsets_from_lengths(lengths), b.idx[perm].copy(), b.scale[perm].copy())
    c2 = W.Case("perm", case.dtype, b2, case.pool, case.x[rows].copy(), case.y[rows].copy())
    o1 = DevCase(case).apply()
    o2 = DevCase(c2).apply()
    assert np.array_equal(o2, o1[rows])


@pytest.mark.parametrize("name", ["bf16_decode_r16", "bf16_hot_per_token_mfma"])
def test_per_token_permutation_bitwise(orc, name):
    """Shuffling the rows of a decode batch regroups them into different tiles;
    each row's result must not change by a single bit."""
    case = _rand(5005, **GRID[name])
    b = case.batch
    assert b.seg_off is None
    perm = np.random.default_rng(2).permutation(b.T)
    b2 = W.Batch(b.T, b.S, b.K, None, b.idx[perm].copy(), None if b.scale is None else b.scale[perm].copy())
    c2 = W.Case("perm", case.dtype, b2, case.pool, case.x[perm].copy(), case.y[perm].copy())
    o1 = DevCase(case).apply()
    o2 = DevCase(c2).apply()
    assert np.array_equal(o2, o1[perm])


def test_invalid_indices_are_skipped_and_counted(orc):
    case = _rand(5003, dtype=W.BF16, n=5, r=16, d_in=64, d_out=64, S=12, K=2, min_len=1, max_len=10,
                 p_invalid=0.25, p_empty=0.2)
    bad = (case.batch.idx < -1) | (case.batch.idx >= 5)
    assert bad.sum() > 0
    dc = DevCase(case)
    out = dc.apply()
    assert L.lora_read_device_errors(dc.ws) == int(bad.sum())
    idx_ok = np.where(bad, -1, case.batch.idx).astype(np.int32)
    ref_case = dataclasses.replace(case, batch=dataclasses.replace(case.batch, idx=idx_ok))
    y_ref, touched, _, _ = orc.apply_case(ref_case)
    assert_parity(case, out, y_ref, touched, what="invalid indices")


def test_bad_offsets_are_clamped_and_counted(orc):
    case = _rand(5004, dtype=W.BF16, n=4, r=16, d_in=64, d_out=64, S=6, min_len=2, max_len=8)
    seg = case.batch.seg_off.copy()
    T = case.batch.T
    seg[2], seg[3] = seg[3], seg[2] - 1       # offsets 2..3 go down
    seg[-1] = T + 5                           # beyond T
    sane = np.minimum(np.maximum.accumulate(np.maximum(seg, 0)), T).astype(np.int32)
    bad_batch = dataclasses.replace(case.batch, seg_off=seg)
    dc = DevCase(dataclasses.replace(case, batch=bad_batch))
    out = dc.apply()
    assert L.lora_read_device_errors(dc.ws) == 2
    y_ref, touched, _, _ = orc.apply_case(dataclasses.replace(case, batch=dataclasses.replace(case.batch, seg_off=sane)))
    assert_parity(case, out, y_ref, touched, what="clamped offsets")


def test_empty_and_degenerate_batches(orc):
    for kw in [dict(S=0), dict(S=5, min_len=0, max_len=0), dict(S=6, p_empty=1.0, min_len=1, max_len=5),
               dict(per_token=True, S=0)]:
        case = _rand(6000, dtype=W.BF16, n=3, r=16, d_in=64, d_out=64, **kw)
        dc = DevCase(case)
        out = dc.apply()
        assert np.array_equal(out, case.y), kw
