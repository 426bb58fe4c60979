"""GPU parity of lora_apply_sliced: groups of projections that read one x
(attention's query / key / value, an MLP's gate / up) in one launch.

Each slice must equal, within the tolerances of tests/_gpu.py, the fp64
oracle's plain apply of that slice's own pool on the shared x; and, bit for
bit, what one lora_apply_multi launch per slice gives (the same arithmetic
per output: only the order of the work differs).
"""
import numpy as np
import pytest
import torch

import oracle
import rank_sgmv_bgmv_amd as L
import workloads as W
from _gpu import DEV, assert_parity, dev_batch, from_dev, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


class Group:
    """One x and its slices (pool, initial y) on the host and on the device."""

    def __init__(self, rng, dtype, batch, n, r, d_in, d_outs, ranks=None):
        self.dtype = dtype
        self.x, _ = W.make_xy(rng, dtype, batch.T, d_in, 8, ldx=d_in + 8)
        self.pools = [W.make_pool(rng, dtype, n, r, d_in, d) for d in d_outs]
        self.ys = [W.make_xy(rng, dtype, batch.T, 8, d, ldy=d + 8)[1] for d in d_outs]
        self.x_dev = to_dev(self.x, dtype)[:, :d_in]
        self.AB = [(to_dev(p.A, dtype), to_dev(p.B, dtype)) for p in self.pools]
        self.y_dev = [to_dev(y, dtype) for y in self.ys]

    def views(self):
        return [(A, B, y[:, :p.d_out]) for (A, B), y, p in zip(self.AB, self.y_dev, self.pools)]

    def reset(self):
        for yd, y in zip(self.y_dev, self.ys):
            yd.copy_(to_dev(y, self.dtype))


def _run_sliced(groups, db, plan, ranks_dev=None):
    table, d_outs, aligned = L.sliced_table([(g.x_dev, g.views()) for g in groups], DEV)
    A0, B0 = groups[0].AB[0]
    L.lora_apply_sliced(L.Pool(A0, B0, ranks_dev), db, plan, table, d_outs, aligned)
    torch.cuda.synchronize()
    return [[from_dev(y, g.dtype) for y in g.y_dev] for g in groups]


def _run_multi_per_slice(groups, db, plan, ranks_dev=None):
    for p in range(len(groups[0].pools)):
        probs = [(g.AB[p][0], g.AB[p][1], g.x_dev, g.views()[p][2]) for g in groups]
        table, aligned = L.problems_table(probs, DEV)
        L.lora_apply_multi(L.Pool(groups[0].AB[p][0], groups[0].AB[p][1], ranks_dev), db, plan, table, aligned)
    torch.cuda.synchronize()
    return [[from_dev(y, g.dtype) for y in g.y_dev] for g in groups]


def _check_oracle(orc, groups, batch, outs, rows=None, ranks=None):
    for gi, g in enumerate(groups):
        for p, (pool, y0) in enumerate(zip(g.pools, g.ys)):
            case = W.Case(f"group{gi}_slice{p}", g.dtype, batch, pool, g.x, y0)
            y_ref, touched, _, _ = orc.apply_case(case, rows=rows, ranks=ranks)
            assert_parity(case, outs[gi][p], y_ref, touched, rows=rows, what=case.name)


GRID = {
    # decode: one token per request, VALU tiles only
    "qkv_decode_bf16": dict(dtype=W.BF16, n=20, r=16, d_in=512, d_outs=(512, 128, 128), groups=2,
                            batch=dict(per_token=True, S=64, K=1, p_empty=0.1)),
    # prefill: long requests (MFMA tiles) mixed with short ones, two stacked slots
    "qkv_prefill_bf16_mfma": dict(dtype=W.BF16, n=5, r=32, d_in=256, d_outs=(384, 128, 128), groups=2,
                                  batch=dict(S=6, K=2, min_len=1, max_len=200, with_scale=True)),
    "gate_up_prefill_r64": dict(dtype=W.BF16, n=4, r=64, d_in=192, d_outs=(640, 640), groups=1,
                                batch=dict(S=4, K=1, min_len=60, max_len=180, p_empty=0.0)),
    # fp32 vector path, rows outside every request
    "two_slices_f32": dict(dtype=W.F32, n=6, r=8, d_in=72, d_outs=(96, 40), groups=3,
                           batch=dict(S=9, K=1, min_len=0, max_len=20, gaps=True)),
    # widths that are not a multiple of 8: scalar path
    "odd_widths_bf16": dict(dtype=W.BF16, n=4, r=16, d_in=64, d_outs=(100, 36, 20), groups=2,
                            batch=dict(S=7, K=2, min_len=0, max_len=12)),
    # one slot per request on the MFMA path: one walk over x for all slices of a tile
    "four_slices_prefill_r16": dict(dtype=W.BF16, n=5, r=16, d_in=320, d_outs=(128, 64, 192, 64), groups=2,
                                    batch=dict(S=5, K=1, min_len=40, max_len=120, with_scale=True, p_empty=0.1)),
    "two_slices_prefill_r128": dict(dtype=W.BF16, n=4, r=128, d_in=264, d_outs=(384, 136), groups=2,
                                    batch=dict(S=4, K=1, min_len=50, max_len=150)),
    # many slices, one of them narrow
    "eight_slices": dict(dtype=W.BF16, n=3, r=16, d_in=128, d_outs=(64, 128, 8, 64, 256, 64, 64, 128), groups=1,
                         batch=dict(S=5, K=1, min_len=1, max_len=40)),
}


@pytest.mark.parametrize("name", sorted(GRID))
def test_sliced_grid(orc, name):
    cfg = GRID[name]
    rng = np.random.default_rng(5000 + sorted(GRID).index(name))
    batch = W.random_batch(rng, n=cfg["n"], **cfg["batch"])
    groups = [Group(rng, cfg["dtype"], batch, cfg["n"], cfg["r"], cfg["d_in"], cfg["d_outs"])
              for _ in range(cfg["groups"])]
    db = dev_batch(batch)
    plan = L.new_workspace(db, cfg["n"], DEV)
    L.lora_plan_build(db, cfg["n"], plan)
    sliced = _run_sliced(groups, db, plan)
    _check_oracle(orc, groups, batch, sliced)
    for g in groups:
        g.reset()
    multi = _run_multi_per_slice(groups, db, plan)
    for gi in range(len(groups)):
        for p in range(len(cfg["d_outs"])):
            assert np.array_equal(sliced[gi][p], multi[gi][p]), f"group {gi} slice {p}: sliced != per-slice launch"


def test_sliced_fused_output(orc):
    """The slices write disjoint column ranges of one fused output [T][q|k|v]
    with a shared ldy; columns past the last slice keep their bits."""
    rng = np.random.default_rng(5100)
    n, r, d_in, d_outs = 5, 32, 256, (512, 128, 128)
    batch = W.random_batch(rng, n=n, S=5, K=1, min_len=20, max_len=160)
    x, _ = W.make_xy(rng, W.BF16, batch.T, d_in, 8)
    pools = [W.make_pool(rng, W.BF16, n, r, d_in, d) for d in d_outs]
    width = sum(d_outs) + 16
    y0 = W.encode(rng.standard_normal((batch.T, width)), W.BF16)
    xd, yd = to_dev(x, W.BF16), to_dev(y0, W.BF16)
    offs = np.concatenate([[0], np.cumsum(d_outs)])
    slices = []
    for p, pool in enumerate(pools):
        slices.append((to_dev(pool.A, W.BF16), to_dev(pool.B, W.BF16), yd[:, offs[p]:offs[p + 1]]))
    db = dev_batch(batch)
    plan = L.new_workspace(db, n, DEV)
    L.lora_plan_build(db, n, plan)
    table, widths, aligned = L.sliced_table([(xd, slices)], DEV)
    assert aligned and widths == list(d_outs)
    L.lora_apply_sliced(L.Pool(slices[0][0], slices[0][1]), db, plan, table, widths, aligned)
    torch.cuda.synchronize()
    out = from_dev(yd, W.BF16)
    assert np.array_equal(out[:, offs[-1]:], y0[:, offs[-1]:]), "columns past the last slice written"
    for p, pool in enumerate(pools):
        cols = slice(offs[p], offs[p + 1])
        case = W.Case(f"fused_slice{p}", W.BF16, batch, pool, x, np.ascontiguousarray(y0[:, cols]))
        y_ref, touched, _, _ = orc.apply_case(case)
        assert_parity(case, np.ascontiguousarray(out[:, cols]), y_ref, touched, what=case.name)


def test_sliced_with_ranks(orc):
    """Per-adapter ranks apply to every slice; the padding past each adapter's
    rank holds NaN, which must never reach y."""
    rng = np.random.default_rng(5200)
    n, r, d_in, d_outs = 6, 32, 256, (256, 256)
    ranks = np.array([8, 32, 16, 24, 32, 8], np.int32)
    batch = W.random_batch(rng, n=n, S=6, K=2, min_len=1, max_len=150, p_empty=0.1)
    g = Group(rng, W.BF16, batch, n, r, d_in, d_outs)
    for pool, (A, B) in zip(g.pools, g.AB):
        for i, rk in enumerate(ranks):
            pool.A[i, rk:, :] = 0
            pool.B[i, :, rk:] = 0
        A.copy_(to_dev(pool.A, W.BF16))
        B.copy_(to_dev(pool.B, W.BF16))
        for i, rk in enumerate(ranks):
            A[i, rk:, :] = torch.nan
            B[i, :, rk:] = torch.nan
    db = dev_batch(batch)
    plan = L.new_workspace(db, n, DEV)
    L.lora_plan_build(db, n, plan)
    outs = _run_sliced([g], db, plan, torch.from_numpy(ranks).to(DEV))
    _check_oracle(orc, [g], batch, outs, ranks=ranks)


def test_sliced_c4_qkv_sampled(orc):
    """One layer's query / key / value of the Llama-3-8B-shaped stack (4096 ->
    4096 / 1024 / 1024, rank 32, 256 adapters) on the mixed prefill + decode
    batch, one x for all three; sampled rows against the oracle, every row
    against one launch per projection."""
    rng = np.random.default_rng(W.SEEDS["C4"])
    batch = W.batch_c4(rng)
    n, r, d_in = 256, 32, 4096
    d_outs = [d for name, _, d in W.LLAMA3_8B_PROJ if name in ("q", "k", "v")]
    g = Group(np.random.default_rng([W.SEEDS["C4"], 77]), W.BF16, batch, n, r, d_in, d_outs)
    db = dev_batch(batch)
    plan = L.new_workspace(db, n, DEV)
    L.lora_plan_build(db, n, plan)
    sliced = _run_sliced([g], db, plan)
    rows = sample_rows(batch, 24, 11)
    _check_oracle(orc, [g], batch, sliced, rows=rows)
    g.reset()
    multi = _run_multi_per_slice([g], db, plan)
    for p in range(3):
        assert np.array_equal(sliced[0][p], multi[0][p]), f"slice {p}"


def test_sliced_distinct_x(orc):
    """The call allows each slice its own x.  Three groups of three slices on
    the MFMA path: one whose slices share one x (one walk over x for all three),
    one whose slices each read another x, and one where two of three share.
    Each slice against the oracle on its own x, and bit for bit against one
    launch per slice."""
    rng = np.random.default_rng(5300)
    n, r, d_in, d_outs = 6, 32, 256, (256, 128, 96)
    batch = W.random_batch(rng, n=n, S=5, K=1, min_len=30, max_len=120, with_scale=True, p_empty=0.1)
    assert batch.T >= 128  # the MFMA path
    xs = [W.make_xy(rng, W.BF16, batch.T, d_in, 8)[0] for _ in range(4)]
    xs_dev = [to_dev(x, W.BF16) for x in xs]
    x_of = [(0, 0, 0), (1, 2, 3), (1, 1, 2)]  # which x each slice of each group reads
    groups = []
    for gi in range(3):
        pools = [W.make_pool(rng, W.BF16, n, r, d_in, d) for d in d_outs]
        ys = [W.make_xy(rng, W.BF16, batch.T, 8, d)[1] for d in d_outs]
        groups.append((pools, ys, [(to_dev(p.A, W.BF16), to_dev(p.B, W.BF16)) for p in pools],
                       [to_dev(y, W.BF16) for y in ys]))
    db = dev_batch(batch)
    plan = L.new_workspace(db, n, DEV)
    L.lora_plan_build(db, n, plan)
    rows = [(A, B, xs_dev[x_of[gi][p]], yd)
            for gi, (_, _, AB, yds) in enumerate(groups) for p, ((A, B), yd) in enumerate(zip(AB, yds))]
    table, aligned = L.problems_table(rows, DEV)
    A0, B0 = groups[0][2][0]
    L.lora_apply_sliced(L.Pool(A0, B0), db, plan, table, list(d_outs), aligned)
    torch.cuda.synchronize()
    sliced = [[from_dev(yd, W.BF16) for yd in g[3]] for g in groups]
    for gi, (pools, ys, _, _) in enumerate(groups):
        for p, (pool, y0) in enumerate(zip(pools, ys)):
            case = W.Case(f"group{gi}_slice{p}", W.BF16, batch, pool, xs[x_of[gi][p]], y0)
            y_ref, touched, _, _ = orc.apply_case(case)
            assert_parity(case, sliced[gi][p], y_ref, touched, what=case.name)
    for gi, (pools, ys, AB, yds) in enumerate(groups):
        for yd, y in zip(yds, ys):
            yd.copy_(to_dev(y, W.BF16))
    for p in range(len(d_outs)):
        probs = [(g[2][p][0], g[2][p][1], xs_dev[x_of[gi][p]], g[3][p]) for gi, g in enumerate(groups)]
        t, al = L.problems_table(probs, DEV)
        L.lora_apply_multi(L.Pool(groups[0][2][p][0], groups[0][2][p][1]), db, plan, t, al)
    torch.cuda.synchronize()
    for gi, g in enumerate(groups):
        for p, yd in enumerate(g[3]):
            assert np.array_equal(sliced[gi][p], from_dev(yd, W.BF16)), f"group {gi} slice {p}: sliced != per-slice"
