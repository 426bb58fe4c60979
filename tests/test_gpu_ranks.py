"""Adapters of different ranks in one pool ("LoRA: merged or alongside": r is
usually 8 to 128), through the C ABI, against the fp64 oracle with the same
rank array.  Everything past an adapter's rank is filled with NaN: reading
it at all would turn the outputs into NaN, so these tests also show that the
padding is never read (ranks here are multiples of 8 for bf16, 4 for fp32)."""
import numpy as np
import pytest
import torch

import oracle
import rank_sgmv_bgmv_amd as L
import workloads as W
from _gpu import DEV, assert_parity, dev_batch, from_dev, to_dev

pytestmark = pytest.mark.gpu

NAN = {W.BF16: np.uint16(0x7FC0), W.F32: np.float32(np.nan)}


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _poison(pool: W.Pool, ranks):
    A, B = pool.A.copy(), pool.B.copy()
    for i, rk in enumerate(ranks):
        A[i, rk:, :] = NAN[pool.dtype]
        B[i, :, rk:] = NAN[pool.dtype]
    return W.Pool(pool.dtype, pool.n, pool.r, pool.d_in, pool.d_out, A, B)


def _run(case, ranks, split=False):
    p = case.pool
    A, B = to_dev(p.A, case.dtype), to_dev(p.B, case.dtype)
    rk = torch.from_numpy(np.asarray(ranks, np.int32)).to(DEV)
    pool = L.Pool(A, B, rk)
    db = dev_batch(case.batch)
    x, y = to_dev(case.x, case.dtype), to_dev(case.y, case.dtype)
    ws = L.new_workspace(db, p.n, DEV)
    xv, yv = x[:, :p.d_in], y[:, :p.d_out]
    if split:
        v = torch.full((case.batch.T, case.batch.K * p.r), float("nan"), dtype=torch.float32, device=DEV)
        L.lora_shrink(pool, db, xv, v, ws)
        L.lora_expand(pool, db, v, yv, ws)
    else:
        L.lora_apply(pool, db, xv, yv, ws)
    torch.cuda.synchronize()
    return from_dev(y, case.dtype)


CASES = {
    # decode-shaped: every tile on the VALU kernel
    "bf16_decode_r32": (dict(dtype=W.BF16, n=8, r=32, d_in=256, d_out=320, per_token=True, S=48, K=2),
                        [8, 16, 32, 24, 8, 16, 32, 16]),
    # long groups: MFMA tiles (ranks multiples of 16 skip whole 16-wide blocks; 24 masks half of one)
    "bf16_prefill_r64": (dict(dtype=W.BF16, n=4, r=64, d_in=256, d_out=256, S=6, min_len=40, max_len=90),
                         [16, 64, 24, 48]),
    "bf16_prefill_r128_k2": (dict(dtype=W.BF16, n=5, r=128, d_in=128, d_out=128, S=4, K=2, min_len=30,
                                  max_len=80, with_scale=True), [8, 128, 64, 40, 96]),
    "f32_mixed_r16": (dict(dtype=W.F32, n=6, r=16, d_in=64, d_out=96, S=10, K=2, min_len=1, max_len=30,
                           with_scale=True), [4, 16, 8, 12, 4, 16]),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("split", [False, True], ids=["fused", "split"])
def test_ranks_parity(orc, name, split):
    kw, ranks = CASES[name]
    case = W.random_case(5100 + sorted(CASES).index(name), **kw)
    poisoned = _poison(case.pool, ranks)
    c = W.Case(name, case.dtype, case.batch, poisoned, case.x, case.y)
    out = _run(c, ranks, split)
    y_ref, touched, _, _ = orc.apply_case(case, ranks=ranks)  # the oracle never reads the padding either
    assert_parity(case, out, y_ref, touched, what=f"{name} {'split' if split else 'fused'}")


def test_ranks_in_multi_launch_and_merge(orc):
    """The shape's rank array serves every problem of lora_apply_multi; lora_merge
    honours it too (reference: the oracle's merge on the zero-padded pool)."""
    rng = np.random.default_rng(5200)
    n, r, d = 4, 32, 256
    ranks = [8, 32, 16, 24]
    base = W.make_pool(rng, W.BF16, n, r, d, d)
    zero = base.A.copy(), base.B.copy()
    for i, rk in enumerate(ranks):
        zero[0][i, rk:, :] = 0
        zero[1][i, :, rk:] = 0
    poisoned = _poison(base, ranks)
    A, B = to_dev(poisoned.A, W.BF16), to_dev(poisoned.B, W.BF16)
    rk = torch.from_numpy(np.asarray(ranks, np.int32)).to(DEV)
    Wm = W.encode(rng.standard_normal((d, d)), W.BF16)
    Wd = to_dev(Wm, W.BF16)
    L.lora_merge(L.Pool(A, B, rk), [1, 3], Wd, [1.0, -0.5], 1.0)
    torch.cuda.synchronize()
    ref = orc.merge(W.BF16, zero[0], zero[1], Wm, np.array([1, 3], np.int32), np.array([1.0, -0.5], np.float32))
    got = W.decode_f64(from_dev(Wd, W.BF16), W.BF16)
    assert np.all(np.abs(got - ref) <= 1e-2 * (1 + np.abs(ref)))
    # two problems sharing the shape (and its rank array)
    batch = W.batch_c2(rng, n, T=40)
    xs = [W.encode(rng.standard_normal((40, d)), W.BF16) for _ in range(2)]
    ys = [W.encode(rng.standard_normal((40, d)), W.BF16) for _ in range(2)]
    xd, yd = [to_dev(v, W.BF16) for v in xs], [to_dev(v, W.BF16) for v in ys]
    db = dev_batch(batch)
    plan = L.new_workspace(db, n, DEV)
    L.lora_plan_build(db, n, plan)
    table, al = L.problems_table([(A, B, xd[0], yd[0]), (A, B, xd[1], yd[1])], DEV)
    L.lora_apply_multi(L.Pool(A, B, rk), db, plan, table, al)
    torch.cuda.synchronize()
    for q in range(2):
        c = W.Case(f"multi{q}", W.BF16, batch, base, xs[q], ys[q])
        y_ref, touched, _, _ = orc.apply_case(c, ranks=ranks)
        assert_parity(c, from_dev(yd[q], W.BF16), y_ref, touched, what=f"multi problem {q}")


def test_ranks_decode_full_size_sampled(orc):
    """The mixed-rank decode as it is timed: rank-64 pools of 1000 4096 x 4096
    adapters whose ranks are 8, 16, 32 or 64, the 64-token Zipf batch, several
    layers in one multi-problem launch with the pool's rank array.  Every
    element past an adapter's rank is NaN; two layers are checked in full
    against the oracle (on the adapters the batch uses)."""
    layers, n, r, d = 4, 1000, 64, 4096
    ranks_np = np.random.default_rng(W.SEEDS["C2"]).choice([8, 16, 32, 64], size=n).astype(np.int32)
    ranks = torch.from_numpy(ranks_np).to(DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(W.SEEDS["C2"] + 7)

    def rnd(*shape, std=1.0):
        return (torch.randn(shape, generator=gen, device=DEV) * std).to(torch.bfloat16)

    live_rows = torch.arange(r, device=DEV)[None, :] < ranks[:, None]  # [n][r]
    pools = []
    for _ in range(layers):
        A, B = rnd(n, r, d, std=0.02), rnd(n, d, r, std=0.02)
        A.masked_fill_(~live_rows[:, :, None], float("nan"))
        B.masked_fill_(~live_rows[:, None, :], float("nan"))
        pools.append((A, B))
    xs = [rnd(64, d) for _ in range(layers)]
    y0 = [rnd(64, d) for _ in range(layers)]
    ys = [y.clone() for y in y0]
    batch = W.batch_c2(np.random.default_rng(W.SEEDS["C2"]), n)
    db = dev_batch(batch)
    plan = L.new_workspace(db, n, DEV)
    L.lora_plan_build(db, n, plan)
    table, aligned = L.problems_table([(A, B, x, y) for (A, B), x, y in zip(pools, xs, ys)], DEV)
    assert aligned
    L.lora_apply_multi(L.Pool(pools[0][0], pools[0][1], ranks), db, plan, table, aligned)
    torch.cuda.synchronize()
    used = np.unique(batch.idx[batch.idx >= 0])
    remap = np.full(n, -1, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    idx_small = np.where(batch.idx >= 0, remap[np.maximum(batch.idx, 0)], -1).astype(np.int32)
    sel = torch.from_numpy(used.astype(np.int64)).to(DEV)
    for li in (0, layers - 1):
        assert not torch.isnan(ys[li].float()).any(), f"layer {li}: the padding past a rank was read"
        A_s = from_dev(torch.nan_to_num(pools[li][0][sel], nan=0.0), W.BF16)
        B_s = from_dev(torch.nan_to_num(pools[li][1][sel], nan=0.0), W.BF16)
        pool = W.Pool(W.BF16, len(used), r, d, d, A_s, B_s)
        small = W.Batch(64, 64, 1, None, idx_small, None)
        case = W.Case(f"ranks_decode_layer{li}", W.BF16, small, pool, from_dev(xs[li], W.BF16), from_dev(y0[li], W.BF16))
        y_ref, touched, _, _ = orc.apply_case(case, ranks=ranks_np[used])
        assert_parity(case, from_dev(ys[li], W.BF16), y_ref, touched, what=case.name)
