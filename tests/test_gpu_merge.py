"""GPU parity of lora_merge (merge / unmerge of stacked adapters into a weight)
against the fp64 oracle, through the C ABI.

Tolerances as for the apply path (tests/_gpu.py): bf16 |W_gpu - W_ref| <=
1e-2 (1 + |W_ref|), fp32 1e-5 (1 + |W_ref|), elementwise; columns past d_in
(ldw > d_in) must keep their bits.
"""
import numpy as np
import pytest
import torch

import oracle
import rank_sgmv_bgmv_amd as L
import workloads as W
from _gpu import DEV, TOL, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _case(seed, dtype, n, r, d_in, d_out, K, ldw=None, with_scale=True, p_empty=0.0):
    rng = np.random.default_rng(seed)
    pool = W.make_pool(rng, dtype, n, r, d_in, d_out)
    ldw = d_in if ldw is None else ldw
    Wm = W.encode(rng.standard_normal((d_out, ldw)), dtype)
    idx = rng.choice(n, size=K, replace=False).astype(np.int32)
    idx[rng.random(K) < p_empty] = -1
    scale = rng.uniform(-2.0, 2.0, K).astype(np.float32) if with_scale else None
    return pool, Wm, idx, scale


def _run(pool, Wm, idx, scale, alpha, dtype):
    A, B = to_dev(pool.A, dtype), to_dev(pool.B, dtype)
    Wd = to_dev(Wm, dtype)
    L.lora_merge(L.Pool(A, B), idx.tolist(), Wd, None if scale is None else scale.tolist(), alpha)
    torch.cuda.synchronize()
    return from_dev(Wd, dtype)


def _check(dtype, got, ref, Wm, d_in, rows=None, what=""):
    rows = np.arange(got.shape[0]) if rows is None else np.asarray(rows)
    g = W.decode_f64(got[rows, :d_in], dtype)
    bound = TOL[dtype] * (1.0 + np.abs(ref))
    err = np.abs(g - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} out of tolerance, max err/bound {np.max(err / bound):.3g}"
    # columns past d_in keep their bits
    assert np.array_equal(got[rows, d_in:].view(np.uint8), Wm[rows, d_in:].view(np.uint8)), f"{what}: padding written"


GRID = {
    # matrix-core path (bf16, r % 8 == 0, K * r padded to 32 <= 256, d_in % 8 == 0)
    "bf16_r16_k1": dict(dtype=W.BF16, n=4, r=16, d_in=136, d_out=200, K=1),
    "bf16_r64_k2_alpha1": dict(dtype=W.BF16, n=5, r=64, d_in=512, d_out=256, K=2),
    "bf16_r24_k3_unmerge": dict(dtype=W.BF16, n=6, r=24, d_in=264, d_out=130, K=3, alpha=-1.0),
    "bf16_r128_k2": dict(dtype=W.BF16, n=3, r=128, d_in=256, d_out=96, K=2),
    "bf16_r256_k1": dict(dtype=W.BF16, n=2, r=256, d_in=384, d_out=70, K=1),
    "bf16_r8_k8_empty": dict(dtype=W.BF16, n=9, r=8, d_in=128, d_out=64, K=8, p_empty=0.3),
    "bf16_ldw_padded": dict(dtype=W.BF16, n=3, r=32, d_in=256, d_out=300, K=1, ldw=272),
    # 256-column strips (one slot up to rank 64, rank 128 alone): a ragged last strip, rows past one item
    "bf16_r64_k1_wide_ragged": dict(dtype=W.BF16, n=3, r=64, d_in=776, d_out=1100, K=1),
    "bf16_r128_k1_wide_ragged": dict(dtype=W.BF16, n=2, r=128, d_in=392, d_out=100, K=1, alpha=-1.0),
    # VALU path: fp32, odd shapes, K * r beyond the matrix-core limit
    "f32_r64_k2": dict(dtype=W.F32, n=4, r=64, d_in=200, d_out=150, K=2),
    "f32_r5_odd": dict(dtype=W.F32, n=3, r=5, d_in=37, d_out=23, K=2, ldw=41, alpha=-1.0),
    "bf16_odd_d_in": dict(dtype=W.BF16, n=3, r=16, d_in=100, d_out=64, K=1),
    "bf16_r5_k2": dict(dtype=W.BF16, n=4, r=5, d_in=64, d_out=48, K=2),
    "bf16_r128_k3_valu": dict(dtype=W.BF16, n=4, r=128, d_in=128, d_out=64, K=3),
}


@pytest.mark.parametrize("name", sorted(GRID))
def test_merge_grid(orc, name):
    kw = dict(GRID[name])
    alpha = kw.pop("alpha", 1.0)
    dtype = kw["dtype"]
    pool, Wm, idx, scale = _case(3000 + sorted(GRID).index(name), **kw)
    got = _run(pool, Wm, idx, scale, alpha, dtype)
    ref = orc.merge(dtype, pool.A, pool.B, Wm, idx, scale, alpha=alpha)
    _check(dtype, got, ref, Wm, pool.d_in, what=name)


@pytest.mark.parametrize("dtype,r,K", [(W.BF16, 64, 2), (W.BF16, 16, 1), (W.F32, 32, 2), (W.BF16, 5, 3)])
def test_merge_integer_probe_bitwise(orc, dtype, r, K):
    """Small integers: every product and partial sum is exact in fp32, so the
    result must equal the oracle's, rounded once, bit for bit (any order)."""
    rng = np.random.default_rng(77 + r)
    n, d_in, d_out = 4, 160, 96
    A = np.zeros((n, r, d_in))
    for i in range(n):
        for j in range(r):
            cols = rng.choice(d_in, size=4, replace=False)
            A[i, j, cols] = rng.choice([-1.0, 1.0], size=4)
    B = rng.integers(-2, 3, (n, d_out, r)).astype(np.float64)
    Wm = rng.integers(-64, 65, (d_out, d_in)).astype(np.float64)
    pool = W.Pool(dtype, n, r, d_in, d_out, W.encode(A, dtype), W.encode(B, dtype))
    We = W.encode(Wm, dtype)
    idx = np.arange(K, dtype=np.int32)
    scale = np.array([1.0, -2.0, 0.5][:K], np.float32)
    got = _run(pool, We, idx, scale, 1.0, dtype)
    ref = orc.merge(dtype, pool.A, pool.B, We, idx, scale, alpha=1.0)
    assert np.array_equal(got, W.encode(ref, dtype))


def test_merge_then_unmerge(orc):
    pool, Wm, idx, scale = _case(3100, W.BF16, 4, 64, 512, 384, 2)
    A, B = to_dev(pool.A, W.BF16), to_dev(pool.B, W.BF16)
    p = L.Pool(A, B)
    Wd = to_dev(Wm, W.BF16)
    L.lora_merge(p, idx.tolist(), Wd, scale.tolist(), 1.0)
    merged = from_dev(Wd, W.BF16)
    L.lora_merge(p, idx.tolist(), Wd, scale.tolist(), -1.0)
    torch.cuda.synchronize()
    back = W.decode_f64(from_dev(Wd, W.BF16), W.BF16)
    w0 = W.decode_f64(Wm, W.BF16)
    assert not np.array_equal(merged, Wm)
    # two roundings to bf16 (relative 2^-8 each) of values of the size of W + delta
    delta = np.abs(W.decode_f64(merged, W.BF16) - w0)
    assert np.all(np.abs(back - w0) <= 2 ** -7 * (np.abs(w0) + delta) + 1e-30)


def test_merged_weight_matches_unmerged_apply(orc):
    """The merged form on the GPU against the unmerged form on the GPU: for
    every row t, x_t W'^T - x_t W^T equals the delta lora_apply adds."""
    rng = np.random.default_rng(3200)
    n, r, d_in, d_out, T, K = 4, 32, 256, 192, 48, 2
    pool = W.make_pool(rng, W.BF16, n, r, d_in, d_out)
    Wm = W.encode(rng.standard_normal((d_out, d_in)) * 0.05, W.BF16)
    x = W.encode(rng.standard_normal((T, d_in)), W.BF16)
    idx = np.array([2, 0], np.int32)
    scale = np.array([0.75, -1.5], np.float32)
    merged = _run(pool, Wm, idx, scale, 1.0, W.BF16)
    A, B = to_dev(pool.A, W.BF16), to_dev(pool.B, W.BF16)
    batch = L.Batch(T, torch.from_numpy(np.tile(idx, (1, 1))).to(DEV),
                    torch.tensor([0, T], dtype=torch.int32, device=DEV),
                    torch.from_numpy(np.tile(scale, (1, 1))).to(DEV))
    y = torch.zeros((T, d_out), dtype=torch.bfloat16, device=DEV)
    xd = to_dev(x, W.BF16)
    ws = L.new_workspace(batch, n, DEV)
    L.lora_apply(L.Pool(A, B), batch, xd, y, ws)
    torch.cuda.synchronize()
    delta_apply = W.decode_f64(from_dev(y, W.BF16), W.BF16)
    xf = W.decode_f64(x, W.BF16)
    delta_merged = xf @ W.decode_f64(merged, W.BF16).T - xf @ W.decode_f64(Wm, W.BF16).T
    # merged weights carry one bf16 rounding of W + delta per element
    bound = 2 ** -8 * (np.abs(xf) @ np.abs(W.decode_f64(merged, W.BF16)).T) + 1e-2 * (1 + np.abs(delta_apply))
    assert np.all(np.abs(delta_merged - delta_apply) <= bound)


def test_merge_full_size_sampled(orc):
    """One FLUX-sized projection (3072 x 3072, rank 64) merged on the GPU; rows
    sampled at the start, the middle and the end checked against the oracle."""
    rng = np.random.default_rng(3300)
    n, r, d = 4, 64, 3072
    pool = W.make_pool(rng, W.BF16, n, r, d, d)
    Wm = W.encode(rng.standard_normal((d, d)) * 0.02, W.BF16)
    idx, scale = np.array([3], np.int32), np.array([1.0], np.float32)
    got = _run(pool, Wm, idx, scale, 1.0, W.BF16)
    for lo, hi in [(0, 8), (1531, 1541), (d - 8, d)]:
        ref = orc.merge(W.BF16, pool.A, pool.B, Wm, idx, scale, alpha=1.0, rows=(lo, hi))
        _check(W.BF16, got, ref, Wm, d, rows=np.arange(lo, hi), what=f"rows {lo}..{hi}")


@pytest.mark.parametrize("dtype,r,aligned", [(W.BF16, 64, True), (W.BF16, 16, False), (W.F32, 8, True)])
def test_merge_multi_equals_single_calls(orc, dtype, r, aligned):
    """Several weights of one shape in one launch give, bit for bit, what one
    call per weight gives (the same arithmetic), and match the oracle."""
    rng = np.random.default_rng(3400 + r)
    n, d_in, d_out, P = 3, 256, 136, 5
    pools = [W.make_pool(rng, dtype, n, r, d_in, d_out) for _ in range(P)]
    Ws = [W.encode(rng.standard_normal((d_out, d_in + 8)), dtype) for _ in range(P)]
    idx, scale = [2, 0], [0.5, -1.25]
    dev = [(to_dev(p.A, dtype), to_dev(p.B, dtype), to_dev(w, dtype)) for p, w in zip(pools, Ws)]
    views = [(A, B, Wd[:, :d_in]) for A, B, Wd in dev]
    table, al = L.merge_table(views, DEV)
    assert al
    L.lora_merge_multi(L.Pool(dev[0][0], dev[0][1]), idx, table, aligned and al, scale, 1.0)
    torch.cuda.synchronize()
    multi = [from_dev(Wd, dtype) for _, _, Wd in dev]
    for (A, B, Wd), w in zip(dev, Ws):
        Wd.copy_(to_dev(w, dtype))
    for A, B, Wv in views:
        L.lora_merge(L.Pool(A, B), idx, Wv, scale, 1.0)
    torch.cuda.synchronize()
    for q, ((A, B, Wd), p, w) in enumerate(zip(dev, pools, Ws)):
        single = from_dev(Wd, dtype)
        if aligned:
            assert np.array_equal(multi[q], single), f"problem {q}"
        ref = orc.merge(dtype, p.A, p.B, w[:, :d_in], np.array(idx, np.int32), np.array(scale, np.float32), alpha=1.0)
        _check(dtype, multi[q], np.pad(ref, ((0, 0), (0, 0))), w, d_in, what=f"problem {q}")
