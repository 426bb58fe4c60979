"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on failure.  They
are run on the real oracle (test_oracle_pins.py) and on deliberately broken
copies of it (test_oracle_mutations.py), which must each fail at least one pin.

What pins what (pages named by title and section):
  merged_form      -- "Serving several LoRAs, ControlNet and IP-Adapter",
                      "LoRA: merged or alongside": x(W + BA)^T - xW^T equals the
                      unmerged delta x A^T B^T (non-square shapes catch transposes).
  rank1_closed     -- with r = 1 the delta is s (x.a) b_o; exact on small integers.
  linearity        -- the delta is linear in x.
  untouched        -- slots of -1 and rows outside every request are left as they are.
  permutation      -- reordering requests (with their rows) reorders the output rows;
                      "Exercises" (four requests): results go back in the original order.
  stacking         -- comparison table, stacking row: K stacked adapters
                      equal one adapter of rank K*r with A's stacked by rows and B's
                      by columns.
  numpy_special    -- one request, one adapter: (x A^T) B^T by numpy matmul.
  exact_bruteforce -- tiny integer inputs evaluated with Python integers.
  macs_formula     -- the multiply-adds performed match the page's lora_costs count
                      2 N (d r + r d) (section "LoRA: merged or alongside").
  shrink_numpy, expand_numpy, shrink_expand_compose -- the two halves.
  merge_vs_unmerged -- "LoRA: merged or alongside": with K stacked slots,
                      x W'^T - x W^T for the merged W' equals the unmerged
                      delta of the apply oracle (a different association;
                      non-square shapes catch transposes).
  merge_rank1      -- r = 1: W' = W + alpha s b a^T, exact on small integers.
  merge_inverse    -- unmerging (alpha = -1) what was merged gives W back
                      exactly on small integers; rows subsets agree.
  merge_numpy      -- W + alpha sum_k s_k B_k A_k by numpy matmul; -1 slots skipped.
  ranks_padding    -- "LoRA: merged or alongside" (r usually 8 to 128): adapters of
                      different ranks in one pool; with a rank array, apply, shrink
                      and expand equal the same calls on the pool with everything
                      past each adapter's rank set to zero (the padding holds
                      nonzero values here, so reading it would show).
"""
from __future__ import annotations

import numpy as np

import workloads as W

F32 = W.F32


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def _apply_case(orc, case, **kw):
    b, p = case.batch, case.pool
    return orc.apply(case.dtype, p.A, p.B, case.x, case.y, T=b.T, S=b.S, K=b.K,
                     seg_off=b.seg_off, idx=b.idx, scale=b.scale, **kw)


def _delta(orc, case):
    y_ref, touched, routing, _ = _apply_case(orc, case)
    y0 = W.decode_f64(case.y, case.dtype)
    return y_ref - y0, touched, routing


# ---------------------------------------------------------------------------
def pin_merged_form(orc):
    rng = _rng(11)
    n, r, d_in, d_out = 3, 3, 5, 7
    lengths = [2, 0, 3, 1, 2]
    S, K = len(lengths), 1
    seg = W.offsets_from_lengths(lengths)
    T = int(seg[-1])
    idx = np.array([[2], [0], [1], [-1], [0]], np.int32)
    scale = _f32(rng.uniform(0.5, 2.0, size=(S, K)))
    A = _f32(rng.standard_normal((n, r, d_in)))
    B = _f32(rng.standard_normal((n, d_out, r)))
    x = _f32(rng.standard_normal((T, d_in)))
    y = _f32(rng.standard_normal((T, d_out)))
    Wt = rng.standard_normal((d_out, d_in))
    y_ref, touched, _, _ = orc.apply(F32, A, B, x, y, T=T, S=S, K=K, seg_off=seg, idx=idx, scale=scale)
    got = y_ref - y.astype(np.float64)
    for s in range(S):
        for t in range(seg[s], seg[s + 1]):
            i = idx[s, 0]
            xt = x[t].astype(np.float64)
            if i < 0:
                assert not touched[t]
                assert np.array_equal(y_ref[t], y[t].astype(np.float64))
                continue
            assert touched[t]
            merged = Wt + float(scale[s, 0]) * (B[i].astype(np.float64) @ A[i].astype(np.float64))
            want = xt @ merged.T - xt @ Wt.T
            assert np.allclose(got[t], want, rtol=1e-11, atol=1e-11), (t, got[t], want)


def pin_rank1_closed(orc):
    rng = _rng(12)
    n, d_in, d_out = 4, 9, 6
    lengths = [3, 1, 4, 2]
    S, K = len(lengths), 1
    seg = W.offsets_from_lengths(lengths)
    T = int(seg[-1])
    idx = np.array([[1], [3], [0], [1]], np.int32)
    scale = _f32([[2.0], [-1.0], [3.0], [0.5]])
    A = _f32(rng.integers(-3, 4, (n, 1, d_in)))
    B = _f32(rng.integers(-3, 4, (n, d_out, 1)))
    x = _f32(rng.integers(-3, 4, (T, d_in)))
    y = _f32(rng.integers(-9, 10, (T, d_out)))
    y_ref, _, _, _ = orc.apply(F32, A, B, x, y, T=T, S=S, K=K, seg_off=seg, idx=idx, scale=scale)
    for s in range(S):
        i = int(idx[s, 0])
        for t in range(seg[s], seg[s + 1]):
            xa = int(np.dot(x[t].astype(np.int64), A[i, 0].astype(np.int64)))
            for o in range(d_out):
                want = float(y[t, o]) + float(scale[s, 0]) * xa * float(B[i, o, 0])
                assert y_ref[t, o] == want, (t, o, y_ref[t, o], want)


def pin_linearity(orc):
    rng = _rng(13)
    case = W.random_case(5, dtype=F32, n=3, r=4, d_in=11, d_out=9, S=5, K=2, min_len=1, max_len=4,
                         with_scale=True, std_w=0.5)
    x1 = _f32(rng.integers(-4, 5, case.x.shape))
    x2 = _f32(rng.integers(-4, 5, case.x.shape))
    al, be = 3.0, -2.0
    c1 = W.dataclasses.replace(case, x=x1)
    c2 = W.dataclasses.replace(case, x=x2)
    c3 = W.dataclasses.replace(case, x=_f32(al * x1 + be * x2))
    d1, t1, _ = _delta(orc, c1)
    d2, _, _ = _delta(orc, c2)
    d3, _, _ = _delta(orc, c3)
    assert t1.any()
    assert np.allclose(d3, al * d1 + be * d2, rtol=1e-11, atol=1e-11)


def pin_untouched(orc):
    rng = _rng(14)
    n, r, d_in, d_out, K = 3, 2, 6, 5, 2
    seg = np.array([2, 4, 7, 9], np.int32)          # rows 0,1 and 9,10 belong to no request
    T, S = 11, 3
    idx = np.array([[-1, -1], [1, -1], [-1, -1]], np.int32)
    A = _f32(rng.standard_normal((n, r, d_in)))
    B = _f32(rng.standard_normal((n, d_out, r)))
    x = _f32(rng.standard_normal((T, d_in)))
    y = _f32(rng.standard_normal((T, d_out)))
    yu = y.view(np.uint32)
    for t in (0, 1, 2, 3, 7, 8, 9, 10):
        yu[t, 0] = 0x80000000                          # -0.0
        yu[t, 1] = 0x7FC01234                          # NaN with a payload
    y_ref, touched, routing, _ = orc.apply(F32, A, B, x, y, T=T, S=S, K=K, seg_off=seg, idx=idx)
    assert list(touched) == [False] * 4 + [True] * 3 + [False] * 4
    for t in (0, 1, 2, 3, 7, 8, 9, 10):
        assert np.all(routing[t] == -1)
        assert np.signbit(y_ref[t, 0]) and y_ref[t, 0] == 0.0
        assert np.isnan(y_ref[t, 1])
        assert np.array_equal(y_ref[t, 2:], y[t, 2:].astype(np.float64))
    assert np.all(routing[4:7, 0] == 1) and np.all(routing[4:7, 1] == -1)
    assert not np.array_equal(y_ref[4:7], y[4:7].astype(np.float64))


def pin_permutation(orc):
    rng = _rng(15)
    case = W.random_case(7, dtype=F32, n=4, r=3, d_in=8, d_out=6, S=6, K=2, min_len=0, max_len=4,
                         with_scale=True, std_w=0.5)
    b = case.batch
    perm = rng.permutation(b.S)
    bounds = b.seg_bounds()
    rows = np.concatenate([np.arange(*bounds[s]) for s in perm]).astype(np.int64) if b.T else np.zeros(0, np.int64)
    lengths = [bounds[s][1] - bounds[s][0] for s in perm]
    b2 = W.Batch(b.T, b.S, b.K, W.offsets_from_lengths(lengths), b.idx[perm].copy(), b.scale[perm].copy())
    c2 = W.Case("perm", case.dtype, b2, case.pool, case.x[rows].copy(), case.y[rows].copy())
    y1, t1, r1, _ = _apply_case(orc, case)
    y2, t2, r2, _ = _apply_case(orc, c2)
    assert np.array_equal(y2, y1[rows]) and np.array_equal(t2, t1[rows]) and np.array_equal(r2, r1[rows])


def pin_stacking(orc):
    rng = _rng(16)
    n, r, d_in, d_out, K = 5, 3, 7, 6, 3
    lengths = [2, 3, 1]
    S = len(lengths)
    seg = W.offsets_from_lengths(lengths)
    T = int(seg[-1])
    idx = np.array([[4, 1, 2], [0, -1, 3], [2, 2, -1]], np.int32)
    scale = _f32([[0.5, 2.0, -1.0], [4.0, 1.0, 0.25], [1.0, -2.0, 8.0]])   # powers of two: exact
    A = _f32(rng.standard_normal((n, r, d_in)))
    B = _f32(rng.standard_normal((n, d_out, r)))
    x = _f32(rng.standard_normal((T, d_in)))
    y = _f32(rng.standard_normal((T, d_out)))
    y_ref, _, _, _ = orc.apply(F32, A, B, x, y, T=T, S=S, K=K, seg_off=seg, idx=idx, scale=scale)
    for s in range(S):
        As, Bs = [], []
        for k in range(K):
            i = idx[s, k]
            if i < 0:
                continue
            As.append(A[i])
            Bs.append(B[i] * scale[s, k])
        Acat = np.concatenate(As, 0)[None]           # one adapter of rank len(As)*r
        Bcat = np.concatenate(Bs, 1)[None]
        L = int(seg[s + 1] - seg[s])
        one = np.array([0, L], np.int32)
        y1, _, _, _ = orc.apply(F32, _f32(Acat), _f32(Bcat), x[seg[s]:seg[s + 1]], y[seg[s]:seg[s + 1]],
                                T=L, S=1, K=1, seg_off=one, idx=np.zeros((1, 1), np.int32))
        assert np.allclose(y_ref[seg[s]:seg[s + 1]], y1, rtol=1e-11, atol=1e-11)


def pin_numpy_special(orc):
    rng = _rng(17)
    n, r, d_in, d_out, T = 2, 5, 13, 10, 4
    A = _f32(rng.standard_normal((n, r, d_in)))
    B = _f32(rng.standard_normal((n, d_out, r)))
    x = _f32(rng.standard_normal((T, d_in)))
    y = _f32(rng.standard_normal((T, d_out)))
    y_ref, _, _, _ = orc.apply(F32, A, B, x, y, T=T, S=1, K=1, seg_off=np.array([0, T], np.int32),
                               idx=np.array([[1]], np.int32))
    want = y.astype(np.float64) + (x.astype(np.float64) @ A[1].astype(np.float64).T) @ B[1].astype(np.float64).T
    assert np.allclose(y_ref, want, rtol=1e-12, atol=1e-12)


def pin_exact_bruteforce(orc):
    rng = _rng(18)
    n, r, d_in, d_out, K = 3, 2, 4, 3, 2
    lengths = [1, 2, 0, 2]
    S = len(lengths)
    seg = W.offsets_from_lengths(lengths)
    T = int(seg[-1]) + 1                              # the last row belongs to no request
    idx = np.array([[0, 2], [1, -1], [2, 0], [-1, 1]], np.int32)
    scale = _f32(rng.integers(-3, 4, (S, K)))
    A = rng.integers(-3, 4, (n, r, d_in))
    B = rng.integers(-3, 4, (n, d_out, r))
    x = rng.integers(-3, 4, (T, d_in))
    y = rng.integers(-20, 21, (T, d_out))
    y_ref, touched, _, _ = orc.apply(F32, _f32(A), _f32(B), _f32(x), _f32(y), T=T, S=S, K=K, seg_off=seg,
                                     idx=idx, scale=scale)
    for t in range(T):
        owner = [s for s in range(S) if seg[s] <= t < seg[s + 1]]
        out = [int(v) for v in y[t]]
        hit = False
        if owner:
            s = owner[0]
            for k in range(K):
                i = int(idx[s, k])
                if i == -1:
                    continue
                hit = True
                for o in range(d_out):
                    tot = 0
                    for j in range(r):
                        vj = sum(int(x[t, c]) * int(A[i, j, c]) for c in range(d_in))
                        tot += vj * int(B[i, o, j])
                    out[o] += int(scale[s, k]) * tot
        assert bool(touched[t]) == hit
        assert [float(v) for v in out] == list(y_ref[t]), (t, out, y_ref[t])


def pin_macs_formula(orc):
    # lora_costs counts 2 N (d r + r d) FLOPs per adapted layer: N (d_in r + r d_out) multiply-adds
    rng = _rng(19)
    n, r, d_in, d_out = 2, 4, 12, 10
    lengths = [3, 5, 2]
    seg = W.offsets_from_lengths(lengths)
    T = int(seg[-1])
    idx = np.array([[0], [1], [0]], np.int32)
    A = _f32(rng.standard_normal((n, r, d_in)))
    B = _f32(rng.standard_normal((n, d_out, r)))
    x = _f32(rng.standard_normal((T, d_in)))
    y = _f32(rng.standard_normal((T, d_out)))
    _, _, _, macs = orc.apply(F32, A, B, x, y, T=T, S=3, K=1, seg_off=seg, idx=idx)
    assert 2 * macs == 2 * T * (d_in * r + r * d_out)


def pin_shrink_numpy(orc):
    rng = _rng(20)
    n, r, d_in, T, K = 3, 4, 9, 5, 2
    A = _f32(rng.standard_normal((n, r, d_in)))
    x = _f32(rng.standard_normal((T, d_in)))
    seg = np.array([0, 2, 5], np.int32)
    idx = np.array([[2, -1], [0, 1]], np.int32)
    scale = _f32([[1.5, 3.0], [-0.5, 2.0]])
    v, touched = orc.shrink(F32, A, x, T=T, S=2, K=K, seg_off=seg, idx=idx, scale=scale)
    assert touched.all()
    X = x.astype(np.float64)
    for s, (lo, hi) in enumerate([(0, 2), (2, 5)]):
        for k in range(K):
            i = idx[s, k]
            want = np.zeros((hi - lo, r)) if i < 0 else float(scale[s, k]) * (X[lo:hi] @ A[i].astype(np.float64).T)
            assert np.allclose(v[lo:hi, k * r:(k + 1) * r], want, rtol=1e-12, atol=1e-12)


def pin_expand_numpy(orc):
    rng = _rng(21)
    n, r, d_out, T, K = 3, 4, 7, 5, 2
    B = _f32(rng.standard_normal((n, d_out, r)))
    v = _f32(rng.standard_normal((T, K * r)))
    y = _f32(rng.standard_normal((T, d_out)))
    seg = np.array([0, 2, 4], np.int32)              # row 4 belongs to no request
    idx = np.array([[2, -1], [0, 1]], np.int32)
    y_ref, touched = orc.expand(F32, B, v, y, T=T, S=2, K=K, seg_off=seg, idx=idx)
    assert list(touched) == [True] * 4 + [False]
    V, Y = v.astype(np.float64), y.astype(np.float64)
    want = Y.copy()
    want[0:2] += V[0:2, 0:r] @ B[2].astype(np.float64).T
    want[2:4] += V[2:4, 0:r] @ B[0].astype(np.float64).T + V[2:4, r:2 * r] @ B[1].astype(np.float64).T
    assert np.allclose(y_ref, want, rtol=1e-12, atol=1e-12)


def pin_shrink_expand_compose(orc):
    rng = _rng(22)
    n, r, d_in, d_out, K = 3, 3, 6, 5, 2
    seg = np.array([0, 1, 4, 6], np.int32)
    T, S = 7, 3
    idx = np.array([[1, 2], [-1, 0], [2, -1]], np.int32)
    scale = _f32(rng.integers(-2, 3, (S, K)))
    A = _f32(rng.integers(-2, 3, (n, r, d_in)))
    B = _f32(rng.integers(-2, 3, (n, d_out, r)))
    x = _f32(rng.integers(-2, 3, (T, d_in)))
    y = _f32(rng.integers(-5, 6, (T, d_out)))
    v, _ = orc.shrink(F32, A, x, T=T, S=S, K=K, seg_off=seg, idx=idx, scale=scale)
    y2, _ = orc.expand(F32, B, _f32(v), y, T=T, S=S, K=K, seg_off=seg, idx=idx)
    y1, _, _, _ = orc.apply(F32, A, B, x, y, T=T, S=S, K=K, seg_off=seg, idx=idx, scale=scale)
    assert np.array_equal(y1, y2)


def pin_merge_vs_unmerged(orc):
    rng = _rng(31)
    n, r, d_in, d_out, T = 4, 3, 6, 5, 7
    slots = np.array([2, -1, 0], np.int32)
    sc = _f32([1.5, 4.0, -0.75])
    A = _f32(rng.standard_normal((n, r, d_in)))
    B = _f32(rng.standard_normal((n, d_out, r)))
    Wm = _f32(rng.standard_normal((d_out, d_in)))
    x = _f32(rng.standard_normal((T, d_in)))
    merged = orc.merge(F32, A, B, Wm, slots, sc, alpha=1.0)
    # one request covering every row, the same slots
    y0 = np.zeros((T, d_out), np.float32)
    seg = np.array([0, T], np.int32)
    y_ref, touched, _, _ = orc.apply(F32, A, B, x, y0, T=T, S=1, K=3, seg_off=seg, idx=slots[None, :],
                                     scale=sc[None, :])
    assert touched.all()
    xd = x.astype(np.float64)
    want = xd @ merged.T - xd @ Wm.astype(np.float64).T
    assert np.allclose(y_ref, want, rtol=1e-11, atol=1e-11)


def pin_merge_rank1(orc):
    rng = _rng(32)
    n, d_in, d_out = 3, 7, 4
    A = _f32(rng.integers(-3, 4, (n, 1, d_in)))
    B = _f32(rng.integers(-3, 4, (n, d_out, 1)))
    Wm = _f32(rng.integers(-9, 10, (d_out, d_in)))
    for alpha, i, s in [(1.0, 1, 2.0), (-1.0, 2, 0.5), (1.0, 0, -3.0)]:
        got = orc.merge(F32, A, B, Wm, np.array([i], np.int32), _f32([s]), alpha=alpha)
        for o in range(d_out):
            for c in range(d_in):
                want = float(Wm[o, c]) + alpha * s * float(B[i, o, 0]) * float(A[i, 0, c])
                assert got[o, c] == want, (o, c, got[o, c], want)


def pin_merge_inverse(orc):
    rng = _rng(33)
    n, r, d_in, d_out = 3, 4, 9, 6
    A = _f32(rng.integers(-2, 3, (n, r, d_in)))
    B = _f32(rng.integers(-2, 3, (n, d_out, r)))
    Wm = _f32(rng.integers(-20, 21, (d_out, d_in)))
    slots, sc = np.array([1, 2], np.int32), _f32([2.0, -1.0])
    merged = orc.merge(F32, A, B, Wm, slots, sc, alpha=1.0)
    assert not np.array_equal(merged, Wm.astype(np.float64))
    back = orc.merge(F32, A, B, _f32(merged), slots, sc, alpha=-1.0)
    assert np.array_equal(back, Wm.astype(np.float64))
    part = orc.merge(F32, A, B, Wm, slots, sc, alpha=1.0, rows=(2, 5))
    assert np.array_equal(part, merged[2:5])


def pin_merge_numpy(orc):
    rng = _rng(34)
    n, r, d_in, d_out = 5, 6, 10, 8
    A = _f32(rng.standard_normal((n, r, d_in)))
    B = _f32(rng.standard_normal((n, d_out, r)))
    Wm = _f32(rng.standard_normal((d_out, d_in + 3)))  # ld > d_in
    slots, sc = np.array([4, -1, 1, 3], np.int32), _f32([0.5, 9.0, -2.0, 1.25])
    got = orc.merge(F32, A, B, Wm, slots, sc, alpha=-1.0)
    want = Wm[:, :d_in].astype(np.float64).copy()
    for i, s in zip(slots, sc):
        if i >= 0:
            want -= float(s) * (B[i].astype(np.float64) @ A[i].astype(np.float64))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def pin_ranks_padding(orc):
    rng = _rng(35)
    n, r, d_in, d_out = 4, 8, 10, 7
    ranks = np.array([3, 8, 1, 5], np.int32)
    case = W.random_case(36, dtype=F32, n=n, r=r, d_in=d_in, d_out=d_out, S=6, K=2, min_len=1, max_len=4,
                         with_scale=True)
    p, b = case.pool, case.batch
    A0, B0 = p.A.copy(), p.B.copy()
    for i in range(n):
        A0[i, ranks[i]:, :] = 0
        B0[i, :, ranks[i]:] = 0
    kw = dict(T=b.T, S=b.S, K=b.K, seg_off=b.seg_off, idx=b.idx, scale=b.scale)
    y1, t1, _, m1 = orc.apply(F32, p.A, p.B, case.x, case.y, ranks=ranks, **kw)
    y0, t0, _, m0 = orc.apply(F32, A0, B0, case.x, case.y, **kw)
    assert np.array_equal(t1, t0) and np.allclose(y1, y0, rtol=1e-13, atol=1e-13)
    assert m1 < m0  # fewer multiply-adds: the padding is not touched
    v1, _ = orc.shrink(F32, p.A, case.x, ranks=ranks, **kw)
    v0, _ = orc.shrink(F32, A0, case.x, **kw)
    assert np.allclose(v1, v0, rtol=1e-13, atol=1e-13)
    ekw = {k: v for k, v in kw.items() if k != "scale"}
    vr = _f32(rng.standard_normal((b.T, b.K * r)))  # nonzero past every rank too
    e1, _ = orc.expand(F32, p.B, vr, case.y, ranks=ranks, **ekw)
    e0, _ = orc.expand(F32, B0, vr, case.y, **ekw)
    assert np.allclose(e1, e0, rtol=1e-13, atol=1e-13)
    yf, _, _, _ = orc.apply(F32, p.A, p.B, case.x, case.y, ranks=np.full(n, r, np.int32), **kw)
    yn, _, _, _ = orc.apply(F32, p.A, p.B, case.x, case.y, **kw)
    assert np.array_equal(yf, yn)


ALL_PINS = [pin_merged_form, pin_rank1_closed, pin_linearity, pin_untouched, pin_permutation, pin_stacking,
            pin_numpy_special, pin_exact_bruteforce, pin_macs_formula, pin_shrink_numpy, pin_expand_numpy,
            pin_shrink_expand_compose, pin_merge_vs_unmerged, pin_merge_rank1, pin_merge_inverse, pin_merge_numpy,
            pin_ranks_padding]


def run_all(orc):
    """Run every pin; return the names of those that failed."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:  # a mutant may also crash a pin with a bad index
            failed.append(pin.__name__)
    return failed
