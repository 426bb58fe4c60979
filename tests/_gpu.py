"""Helpers for the GPU parity tests: seeded cases -> device tensors -> HIP
library -> comparison with the fp64 oracle.

Tolerances (stated for floating-point outputs of touched rows, elementwise):
  bf16 inputs, fp32 accumulation:  |y_gpu - y_ref| <= 1e-2 * (1 + |y_ref|)
  fp32 inputs:                     |y_gpu - y_ref| <= 1e-5 * (1 + |y_ref|)
Untouched rows (every slot -1, or no request) must keep their bits exactly,
and so must the padding columns beyond d_out of every row.
"""
from __future__ import annotations

import numpy as np
import torch

import rank_sgmv_bgmv_amd as L
import workloads as W

TOL = {W.BF16: 1e-2, W.F32: 1e-5}
DEV = "cuda:0"


def tdtype(dtype):
    return torch.bfloat16 if dtype == W.BF16 else torch.float32


def to_dev(a: np.ndarray, dtype: str, dev=DEV):
    if dtype == W.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def from_dev(t, dtype: str) -> np.ndarray:
    if dtype == W.BF16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def dev_batch(b: W.Batch, dev=DEV) -> L.Batch:
    idx = torch.from_numpy(np.ascontiguousarray(b.idx, dtype=np.int32)).to(dev)
    seg = None if b.seg_off is None else torch.from_numpy(np.ascontiguousarray(b.seg_off, dtype=np.int32)).to(dev)
    sc = None if b.scale is None else torch.from_numpy(np.ascontiguousarray(b.scale, dtype=np.float32)).to(dev)
    return L.Batch(b.T, idx, seg, sc)


class DevCase:
    """A workloads.Case on the device: pool, batch, x view [T][d_in], y buffer."""

    def __init__(self, case: W.Case, dev=DEV):
        self.case = case
        p = case.pool
        self.A = to_dev(p.A, case.dtype, dev)
        self.B = to_dev(p.B, case.dtype, dev)
        self.pool = L.Pool(self.A, self.B)
        self.batch = dev_batch(case.batch, dev)
        self.x_full = to_dev(case.x, case.dtype, dev)
        self.x = self.x_full[:, :p.d_in]
        self.y_full = to_dev(case.y, case.dtype, dev)
        self.y = self.y_full[:, :p.d_out]
        self.ws = L.new_workspace(self.batch, p.n, dev)

    def reset_y(self):
        self.y_full.copy_(to_dev(self.case.y, self.case.dtype, self.y_full.device))

    def apply(self):
        L.lora_apply(self.pool, self.batch, self.x, self.y, self.ws)
        torch.cuda.synchronize()
        return from_dev(self.y_full, self.case.dtype)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    return W.decode_f64(bits, dtype)


def assert_parity(case: W.Case, y_out_full: np.ndarray, y_ref: np.ndarray, touched: np.ndarray, rows=None,
                  tol=None, what=""):
    """y_out_full: the device's y after the call (encoded, [T][ldy]); y_ref, touched
    from the oracle for `rows` (all rows when None)."""
    d_out = case.pool.d_out
    tol = TOL[case.dtype] if tol is None else tol
    rows = np.arange(case.batch.T) if rows is None else np.asarray(rows)
    y_in = case.y
    if len(rows) == 0:
        return
    out = y_out_full[rows]
    inp = y_in[rows]
    # padding columns never change
    assert np.array_equal(out[:, d_out:].view(np.uint8), inp[:, d_out:].view(np.uint8)), f"{what}: padding written"
    # untouched rows keep their bits
    un = ~touched
    if un.any():
        assert np.array_equal(out[un].view(np.uint8), inp[un].view(np.uint8)), f"{what}: untouched row written"
    if touched.any():
        got = decode(out[touched][:, :d_out], case.dtype)
        ref = y_ref[touched]
        err = np.abs(got - ref)
        bound = tol * (1.0 + np.abs(ref))
        bad = ~(err <= bound)
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; first at row "
                                 f"{rows[touched][i[0]]} col {i[1]}: got {got[tuple(i)]} ref {ref[tuple(i)]}; "
                                 f"max err/bound {np.max(err / bound):.3g}")


def sample_rows(batch: W.Batch, n_random: int, seed: int) -> np.ndarray:
    """First and last row of every request plus random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    rows = set()
    for lo, hi in batch.seg_bounds():
        if hi > lo:
            rows.add(lo)
            rows.add(hi - 1)
    if batch.T:
        rows.update(int(v) for v in rng.integers(0, batch.T, size=n_random))
    return np.array(sorted(rows), dtype=np.int32)


def check_problem_sampled(orc, batch: W.Batch, A, B, x, y0, y_out, rows, what, ranks=None):
    """One problem of a large launch against the oracle on `rows`: the adapters
    the batch uses are copied to the host (the oracle's result does not depend
    on the others) and the batch's indices remapped to them.  A, B, x, y0 (y
    before the launch) and y_out are device tensors of one dtype."""
    dtype = W.BF16 if A.dtype == torch.bfloat16 else W.F32
    n = int(A.shape[0])
    idx = np.asarray(batch.idx)
    used = np.unique(idx[(idx >= 0) & (idx < n)])
    remap = np.full(n, -1, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    idx_small = np.where((idx >= 0) & (idx < n), remap[np.clip(idx, 0, n - 1)], -1).astype(np.int32)
    sel = torch.from_numpy(used.astype(np.int64)).to(A.device)
    pool = W.Pool(dtype, len(used), int(A.shape[1]), int(A.shape[2]), int(B.shape[1]),
                  from_dev(A.index_select(0, sel), dtype), from_dev(B.index_select(0, sel), dtype))
    small = W.Batch(batch.T, batch.S, batch.K, batch.seg_off, idx_small, batch.scale)
    case = W.Case(what, dtype, small, pool, from_dev(x, dtype), from_dev(y0, dtype))
    rk = None if ranks is None else np.asarray(ranks)[used]
    y_ref, touched, _, _ = orc.apply_case(case, rows=rows, ranks=rk)
    assert_parity(case, from_dev(y_out, dtype), y_ref, touched, rows=rows, what=what)
    return touched
