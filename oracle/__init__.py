"""fp64 CPU oracle for unmerged multi-LoRA application: TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and the
two share no code: the oracle is ``lora_oracle.c`` (plain C, double precision,
OpenMP over rows) built with gcc, wrapped here with ctypes.

Functions and the passages they follow (pages named by title and section):
  * ``apply``  -- "Serving several LoRAs, ControlNet and IP-Adapter", section
    "LoRA: merged or alongside" (unmerged form adds x A^T B^T to x W^T) and the
    "Exercises" answer on four requests (group by LoRA index, add back in the
    original order); stacked LoRAs summed (comparison table, "Stacking").
  * ``shrink`` -- the x A^T half of the same formula, per slot, scale folded in.
  * ``expand`` -- the (.) B^T half, given the float32 intermediate.
  * ``merge``  -- same section: the merged form W + BA computed ahead of time,
    stacked LoRAs as a weighted sum (comparison table, "Stacking"); alpha = -1
    unmerges.

Pins (tests/test_oracle_pins.py) tie every function to something other than
itself; none of the four is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "lora_oracle.c")
LIB = os.path.join(_HERE, "_build", "liblora_oracle.so")

DTYPE_CODE = {"f32": 0, "bf16": 1}
ERRORS = {-1: "bad shape", -2: "adapter index out of range", -3: "bad segment offsets", -4: "out of memory"}


class OracleError(ValueError):
    pass


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, IEEE double, OpenMP)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-fno-fast-math",
           "-ffp-contract=off", *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(out=path)
        self.path = path
        self.lib = ctypes.CDLL(path)
        self.lib.oracle_apply.restype = _I
        self.lib.oracle_apply.argtypes = [_I, _I, _I, _I, _I, _P, _P, _I, _I, _P, _P, _I, _P,
                                          _P, _L, _P, _L, _P, _I, _P, _P, _P, _P, _I, _P]
        self.lib.oracle_shrink.restype = _I
        self.lib.oracle_shrink.argtypes = [_I, _I, _I, _I, _P, _I, _I, _P, _P, _I, _P,
                                           _P, _L, _P, _I, _P, _P, _I, _P]
        self.lib.oracle_expand.restype = _I
        self.lib.oracle_expand.argtypes = [_I, _I, _I, _I, _P, _I, _I, _P, _P, _I,
                                           _P, _L, _P, _L, _P, _I, _P, _P, _I, _P]
        self.lib.oracle_merge.restype = _I
        self.lib.oracle_merge.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _L, _I, _P, _P,
                                          ctypes.c_double, _I, _I, _P, _I]

    @staticmethod
    def _check(rc: int):
        if rc != 0:
            raise OracleError(ERRORS.get(rc, str(rc)))

    @staticmethod
    def _batch_arrays(seg_off, idx, scale):
        seg_off = None if seg_off is None else np.ascontiguousarray(seg_off, dtype=np.int32)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        scale = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
        return seg_off, idx, scale

    @staticmethod
    def _rows(rows, T):
        if rows is None:
            return None, T
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        return rows, int(rows.size)

    @staticmethod
    def _ranks(ranks):
        return None if ranks is None else np.ascontiguousarray(ranks, dtype=np.int32)

    def apply(self, dtype, A, B, x, y, *, T, S, K, seg_off, idx, scale=None, rows=None, nthreads=0, ranks=None):
        """Returns (y_ref [R][d_out] float64, touched [R] bool, routing [R][K] int32, macs)."""
        n, r, d_in = A.shape
        d_out = B.shape[1]
        assert B.shape == (n, d_out, r)
        A = np.ascontiguousarray(A); B = np.ascontiguousarray(B)
        x = np.ascontiguousarray(x); y = np.ascontiguousarray(y)
        seg_off, idx, scale = self._batch_arrays(seg_off, idx, scale)
        rows, R = self._rows(rows, T)
        y_ref = np.empty((R, d_out), np.float64)
        touched = np.empty(R, np.uint8)
        routing = np.empty((R, K), np.int32)
        macs = ctypes.c_int64(0)
        rc = self.lib.oracle_apply(DTYPE_CODE[dtype], n, r, d_in, d_out, _ptr(A), _ptr(B),
                                   T, S, _ptr(seg_off), _ptr(idx), K, _ptr(scale),
                                   _ptr(x), x.shape[1], _ptr(y), y.shape[1], _ptr(rows), R,
                                   _ptr(y_ref), _ptr(touched), _ptr(routing), ctypes.byref(macs), nthreads,
                                   _ptr(self._ranks(ranks)))
        self._check(rc)
        return y_ref, touched.astype(bool), routing, int(macs.value)

    def shrink(self, dtype, A, x, *, T, S, K, seg_off, idx, scale=None, rows=None, nthreads=0, ranks=None):
        """Returns (v_ref [R][K*r] float64, touched [R] bool)."""
        n, r, d_in = A.shape
        A = np.ascontiguousarray(A); x = np.ascontiguousarray(x)
        seg_off, idx, scale = self._batch_arrays(seg_off, idx, scale)
        rows, R = self._rows(rows, T)
        v_ref = np.empty((R, K * r), np.float64)
        touched = np.empty(R, np.uint8)
        rc = self.lib.oracle_shrink(DTYPE_CODE[dtype], n, r, d_in, _ptr(A), T, S, _ptr(seg_off), _ptr(idx),
                                    K, _ptr(scale), _ptr(x), x.shape[1], _ptr(rows), R,
                                    _ptr(v_ref), _ptr(touched), nthreads, _ptr(self._ranks(ranks)))
        self._check(rc)
        return v_ref, touched.astype(bool)

    def expand(self, dtype, B, v, y, *, T, S, K, seg_off, idx, rows=None, nthreads=0, ranks=None):
        """v: float32 [T][ldv] with v[t][k*r + j].  Returns (y_ref [R][d_out] float64, touched [R] bool)."""
        n, d_out, r = B.shape
        B = np.ascontiguousarray(B)
        v = np.ascontiguousarray(v, dtype=np.float32); y = np.ascontiguousarray(y)
        seg_off, idx, _ = self._batch_arrays(seg_off, idx, None)
        rows, R = self._rows(rows, T)
        y_ref = np.empty((R, d_out), np.float64)
        touched = np.empty(R, np.uint8)
        rc = self.lib.oracle_expand(DTYPE_CODE[dtype], n, r, d_out, _ptr(B), T, S, _ptr(seg_off), _ptr(idx), K,
                                    _ptr(v), v.shape[1], _ptr(y), y.shape[1], _ptr(rows), R,
                                    _ptr(y_ref), _ptr(touched), nthreads, _ptr(self._ranks(ranks)))
        self._check(rc)
        return y_ref, touched.astype(bool)

    def merge(self, dtype, A, B, W, idx, scale=None, alpha=1.0, rows=None, nthreads=0):
        """W [d_out][ldw] encoded; idx [K] adapter indices (-1 skipped); scale [K] or None.
        Returns W_out [row_hi - row_lo][d_in] float64 for rows = (row_lo, row_hi) (all rows by default)."""
        n, r, d_in = A.shape
        d_out = B.shape[1]
        assert B.shape == (n, d_out, r) and W.shape[0] == d_out
        A = np.ascontiguousarray(A); B = np.ascontiguousarray(B); W = np.ascontiguousarray(W)
        idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1)
        sc = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32).reshape(-1)
        lo, hi = (0, d_out) if rows is None else rows
        out = np.empty((hi - lo, d_in), np.float64)
        rc = self.lib.oracle_merge(DTYPE_CODE[dtype], n, r, d_in, d_out, _ptr(A), _ptr(B), _ptr(W), W.shape[1],
                                   int(idx.size), _ptr(idx), _ptr(sc), float(alpha), lo, hi, _ptr(out), nthreads)
        self._check(rc)
        return out

    # convenience over workloads.Case -------------------------------------
    def apply_case(self, case, rows=None, nthreads=0, ranks=None):
        b, p = case.batch, case.pool
        return self.apply(case.dtype, p.A, p.B, case.x, case.y, T=b.T, S=b.S, K=b.K,
                          seg_off=b.seg_off, idx=b.idx, scale=b.scale, rows=rows, nthreads=nthreads, ranks=ranks)

    def shrink_case(self, case, rows=None, nthreads=0):
        b, p = case.batch, case.pool
        return self.shrink(case.dtype, p.A, case.x, T=b.T, S=b.S, K=b.K, seg_off=b.seg_off,
                           idx=b.idx, scale=b.scale, rows=rows, nthreads=nthreads)


_default: Optional[Oracle] = None


def load() -> Oracle:
    """The oracle built from lora_oracle.c (built on first use if absent)."""
    global _default
    if _default is None:
        _default = Oracle(LIB)
    return _default
