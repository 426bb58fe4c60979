"""Unmerged multi-LoRA (SGMV / BGMV) for AMD MI355X (gfx950).

A thin ctypes binding over the C-ABI library ``_build/liblora_hip.so``
(declared in ``include/lora.h``).  Every function here only marshals torch
tensors into pointers, sizes and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback: if
the library has not been built, calls raise ``LoraError``.

Functions carry the C names:
  lora_workspace_size, lora_plan_build, lora_apply, lora_apply_noalloc, lora_shrink, lora_expand,
  lora_apply_planned, lora_shrink_planned, lora_expand_planned,
  lora_apply_multi, lora_apply_sliced, lora_read_device_errors, lora_status_string,
  and the measurement aids lora_calib_gather_read and lora_calib_tile_stream
  (include/lora_calib.h).

Tensors: A [n][r][d_in] and B [n][d_out][r] contiguous (float32 or bfloat16);
x [T][ldx], y [T][ldy] with unit column stride (ld = stride(0)); idx int32
[S][K]; seg_off int32 [S+1] or None (one token per request); scale float32
[S][K] or None; v float32 [T][ldv]; workspace/plan a uint8 device tensor.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

from . import accounting  # noqa: F401  (pure Python byte/FLOP accounting)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "liblora_hip.so")

LORA_F32, LORA_BF16 = 0, 1
STATUS = {0: "LORA_OK", -1: "LORA_EINVAL", -2: "LORA_ESHAPE", -3: "LORA_EWORKSPACE", -4: "LORA_EUNSUPPORTED",
          -5: "LORA_EHIP"}


class LoraError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = STATUS.get(status, str(status))
        super().__init__(f"{what}: {msg}" if what else msg)


class lora_pool(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("n_adapters", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("ranks", ctypes.c_void_p)]


class lora_batch(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("n_segments", ctypes.c_int32), ("seg_off", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("max_slots", ctypes.c_int32), ("scale", ctypes.c_void_p)]


class lora_problem(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("ldx", ctypes.c_int64), ("ldy", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises LoraError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LoraError(-5, f"HIP library not built ({LIB_PATH}); run python -m rank_sgmv_bgmv_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        pp, pb = ctypes.POINTER(lora_pool), ctypes.POINTER(lora_batch)
        sig = {
            "lora_workspace_size": (SZ, [pb, I32]),
            "lora_plan_build": (ctypes.c_int, [pb, I32, P, SZ, P]),
            "lora_apply": (ctypes.c_int, [pp, pb, P, I64, P, I64, P, SZ, P]),
            "lora_apply_noalloc": (ctypes.c_int, [pp, pb, P, I64, P, I64, P]),
            "lora_shrink": (ctypes.c_int, [pp, pb, P, I64, P, I64, P, SZ, P]),
            "lora_expand": (ctypes.c_int, [pp, pb, P, I64, P, I64, P, SZ, P]),
            "lora_apply_planned": (ctypes.c_int, [pp, pb, P, SZ, P, I64, P, I64, P]),
            "lora_shrink_planned": (ctypes.c_int, [pp, pb, P, SZ, P, I64, P, I64, P]),
            "lora_expand_planned": (ctypes.c_int, [pp, pb, P, SZ, P, I64, P, I64, P]),
            "lora_apply_multi": (ctypes.c_int, [pp, pb, P, SZ, I32, P, I32, P]),
            "lora_apply_sliced": (ctypes.c_int, [pp, pb, P, SZ, I32, I32, P, P, I32, P]),
            "lora_read_device_errors": (ctypes.c_int, [P, SZ, ctypes.POINTER(I32), P]),
            "lora_merge": (ctypes.c_int, [pp, P, P, I32, ctypes.c_float, P, I64, P]),
            "lora_merge_multi": (ctypes.c_int, [pp, P, P, I32, ctypes.c_float, I32, P, I32, P]),
            "lora_pool_load": (ctypes.c_int, [pp, I32, P, P, P]),
            "lora_calib_gather_read": (ctypes.c_int, [P, P, I32, I32, I32, P, I32, I32, P, P]),
            "lora_calib_tile_stream": (ctypes.c_int, [P, P, I32, I32, I32, P, I32, I32, I32, P, P]),
            "lora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "lora_abi_version": (I32, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


# ------------------------------------------------------------- marshalling --
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return LORA_F32
    if t.dtype == torch.bfloat16:
        return LORA_BF16
    raise LoraError(-1, f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(st: int, what: str):
    if st != 0:
        raise LoraError(st, what)


class Pool:
    """A resident adapter pool: A [n][r][d_in], B [n][d_out][r]; ranks: an optional
    int32 device tensor [n] of per-adapter ranks (adapters stored at rank r)."""

    def __init__(self, A, B, ranks=None):
        if A.dim() != 3 or B.dim() != 3 or not A.is_contiguous() or not B.is_contiguous():
            raise LoraError(-2, "A and B must be contiguous 3-D tensors")
        n, r, d_in = A.shape
        if B.shape[0] != n or B.shape[2] != r or B.dtype != A.dtype:
            raise LoraError(-2, "B must be [n][d_out][r] with A's dtype")
        if ranks is not None and (ranks.dtype != _torch().int32 or tuple(ranks.shape) != (n,)
                                  or not ranks.is_contiguous() or ranks.device != A.device):
            raise LoraError(-2, "ranks must be a contiguous int32 device tensor [n]")
        self.A, self.B, self.ranks = A, B, ranks
        self.n, self.r, self.d_in, self.d_out = int(n), int(r), int(d_in), int(B.shape[1])
        self.c = lora_pool(_ptr(A), _ptr(B), self.n, self.r, self.d_in, self.d_out, _dtype_code(A), _ptr(ranks))


class Batch:
    """Which adapters apply to which rows (see lora_batch in include/lora.h)."""

    def __init__(self, n_tokens: int, idx, seg_off=None, scale=None):
        torch = _torch()
        if idx.dtype != torch.int32 or idx.dim() != 2 or not idx.is_contiguous():
            raise LoraError(-2, "idx must be a contiguous int32 [S][K] tensor")
        S, K = idx.shape
        if seg_off is not None and (seg_off.dtype != torch.int32 or seg_off.numel() != S + 1):
            raise LoraError(-2, "seg_off must be int32 [S+1]")
        if scale is not None and (scale.dtype != torch.float32 or tuple(scale.shape) != (S, K)
                                  or not scale.is_contiguous()):
            raise LoraError(-2, "scale must be a contiguous float32 [S][K] tensor")
        if seg_off is None and S != n_tokens:
            raise LoraError(-2, "per-token mode needs idx with n_tokens rows")
        self.idx, self.seg_off, self.scale = idx, seg_off, scale
        self.T, self.S, self.K = int(n_tokens), int(S), int(K)
        self.c = lora_batch(self.T, self.S, _ptr(seg_off), _ptr(idx), self.K, _ptr(scale))


def _ld(t) -> int:
    if t.dim() != 2:
        raise LoraError(-2, "activations must be 2-D")
    if t.numel() == 0:  # no rows: torch reports arbitrary strides for empty views
        return max(int(t.shape[1]), 1)
    if t.stride(1) != 1:
        raise LoraError(-2, "activations must have unit column stride")
    return int(t.stride(0))


def _same_device(what: str, dev, *tensors):
    for t in tensors:
        if t is not None and t.device != dev:
            raise LoraError(-1, f"{what}: every tensor must be on {dev} (found {t.device})")


def _check_rows(what: str, pool: "Pool", batch: Batch, x=None, y=None, v=None, ws=None):
    """Shapes, dtypes and devices of one call's tensors against its pool and batch:
    x [>= T][>= d_in] and y [>= T][>= d_out] of the pool's dtype, v float32
    [>= T][>= K*r], everything (batch tensors included) on the pool's device."""
    torch = _torch()
    dev = pool.A.device
    if dev.type != "cuda":
        raise LoraError(-1, f"{what}: the pool must be in device memory")
    _same_device(what, dev, pool.B, pool.ranks, batch.idx, batch.seg_off, batch.scale, x, y, v, ws)
    for name, t, cols, dt in (("x", x, pool.d_in, pool.A.dtype), ("y", y, pool.d_out, pool.A.dtype),
                              ("v", v, batch.K * pool.r, torch.float32)):
        if t is None:
            continue
        if t.dim() != 2 or t.shape[0] < batch.T or t.shape[1] < cols:
            raise LoraError(-2, f"{what}: {name} must be at least [{batch.T}][{cols}] (got {tuple(t.shape)})")
        if t.dtype != dt:
            raise LoraError(-2, f"{what}: {name} must be {dt} (got {t.dtype})")


def lora_workspace_size(batch: Batch, n_adapters: int) -> int:
    return int(lib().lora_workspace_size(ctypes.byref(batch.c), n_adapters))


def new_workspace(batch: Batch, n_adapters: int, device):
    torch = _torch()
    nbytes = lora_workspace_size(batch, n_adapters)
    if nbytes == 0:
        raise LoraError(-2, "invalid batch")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def lora_plan_build(batch: Batch, n_adapters: int, plan):
    _same_device("lora_plan_build", plan.device, batch.idx, batch.seg_off, batch.scale)
    _check(lib().lora_plan_build(ctypes.byref(batch.c), n_adapters, _ptr(plan), plan.numel(), _stream(plan)),
           "lora_plan_build")


def lora_apply(pool: Pool, batch: Batch, x, y, ws):
    _check_rows("lora_apply", pool, batch, x=x, y=y, ws=ws)
    _check(lib().lora_apply(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(x), _ld(x), _ptr(y), _ld(y), _ptr(ws),
                            ws.numel(), _stream(y)), "lora_apply")


def lora_apply_noalloc(pool: Pool, batch: Batch, x, y):
    """lora_apply with the plan in the library's own device array (no workspace,
    nothing allocated); calls that overlap on one GPU race."""
    _check_rows("lora_apply_noalloc", pool, batch, x=x, y=y)
    _check(lib().lora_apply_noalloc(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(x), _ld(x), _ptr(y), _ld(y),
                                    _stream(y)), "lora_apply_noalloc")


def lora_shrink(pool: Pool, batch: Batch, x, v, ws):
    _check_rows("lora_shrink", pool, batch, x=x, v=v, ws=ws)
    _check(lib().lora_shrink(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(x), _ld(x), _ptr(v), _ld(v),
                             _ptr(ws), ws.numel(), _stream(v)), "lora_shrink")


def lora_expand(pool: Pool, batch: Batch, v, y, ws):
    _check_rows("lora_expand", pool, batch, y=y, v=v, ws=ws)
    _check(lib().lora_expand(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(v), _ld(v), _ptr(y), _ld(y),
                             _ptr(ws), ws.numel(), _stream(y)), "lora_expand")


def lora_apply_planned(pool: Pool, batch: Batch, plan, x, y):
    _check_rows("lora_apply_planned", pool, batch, x=x, y=y, ws=plan)
    _check(lib().lora_apply_planned(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(plan), plan.numel(), _ptr(x),
                                    _ld(x), _ptr(y), _ld(y), _stream(y)), "lora_apply_planned")


def lora_shrink_planned(pool: Pool, batch: Batch, plan, x, v):
    _check_rows("lora_shrink_planned", pool, batch, x=x, v=v, ws=plan)
    _check(lib().lora_shrink_planned(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(plan), plan.numel(), _ptr(x),
                                     _ld(x), _ptr(v), _ld(v), _stream(v)), "lora_shrink_planned")


def lora_expand_planned(pool: Pool, batch: Batch, plan, v, y):
    _check_rows("lora_expand_planned", pool, batch, y=y, v=v, ws=plan)
    _check(lib().lora_expand_planned(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(plan), plan.numel(), _ptr(v),
                                     _ld(v), _ptr(y), _ld(y), _stream(y)), "lora_expand_planned")


def problems_table(problems: Sequence, device):
    """Device array of lora_problem for (A, B, x, y) tuples of one shape; returns
    (table tensor, all_aligned).  The tensors must stay alive while it is used."""
    torch = _torch()
    rows, aligned = [], True
    for A, B, x, y in problems:
        e = 8 if A.dtype == torch.bfloat16 else 4
        ldx, ldy = _ld(x), _ld(y)
        ptrs = [_ptr(A), _ptr(B), _ptr(x), _ptr(y)]
        aligned &= all(p % 16 == 0 for p in ptrs) and ldx % e == 0 and ldy % e == 0
        rows.append(ptrs + [ldx, ldy])
    table = torch.tensor(rows, dtype=torch.int64).to(device)
    return table, aligned


def lora_apply_multi(shape: Pool, batch: Batch, plan, table, aligned: bool = True):
    """shape: a Pool whose shape (n, r, d_in, d_out, dtype) all problems share."""
    n = int(table.shape[0]) if table.numel() else 0
    _check_rows("lora_apply_multi", shape, batch, ws=plan)
    _same_device("lora_apply_multi", plan.device, table)
    _check(lib().lora_apply_multi(ctypes.byref(shape.c), ctypes.byref(batch.c), _ptr(plan), plan.numel(), n,
                                  _ptr(table), 1 if aligned else 0, _stream(plan)), "lora_apply_multi")


def sliced_table(groups: Sequence, device):
    """Device array of lora_problem for lora_apply_sliced.  groups: a sequence of
    (x, [(A, B, y), ...]) -- one x and its slices (the same number of slices, of
    the same output widths, in every group).  Returns (table, d_outs, all_aligned).
    The tensors must stay alive while the table is used."""
    rows, d_outs = [], None
    for x, slices in groups:
        widths = [int(B.shape[1]) for _, B, _ in slices]
        if d_outs is None:
            d_outs = widths
        elif widths != d_outs:
            raise LoraError(-2, "every group must have slices of the same output widths")
        rows += [(A, B, x, y) for A, B, y in slices]
    table, aligned = problems_table(rows, device)
    return table, d_outs or [], aligned


def lora_apply_sliced(shape: Pool, batch: Batch, plan, table, d_outs: Sequence[int], aligned: bool = True):
    """Groups of projections that read one x (q / k / v, gate / up), one launch:
    table from sliced_table; shape gives n, rank, d_in, dtype (and ranks)."""
    ns = len(d_outs)
    rows = int(table.shape[0]) if table.numel() else 0
    if ns < 1 or rows % ns:
        raise LoraError(-2, "table rows must be a whole number of groups of len(d_outs) slices")
    widths = (ctypes.c_int32 * ns)(*[int(v) for v in d_outs])
    _check_rows("lora_apply_sliced", shape, batch, ws=plan)
    _same_device("lora_apply_sliced", plan.device, table)
    _check(lib().lora_apply_sliced(ctypes.byref(shape.c), ctypes.byref(batch.c), _ptr(plan), plan.numel(), rows // ns,
                                   ns, widths, _ptr(table), 1 if aligned else 0, _stream(plan)), "lora_apply_sliced")


def lora_merge(pool: Pool, idx: Sequence[int], W, scale: Optional[Sequence[float]] = None, alpha: float = 1.0):
    """W += alpha * sum_k scale[k] B_idx[k] A_idx[k] in place (alpha = -1 unmerges).
    idx and scale are host sequences; W is a [d_out][ldw] device tensor of the pool's dtype."""
    if W.dim() != 2 or W.shape[0] != pool.d_out or W.shape[1] < pool.d_in or W.dtype != pool.A.dtype:
        raise LoraError(-2, "W must be [d_out][>= d_in] with the pool's dtype")
    ids = (ctypes.c_int32 * len(idx))(*[int(i) for i in idx])
    sc = None if scale is None else (ctypes.c_float * len(scale))(*[float(v) for v in scale])
    _check(lib().lora_merge(ctypes.byref(pool.c), ids, sc, len(idx), float(alpha), _ptr(W), _ld(W), _stream(W)),
           "lora_merge")


def merge_table(problems: Sequence, device):
    """Device array of lora_merge_problem for (A, B, W) tuples of one shape;
    returns (table tensor, all_aligned).  The tensors must stay alive while it is used."""
    torch = _torch()
    rows, aligned = [], True
    for A, B, W in problems:
        e = 8 if A.dtype == torch.bfloat16 else 4
        ldw = _ld(W)
        ptrs = [_ptr(A), _ptr(B), _ptr(W)]
        aligned &= all(p % 16 == 0 for p in ptrs) and ldw % e == 0
        rows.append(ptrs + [ldw])
    table = torch.tensor(rows, dtype=torch.int64).to(device)
    return table, aligned


def lora_merge_multi(shape: Pool, idx: Sequence[int], table, aligned: bool = True,
                     scale: Optional[Sequence[float]] = None, alpha: float = 1.0):
    """lora_merge over every (A, B, W) of a merge_table in one launch."""
    ids = (ctypes.c_int32 * len(idx))(*[int(i) for i in idx])
    sc = None if scale is None else (ctypes.c_float * len(scale))(*[float(v) for v in scale])
    n = int(table.shape[0]) if table.numel() else 0
    _check(lib().lora_merge_multi(ctypes.byref(shape.c), ids, sc, len(idx), float(alpha), n, _ptr(table),
                                  1 if aligned else 0, _stream(table)), "lora_merge_multi")


def lora_pool_load(pool: Pool, slot: int, A_host, B_host, stream=None):
    """Copy one adapter (host tensors [r][d_in] and [d_out][r], the pool's dtype,
    contiguous; pinned for an asynchronous copy) into slot `slot` of the pool,
    on `stream` (a torch.cuda.Stream; the current stream by default)."""
    torch = _torch()
    if A_host.device.type != "cpu" or B_host.device.type != "cpu":
        raise LoraError(-1, "A_host and B_host must be host tensors")
    if (tuple(A_host.shape) != (pool.r, pool.d_in) or tuple(B_host.shape) != (pool.d_out, pool.r)
            or not A_host.is_contiguous() or not B_host.is_contiguous()
            or A_host.dtype != pool.A.dtype or B_host.dtype != pool.A.dtype):
        raise LoraError(-2, "A_host must be [r][d_in] and B_host [d_out][r], contiguous, of the pool's dtype")
    s = (stream or torch.cuda.current_stream(pool.A.device)).cuda_stream
    _check(lib().lora_pool_load(ctypes.byref(pool.c), int(slot), _ptr(A_host), _ptr(B_host), s), "lora_pool_load")


def lora_read_device_errors(plan) -> int:
    cnt = ctypes.c_int32(0)
    _check(lib().lora_read_device_errors(_ptr(plan), plan.numel(), ctypes.byref(cnt), _stream(plan)),
           "lora_read_device_errors")
    return int(cnt.value)


def lora_status_string(status: int) -> str:
    return lib().lora_status_string(status).decode()


def plan_header(plan):
    """The plan's header words (a host copy; synchronizes)."""
    return plan[:256].view(_torch().int32).cpu().tolist()[:16]


def lora_calib_gather_read(pool, off, blocks_per_group: int, block_bytes: int, sink, rmw=None, rmw_bytes: int = 0,
                           lds_bytes: int = 0):
    """Measurement aid (include/lora_calib.h): workgroup g reads the
    blocks_per_group blocks of `pool` (a device tensor) that start at byte
    offsets off[g * blocks_per_group ...] (int64 device tensor), block_bytes
    each; with `rmw` it also reads and writes back rmw_bytes of rmw at
    g * rmw_bytes.  Each workgroup reserves lds_bytes of LDS it does not use
    (limiting how many share a compute unit).  sink (int32 device tensor, one
    word per group) receives each group's XOR.  The caller keeps every block
    inside `pool`."""
    torch = _torch()
    if off.dtype != torch.int64 or blocks_per_group < 1 or off.numel() % blocks_per_group:
        raise LoraError(-2, "lora_calib_gather_read: off must be int64, blocks_per_group offsets per group")
    n_groups = off.numel() // blocks_per_group
    if sink.numel() * sink.element_size() < 4 * n_groups:
        raise LoraError(-2, "lora_calib_gather_read: sink must hold one word per group")
    if rmw is not None and rmw.numel() * rmw.element_size() < n_groups * rmw_bytes:
        raise LoraError(-2, "lora_calib_gather_read: rmw must hold rmw_bytes per group")
    _same_device("lora_calib_gather_read", pool.device, off, sink, rmw)
    _check(lib().lora_calib_gather_read(_ptr(pool), _ptr(off), n_groups, blocks_per_group, block_bytes, _ptr(rmw),
                                        rmw_bytes if rmw is not None else 0, lds_bytes, _ptr(sink), _stream(pool)),
           "lora_calib_gather_read")


def lora_calib_tile_stream(x, y, rows: int, row_bytes: int, sink, order: int = 0, adapters=None,
                           n_adapters: int = 0, lds_bytes: int = 0):
    """Measurement aid (include/lora_calib.h): the prefill tiles' traffic with
    no arithmetic.  Workgroup t reads its `rows` rows (row_bytes each) of the
    device tensors x and y and writes y's back unchanged, in the MFMA
    kernel's stage order (order 0, reading a stage of adapter t % n_adapters
    beside each when `adapters` is given) or whole rows at a time (order 1).
    sink (int32 device tensor, one word per tile) receives each tile's XOR."""
    if rows < 1 or row_bytes < 1 or x.numel() * x.element_size() % (rows * row_bytes):
        raise LoraError(-2, "lora_calib_tile_stream: x must hold whole tiles of rows x row_bytes")
    n_tiles = x.numel() * x.element_size() // (rows * row_bytes)
    if y.numel() * y.element_size() != x.numel() * x.element_size():
        raise LoraError(-2, "lora_calib_tile_stream: y must be the size of x")
    if sink.numel() * sink.element_size() < 4 * n_tiles:
        raise LoraError(-2, "lora_calib_tile_stream: sink must hold one word per tile")
    if adapters is not None:
        per = row_bytes // 512 * 32768 + row_bytes // 256 * 16384
        if n_adapters < 1 or adapters.numel() * adapters.element_size() < n_adapters * per:
            raise LoraError(-2, "lora_calib_tile_stream: adapters must hold n_adapters A and B blocks")
    _same_device("lora_calib_tile_stream", x.device, y, sink, adapters)
    _check(lib().lora_calib_tile_stream(_ptr(x), _ptr(y), n_tiles, rows, row_bytes, _ptr(adapters),
                                        n_adapters if adapters is not None else 0, order, lds_bytes, _ptr(sink),
                                        _stream(x)),
           "lora_calib_tile_stream")
