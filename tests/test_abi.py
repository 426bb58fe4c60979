"""The C-ABI library loads and exports what include/lora.h declares; host-side
validation returns the documented status codes without launching anything.
CPU only: no call here reaches a GPU."""
import ctypes
import os
import re

import pytest

import rank_sgmv_bgmv_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "lora_calib.h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(lora_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from rank_sgmv_bgmv_amd import build
        build.build()
    return L.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12, names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_exported_symbols_match_binding(lib):
    for name in declared_functions():
        assert hasattr(L, name) or name in ("lora_abi_version",), f"binding lacks {name}"


def test_abi_version_and_strings(lib):
    assert lib.lora_abi_version() == 104
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.lora_status_string(st)
    assert b"workspace" in lib.lora_status_string(-3)


FAKE = 0x10000  # a non-NULL, 16-byte aligned address that is never dereferenced


def _pool(**kw):
    args = dict(A=FAKE, B=FAKE * 2, n_adapters=4, rank=8, d_in=64, d_out=64, dtype=L.LORA_BF16)
    args.update(kw)
    return L.lora_pool(args["A"], args["B"], args["n_adapters"], args["rank"], args["d_in"], args["d_out"], args["dtype"])


def _batch(**kw):
    args = dict(n_tokens=10, n_segments=3, seg_off=FAKE * 3, idx=FAKE * 4, max_slots=1, scale=None)
    args.update(kw)
    return L.lora_batch(args["n_tokens"], args["n_segments"], args["seg_off"], args["idx"], args["max_slots"], args["scale"])


def test_workspace_size(lib):
    b = _batch()
    n = lib.lora_workspace_size(ctypes.byref(b), 4)
    assert n > 0 and n % 256 == 0
    assert lib.lora_workspace_size(ctypes.byref(_batch(n_tokens=-1)), 4) == 0
    assert lib.lora_workspace_size(ctypes.byref(_batch(max_slots=0)), 4) == 0
    assert lib.lora_workspace_size(ctypes.byref(b), 0) == 0
    big = lib.lora_workspace_size(ctypes.byref(_batch(n_tokens=100000, n_segments=5000)), 1000)
    assert big > n


def _apply(lib, pool, batch, x=FAKE * 5, ldx=64, y=FAKE * 1000, ldy=64, ws=FAKE * 2000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.lora_workspace_size(ctypes.byref(batch), pool.n_adapters) or 1 << 20
    return lib.lora_apply(ctypes.byref(pool), ctypes.byref(batch), x, ldx, y, ldy, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    (dict(pool=dict(A=None)), -1),
    (dict(pool=dict(dtype=7)), -1),
    (dict(pool=dict(rank=0)), -2),
    (dict(pool=dict(rank=257)), -4),
    (dict(pool=dict(d_in=0)), -2),
    (dict(pool=dict(n_adapters=0)), -2),
    (dict(batch=dict(n_tokens=-1)), -2),
    (dict(batch=dict(max_slots=9)), -4),
    (dict(batch=dict(max_slots=0)), -2),
    (dict(batch=dict(idx=None)), -1),
    (dict(batch=dict(n_segments=-2)), -2),
    (dict(pool=dict(rank=256), batch=dict(max_slots=8)), -4),
    (dict(ldx=63), -2),
    (dict(ldy=10), -2),
    (dict(x=None), -1),
    (dict(y=None), -1),
    (dict(y=FAKE * 5 + 64), -1),            # y overlaps x
    (dict(ws=None), -3),
    (dict(ws_bytes=100), -3),
])
def test_apply_validation(lib, case, expect):
    pool = _pool(**case.get("pool", {}))
    batch = _batch(**case.get("batch", {}))
    kw = {k: v for k, v in case.items() if k not in ("pool", "batch")}
    assert _apply(lib, pool, batch, **kw) == expect


def test_split_and_multi_validation(lib):
    pool, batch = _pool(), _batch()
    ws_bytes = lib.lora_workspace_size(ctypes.byref(batch), 4)
    # ldv < K * rank
    assert lib.lora_shrink(ctypes.byref(pool), ctypes.byref(batch), FAKE, 64, FAKE * 1000, 7, FAKE * 2000, ws_bytes, None) == -2
    assert lib.lora_expand(ctypes.byref(pool), ctypes.byref(batch), None, 8, FAKE * 1000, 64, FAKE * 2000, ws_bytes, None) == -1
    assert lib.lora_apply_multi(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, 2, None, 1, None) == -1
    assert lib.lora_apply_multi(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, 16, 2, FAKE, 1, None) == -3
    assert lib.lora_apply_multi(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, -1, FAKE, 1, None) == -2
    # sliced: host array of output widths, 1..8 slices, each width >= 1
    w3 = (ctypes.c_int32 * 3)(64, 16, 16)
    sl = lib.lora_apply_sliced
    assert sl(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, 2, 3, None, FAKE, 1, None) == -1
    assert sl(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, 2, 3, w3, None, 1, None) == -1
    assert sl(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, 2, 0, w3, FAKE, 1, None) == -2
    assert sl(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, 2, 9, w3, FAKE, 1, None) == -2
    assert sl(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, -1, 3, w3, FAKE, 1, None) == -2
    assert sl(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, 2, 3, (ctypes.c_int32 * 3)(64, 0, 16),
              FAKE, 1, None) == -2
    assert sl(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, 16, 2, 3, w3, FAKE, 1, None) == -3
    assert sl(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, 2, 3, w3, FAKE + 4, 1, None) == -1
    # zero groups: nothing to do (no launch)
    assert sl(ctypes.byref(pool), ctypes.byref(batch), FAKE * 2000, ws_bytes, 0, 3, w3, None, 1, None) == 0
    assert lib.lora_plan_build(ctypes.byref(batch), 0, FAKE * 2000, ws_bytes, None) == -2
    assert lib.lora_plan_build(ctypes.byref(batch), 4, FAKE * 2000, 16, None) == -3
    cnt = ctypes.c_int32(0)
    assert lib.lora_read_device_errors(None, 1 << 20, ctypes.byref(cnt), None) == -1


def _merge(lib, pool, idx=(1,), scale=None, n_slots=None, alpha=1.0, W=FAKE * 3000, ldw=64):
    ids = (ctypes.c_int32 * max(len(idx), 1))(*idx)
    sc = None if scale is None else (ctypes.c_float * len(scale))(*scale)
    n = len(idx) if n_slots is None else n_slots
    return lib.lora_merge(ctypes.byref(pool), ids, sc, n, alpha, W, ldw, None)


@pytest.mark.parametrize("case,expect", [
    (dict(idx=(4,)), -1),                   # index >= n_adapters
    (dict(idx=(0, -2)), -1),                # index below -1
    (dict(n_slots=0), -2),
    (dict(idx=(0,) * 9), -4),
    (dict(ldw=63), -2),
    (dict(W=None), -1),
    (dict(W=FAKE + 128), -1),               # W overlaps the pool's A
    (dict(pool=dict(B=None)), -1),
    (dict(pool=dict(rank=300)), -4),
    (dict(idx=(-1, -1)), 0),                # nothing to merge: returns before any launch
])
def test_merge_validation(lib, case, expect):
    pool = _pool(**case.pop("pool", {}))
    assert _merge(lib, pool, **case) == expect


def test_merge_multi_validation(lib):
    shape = _pool()
    ids = (ctypes.c_int32 * 2)(0, 1)
    assert lib.lora_merge_multi(None, ids, None, 2, 1.0, 3, FAKE, 1, None) == -1
    assert lib.lora_merge_multi(ctypes.byref(shape), ids, None, 2, 1.0, 3, None, 1, None) == -1
    assert lib.lora_merge_multi(ctypes.byref(shape), ids, None, 2, 1.0, -1, FAKE, 1, None) == -2
    assert lib.lora_merge_multi(ctypes.byref(shape), None, None, 2, 1.0, 3, FAKE, 1, None) == -1
    bad = (ctypes.c_int32 * 2)(0, 4)
    assert lib.lora_merge_multi(ctypes.byref(shape), bad, None, 2, 1.0, 3, FAKE, 1, None) == -1
    assert lib.lora_merge_multi(ctypes.byref(shape), ids, None, 2, 1.0, 0, FAKE, 1, None) == 0  # nothing to do


def test_pool_load_validation(lib):
    pool = _pool()
    assert lib.lora_pool_load(ctypes.byref(pool), 4, FAKE, FAKE, None) == -2
    assert lib.lora_pool_load(ctypes.byref(pool), -1, FAKE, FAKE, None) == -2
    assert lib.lora_pool_load(ctypes.byref(pool), 0, None, FAKE, None) == -1
    assert lib.lora_pool_load(ctypes.byref(_pool(A=None)), 0, FAKE, FAKE, None) == -1


def test_sliced_table_layout_and_checks():
    """The binding's table for lora_apply_sliced (host-side marshalling only):
    group-major rows of (A, B, x, y, ldx, ldy), the slices' widths, and the
    errors it raises before anything reaches the library."""
    import torch
    n, r, d_in, T = 3, 8, 64, 5
    x = torch.zeros((T, d_in + 8), dtype=torch.bfloat16)[:, :d_in]

    def slice_(d_out):
        return (torch.zeros((n, r, d_in), dtype=torch.bfloat16), torch.zeros((n, d_out, r), dtype=torch.bfloat16),
                torch.zeros((T, d_out), dtype=torch.bfloat16))

    g0, g1 = [slice_(32), slice_(16)], [slice_(32), slice_(16)]
    table, d_outs, aligned = L.sliced_table([(x, g0), (x, g1)], "cpu")
    assert d_outs == [32, 16] and aligned
    assert tuple(table.shape) == (4, 6)
    rows = table.tolist()
    for i, (A, B, y) in enumerate(g0 + g1):
        assert rows[i][:4] == [A.data_ptr(), B.data_ptr(), x.data_ptr(), y.data_ptr()]
        assert rows[i][4:] == [d_in + 8, y.shape[1]]
    with pytest.raises(L.LoraError):
        L.sliced_table([(x, [slice_(32), slice_(16)]), (x, [slice_(32), slice_(24)])], "cpu")
    shape = L.Pool(*g0[0][:2])
    with pytest.raises(L.LoraError):  # 4 rows are not whole groups of 3 slices
        L.lora_apply_sliced(shape, None, None, table, [32, 16, 16])


def test_calib_gather_read_host_checks(lib):
    f = lib.lora_calib_gather_read
    ok = dict(pool=FAKE, off=FAKE, n=4, bpg=2, bb=1 << 17, rmw=None, rb=0, lds=0, sink=FAKE * 2)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["pool"], a["off"], a["n"], a["bpg"], a["bb"], a["rmw"], a["rb"], a["lds"], a["sink"], None)

    assert call(pool=None) == -1 and call(off=None) == -1 and call(sink=None) == -1 and call(n=-1) == -1
    assert call(bpg=0) == -2 and call(bb=0) == -2 and call(bb=16384) == -2
    assert call(rmw=FAKE * 3, rb=0) == -2 and call(rmw=FAKE * 3, rb=1000) == -2
    assert call(rmw=FAKE * 3, rb=5 * 4096) == -2
    assert call(lds=-1) == -2 and call(lds=65537) == -2
    assert call(n=0) == 0 and call(n=0, rmw=FAKE * 3, rb=8192, lds=65536) == 0  # nothing to read: nothing launched


def test_calib_tile_stream_host_checks(lib):
    f = lib.lora_calib_tile_stream
    ok = dict(x=FAKE, y=FAKE * 2, n=4, rows=48, rb=8192, ad=None, na=0, order=0, lds=0, sink=FAKE * 3)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["y"], a["n"], a["rows"], a["rb"], a["ad"], a["na"], a["order"], a["lds"], a["sink"], None)

    assert call(x=None) == -1 and call(y=None) == -1 and call(sink=None) == -1 and call(n=-1) == -1
    assert call(ad=FAKE * 4, na=0) == -1
    assert call(rows=0) == -2 and call(rows=65) == -2 and call(rb=512) == -2 and call(rb=1536) == -2
    assert call(rb=65536 + 1024) == -2 and call(order=2) == -2 and call(order=-1) == -2
    assert call(lds=-1) == -2 and call(lds=65537) == -2
    assert call(n=0) == 0 and call(n=0, ad=FAKE * 4, na=8, order=1, lds=65536) == 0  # nothing launched


def test_calib_binding_checks():
    """The binding refuses offsets that are not int64, an offset count that is
    not whole groups, and a sink or slice buffer too small, before any pointer
    reaches the library (CPU tensors: nothing is launched)."""
    import torch
    pool = torch.zeros(1 << 16, dtype=torch.uint8)
    sink = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(L.LoraError):
        L.lora_calib_gather_read(pool, torch.zeros(4, dtype=torch.int32), 1, 32768, sink)
    with pytest.raises(L.LoraError):
        L.lora_calib_gather_read(pool, torch.zeros(5, dtype=torch.int64), 2, 32768, sink)
    with pytest.raises(L.LoraError):
        L.lora_calib_gather_read(pool, torch.zeros(8, dtype=torch.int64), 1, 32768, sink)
    with pytest.raises(L.LoraError):
        L.lora_calib_gather_read(pool, torch.zeros(4, dtype=torch.int64), 1, 32768, sink,
                                 rmw=torch.zeros(4096, dtype=torch.uint8), rmw_bytes=4096)
    x = torch.zeros(4 * 2 * 1024, dtype=torch.uint8)  # four tiles of 2 rows of 1 KB
    with pytest.raises(L.LoraError):  # not whole tiles
        L.lora_calib_tile_stream(x, x.clone(), 3, 1024, sink)
    with pytest.raises(L.LoraError):  # y not the size of x
        L.lora_calib_tile_stream(x, x[:1024].clone(), 2, 1024, sink)
    with pytest.raises(L.LoraError):  # sink too small
        L.lora_calib_tile_stream(x, x.clone(), 2, 1024, sink[:3])
    with pytest.raises(L.LoraError):  # adapters too small for n_adapters
        L.lora_calib_tile_stream(x, x.clone(), 2, 1024, sink, adapters=torch.zeros(1 << 16, dtype=torch.uint8),
                                 n_adapters=2)
