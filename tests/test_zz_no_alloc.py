"""lora_apply_noalloc -- lora_apply for callers that cannot allocate, with the
plan in the library's own device array -- through the C ABI, against
lora_apply with a caller workspace (bit for bit: the same kernels on the same
plan) and the fp64 oracle, on calls in a row whose second input is smaller
than the first (the array keeps the last call's plan; nothing of it may leak
into the next call).  Batches whose plan does not fit the array are refused
before anything is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import rank_sgmv_bgmv_amd as L
import workloads as W
from _gpu import DevCase, assert_parity, from_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _with_workspace(case):
    return DevCase(case).apply()


def _noalloc(case):
    dc = DevCase(case)
    L.lora_apply_noalloc(dc.pool, dc.batch, dc.x, dc.y)
    torch.cuda.synchronize()
    return from_dev(dc.y_full, case.dtype)


CASES = [
    # prefill and decode tiles (MFMA and VALU kernels), stacked scaled slots, an empty request
    ("mixed_large", dict(dtype=W.BF16, n=6, r=32, d_in=256, d_out=320, S=12, K=2, min_len=0, max_len=120,
                         with_scale=True, p_empty=0.2)),
    # smaller: fewer requests, fewer rows, rows outside every request
    ("segmented_small", dict(dtype=W.BF16, n=4, r=16, d_in=128, d_out=96, S=5, min_len=0, max_len=9, gaps=True)),
    # one token per request, then fp32 on the scalar path
    ("decode", dict(dtype=W.BF16, n=40, r=16, d_in=512, d_out=512, per_token=True, S=64)),
    ("f32_scalar_tiny", dict(dtype=W.F32, n=3, r=3, d_in=17, d_out=29, S=3, min_len=1, max_len=5)),
]


def test_noalloc_matches_apply_on_calls_in_a_row(orc):
    for i, (name, kw) in enumerate(CASES):
        case = W.random_case(8000 + i, **kw)
        want = _with_workspace(case)
        got = _noalloc(case)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), name
        y_ref, touched, _, _ = orc.apply_case(case)
        assert_parity(case, got, y_ref, touched, what=f"noalloc {name}")


def test_noalloc_refuses_a_plan_larger_than_its_array():
    lib = L.lib()
    A = torch.zeros((4, 16, 64), dtype=torch.bfloat16, device="cuda:0")
    B = torch.zeros((4, 64, 16), dtype=torch.bfloat16, device="cuda:0")
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda:0")
    y = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda:0")
    idx = torch.zeros((8, 1), dtype=torch.int32, device="cuda:0")
    pool = L.lora_pool(A.data_ptr(), B.data_ptr(), 4, 16, 64, 64, L.LORA_BF16, None)
    T = 200000  # one-token requests: a plan of about 30 MB
    batch = L.lora_batch(T, T, None, idx.data_ptr(), 1, None)
    assert lib.lora_workspace_size(ctypes.byref(batch), 4) > 8 << 20
    st = lib.lora_apply_noalloc(ctypes.byref(pool), ctypes.byref(batch), x.data_ptr(), 64, y.data_ptr(), 64, None)
    assert st == -4  # LORA_EUNSUPPORTED, nothing launched
    torch.cuda.synchronize()
    assert not y.any()
