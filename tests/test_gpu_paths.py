"""GPU parity of paths the other tests reach only at some sizes:

  * every workgroup running many work items (the item walk of the MFMA and
    merge kernels and the look-ahead of the VALU kernel): a child process with
    the launch grid capped at 16 workgroups reruns a subset of the parity tests
    (the environment is read once per process, so it takes a process of its own);
  * the plan kernel with its working arrays in global memory (batches whose
    arrays exceed its LDS budget) and with scans over more than one 1024-wide
    chunk;
  * rank 1 and eight stacked slots on the apply path; every build of the
    stacked MFMA kernel (2, 3 and 4 slots at ranks 16 to 128);
  * a plan that does not match the call: no work, counted in the error word.

"Serving several LoRAs, ControlNet and IP-Adapter", "Exercises" (four
requests): the grouping of rows by adapter, one kernel for every group, results
back in their original rows -- for any batch size and any number of groups.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import rank_sgmv_bgmv_amd as L
import workloads as W
from _gpu import DEV, DevCase, assert_parity, dev_batch, from_dev

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


# Tests rerun in the child process with 16 workgroups per launch.
GRID_CAP_SUBSET = [
    "test_gpu_parity.py::test_random_grid",
    "test_gpu_parity.py::test_decode_x32_multi_sampled",
    "test_gpu_parity.py::test_decode_stacked_multi_sampled",
    "test_gpu_parity.py::test_c3_stacked_sampled",
    "test_gpu_parity.py::test_c5_diffusion_sampled[640-128]",
    "test_gpu_parity.py::test_integer_probe_bitwise",
    "test_gpu_sliced.py::test_sliced_grid",
    "test_gpu_merge.py::test_merge_grid",
    "test_gpu_merge.py::test_merge_multi_equals_single_calls",
    "test_gpu_ranks.py::test_ranks_parity",
    "test_gpu_paths.py::test_stacked_builds",
]


@pytest.mark.timeout(900)
def test_every_workgroup_runs_many_items():
    env = dict(os.environ, LORA_GRID_CAP="16")
    cmd = [sys.executable, "-u", "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "--timeout", "300",
           "--timeout-method", "thread", *[os.path.join(HERE, t) for t in GRID_CAP_SUBSET]]
    print("child:", " ".join(cmd[3:]), flush=True)
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=840)
    tail = (p.stdout + p.stderr)[-4000:]
    print(tail, flush=True)
    assert p.returncode == 0, tail
    assert " passed" in p.stdout


def _full_case(orc, case):
    out = DevCase(case).apply()
    y_ref, touched, _, _ = orc.apply_case(case)
    assert_parity(case, out, y_ref, touched, what=case.name)
    return touched


def test_plan_in_global_memory_per_token(orc):
    """4096 one-token requests over 1000 adapters (Zipf): the plan's working
    arrays (about 170 KB) exceed its LDS budget and stay in global memory."""
    rng = np.random.default_rng(7001)
    batch = W.batch_c2(rng, n=1000, T=4096)
    pool = W.make_pool(rng, W.BF16, 1000, 16, 128, 192)
    x, y = W.make_xy(rng, W.BF16, batch.T, 128, 192)
    case = W.Case("per_token_4096", W.BF16, batch, pool, x, y)
    S, n = batch.S, 1000
    assert (4 * (S + 1) + 6 * (S + 2) + 2 * (n + 2)) * 4 > 144 * 1024
    assert _full_case(orc, case).all()


@pytest.mark.parametrize("S,n", [(3000, 9), (5000, 40)])
def test_plan_many_requests(orc, S, n):
    """Thousands of short segmented requests with two slots and scales: the
    scans run over several 1024-wide chunks; with 5000 requests the working
    arrays leave LDS for global memory."""
    case = W.random_case(7100 + S, dtype=W.BF16, n=n, r=16, d_in=64, d_out=128, S=S, K=2, min_len=0,
                         max_len=12, with_scale=True, p_empty=0.3, gaps=True)
    touched = _full_case(orc, case)
    assert touched.any() and (~touched).any()


@pytest.mark.parametrize("dtype,vec", [(W.BF16, False), (W.F32, False), (W.F32, True)])
def test_rank_one(orc, dtype, vec):
    """Rank 1: the scalar and vector VALU paths, decode and prefill rows."""
    d_in, d_out = (64, 96) if vec else (61, 37)
    case = W.random_case(7200, dtype=dtype, n=5, r=1 if not vec else 4, d_in=d_in, d_out=d_out, S=12, K=2,
                         min_len=0, max_len=40, with_scale=True, p_empty=0.2)
    if vec:  # rank 1 with the vector path: rank-4 storage, per-adapter rank 1
        ranks = np.ones(5, np.int32)
        dc = DevCase(case)
        dc.pool = L.Pool(dc.A, dc.B, torch.from_numpy(ranks).to(DEV))
        out = dc.apply()
        y_ref, touched, _, _ = orc.apply_case(case, ranks=ranks)
        assert_parity(case, out, y_ref, touched, what="rank 1 (vector path)")
    else:
        _full_case(orc, case)


@pytest.mark.parametrize("name,kw", [
    ("bf16_k8_r16_mfma", dict(dtype=W.BF16, n=12, r=16, d_in=256, d_out=384, S=5, min_len=30, max_len=120)),
    ("bf16_k8_r32_decode", dict(dtype=W.BF16, n=12, r=32, d_in=256, d_out=256, per_token=True, S=40)),
    ("bf16_k8_r64_mfma_half", dict(dtype=W.BF16, n=10, r=64, d_in=192, d_out=160, S=3, min_len=40, max_len=100)),
    ("f32_k8_r8", dict(dtype=W.F32, n=10, r=8, d_in=64, d_out=64, S=9, min_len=0, max_len=30)),
])
def test_eight_slots(orc, name, kw):
    """Eight stacked slots per request (the largest slot count), some empty."""
    case = W.random_case(7300 + len(name), K=8, with_scale=True, p_empty=0.25, **kw)
    _full_case(orc, case)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("r", [16, 32, 64, 128])
def test_stacked_builds(orc, r, K):
    """Every build of the stacked MFMA kernel (ranks 16-128, 2, 3 and 4 slots
    per request): requests with 1 .. K valid slots in one launch, d_in not a
    multiple of any stage width, per-slot scales.  "Serving several LoRAs,
    ControlNet and IP-Adapter", comparison table, stacking row: each stacked
    LoRA adds its own product to the output."""
    case = W.random_case(7500 + 10 * r + K, dtype=W.BF16, n=9, r=r, d_in=328, d_out=200, S=6, K=K,
                         min_len=30, max_len=90, with_scale=True, p_empty=0.2)
    assert case.batch.T >= 128  # the MFMA path
    _full_case(orc, case)


def test_mismatched_plan_does_nothing_and_is_counted(orc):
    """A plan built for another batch size, or a workspace that never held a
    plan: the apply kernels write nothing and count the call."""
    case = W.random_case(7400, dtype=W.BF16, n=4, r=16, d_in=64, d_out=64, S=6, min_len=1, max_len=20)
    other = W.random_case(7401, dtype=W.BF16, n=4, r=16, d_in=64, d_out=64, S=9, min_len=1, max_len=20)
    dc, do = DevCase(case), DevCase(other)
    plan = L.new_workspace(do.batch, 4, DEV)
    L.lora_plan_build(do.batch, 4, plan)
    assert L.lora_read_device_errors(plan) == 0
    big = torch.zeros(max(plan.numel(), L.lora_workspace_size(dc.batch, 4)), dtype=torch.uint8, device=DEV)
    big[:plan.numel()].copy_(plan)
    L.lora_apply_planned(dc.pool, dc.batch, big, dc.x, dc.y)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dc.y_full, W.BF16), case.y), "a mismatched plan wrote y"
    assert L.lora_read_device_errors(big) >= 1
    blank = torch.zeros_like(big)
    L.lora_apply_planned(dc.pool, dc.batch, blank, dc.x, dc.y)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dc.y_full, W.BF16), case.y), "a workspace without a plan wrote y"
    assert L.lora_read_device_errors(blank) >= 1
    # the same call on its own plan works
    L.lora_plan_build(dc.batch, 4, blank)
    L.lora_apply_planned(dc.pool, dc.batch, blank, dc.x, dc.y)
    torch.cuda.synchronize()
    y_ref, touched, _, _ = orc.apply_case(case)
    assert_parity(case, from_dev(dc.y_full, W.BF16), y_ref, touched, what="own plan")
