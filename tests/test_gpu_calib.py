"""The gather-read probe (include/lora_calib.h), a measurement aid the
benchmark reports beside the LoRA kernels: every block a group is given is
read whole, so each sink word equals the XOR of that group's 32-bit words
(computed here with numpy, exactly); the read-and-write-back slice keeps its
values."""
import numpy as np
import pytest
import torch

import rank_sgmv_bgmv_amd as L
from _gpu import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("blk,bpg,rmw_bytes,lds", [(32768, 1, 0, 0), (131072, 1, 0, 65536), (131072, 2, 8192, 65536),
                                                   (65536, 3, 16384, 0)])
def test_gather_read_xor(blk, bpg, rmw_bytes, lds):
    rng = np.random.default_rng(11)
    n_slots, n_groups = 24, 7
    host = rng.integers(0, 2**32, size=(n_slots * blk) // 4, dtype=np.uint32)
    pool = torch.from_numpy(host.view(np.int32)).to(DEV)
    pick = rng.choice(n_slots, size=n_groups * bpg, replace=False).astype(np.int64)
    off = torch.from_numpy(pick * blk).to(DEV)
    sink = torch.zeros(n_groups, dtype=torch.int32, device=DEV)
    rmw = None
    if rmw_bytes:
        rmw_host = rng.integers(0, 2**32, size=n_groups * rmw_bytes // 4, dtype=np.uint32)
        rmw = torch.from_numpy(rmw_host.view(np.int32)).to(DEV)
    L.lora_calib_gather_read(pool, off, bpg, blk, sink, rmw=rmw, rmw_bytes=rmw_bytes, lds_bytes=lds)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    words = host.reshape(n_slots, blk // 4)[pick].reshape(n_groups, -1)
    assert np.array_equal(got, np.bitwise_xor.reduce(words, axis=1))
    if rmw is not None:
        assert np.array_equal(rmw.cpu().numpy().view(np.uint32), rmw_host)
