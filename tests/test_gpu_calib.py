"""The gather-read and tile-stream probes (include/lora_calib.h), measurement aids the
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


@pytest.mark.parametrize("rows,row_bytes,order,n_ad,lds", [(48, 8192, 0, 3, 0), (48, 8192, 1, 0, 65536),
                                                          (5, 2048, 0, 0, 0), (64, 3072, 1, 0, 0),
                                                          (17, 1024, 0, 2, 65536)])
def test_tile_stream_xor(rows, row_bytes, order, n_ad, lds):
    """The tile-stream probe reads every byte of its tiles of x and y (and, in
    stage order, of its adapter's A and B) exactly once and writes y back
    unchanged: each sink word is that XOR, computed here with numpy."""
    rng = np.random.default_rng(12)
    n_tiles = 7
    words = n_tiles * rows * row_bytes // 4
    xh = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    yh = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    x = torch.from_numpy(xh.view(np.int32)).to(DEV)
    y = torch.from_numpy(yh.view(np.int32)).to(DEV)
    sink = torch.zeros(n_tiles, dtype=torch.int32, device=DEV)
    ad = adh = None
    per = row_bytes // 512 * 32768 + row_bytes // 256 * 16384
    if n_ad:
        adh = rng.integers(0, 2**32, size=n_ad * per // 4, dtype=np.uint32)
        ad = torch.from_numpy(adh.view(np.int32)).to(DEV)
    L.lora_calib_tile_stream(x, y, rows, row_bytes, sink, order=order, adapters=ad, n_adapters=n_ad, lds_bytes=lds)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(xh.reshape(n_tiles, -1), axis=1) ^ np.bitwise_xor.reduce(yh.reshape(n_tiles, -1),
                                                                                            axis=1)
    if n_ad and order == 0:
        ad_xor = np.bitwise_xor.reduce(adh.reshape(n_ad, -1), axis=1)
        want = want ^ ad_xor[np.arange(n_tiles) % n_ad]
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), yh)
