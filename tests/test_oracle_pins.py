"""The fp64 oracle against its pins (CPU only)."""
import os

import numpy as np
import pytest

import oracle
import workloads as W
import _pins
from rank_sgmv_bgmv_amd import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_lora_costs_golden_table():
    """The page's printed FLUX table (57 layers x 4 adapted 3072 x 3072 attention
    projections, 4608 tokens, 16-bit weights, 3350 GB/s) follows from the
    accounting used for bytes and FLOPs: extra compute = the adapter's FLOPs over
    the projections' own 2 N d^2; LoRA size = the adapters' bytes; merge time =
    the merge's weight traffic over the bandwidth."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "lora_costs_flux.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 4
    d, n_mats, tokens, elem, gbps = 3072, 57 * 4, 4608, 2, 3350.0
    for rank, extra_s, mb_s, ms_s in rows:
        r = int(rank)
        extra = accounting.lora_flops(tokens, r, d, d) / (2 * tokens * d * d)
        mib = n_mats * accounting.adapter_bytes(r, d, d, elem) / 2 ** 20
        merge_ms = accounting.merge_bytes(n_mats, d, d, elem) / (gbps * 1e9) * 1e3
        assert f"{extra:.1%}" == extra_s
        assert f"{mib:.0f}" == mb_s
        assert f"{merge_ms:.0f}" == ms_s
        # the same ratio in closed form: 2 r / d
        assert abs(extra - 2 * r / d) < 1e-15


def test_oracle_macs_match_accounting(orc):
    case = W.random_case(3, dtype=W.F32, n=3, r=5, d_in=7, d_out=6, S=4, K=2, min_len=1, max_len=3, p_empty=0.3)
    _, _, _, macs = orc.apply_case(case)
    touched, slot_tokens, _ = accounting.batch_work(case.batch.seg_bounds(), case.batch.idx, 3)
    assert 2 * macs == accounting.lora_flops(slot_tokens, 5, 7, 6)


def test_oracle_refuses_bad_input(orc):
    case = W.random_case(4, dtype=W.F32, n=3, r=2, d_in=4, d_out=4, S=3, K=1, min_len=1, max_len=2)
    bad = case.batch.idx.copy(); bad[0, 0] = 3
    with pytest.raises(oracle.OracleError):
        orc.apply(case.dtype, case.pool.A, case.pool.B, case.x, case.y, T=case.batch.T, S=3, K=1,
                  seg_off=case.batch.seg_off, idx=bad)
    bad[0, 0] = -2
    with pytest.raises(oracle.OracleError):
        orc.apply(case.dtype, case.pool.A, case.pool.B, case.x, case.y, T=case.batch.T, S=3, K=1,
                  seg_off=case.batch.seg_off, idx=bad)
    seg = case.batch.seg_off.copy(); seg[1], seg[2] = seg[2], seg[1] - 1
    with pytest.raises(oracle.OracleError):
        orc.apply(case.dtype, case.pool.A, case.pool.B, case.x, case.y, T=case.batch.T, S=3, K=1,
                  seg_off=seg, idx=case.batch.idx)


def test_oracle_bf16_decoding(orc):
    """bf16 inputs are widened exactly: a bf16 case equals the same values given as fp32."""
    case = W.random_case(9, dtype=W.BF16, n=3, r=4, d_in=16, d_out=8, S=4, K=2, min_len=1, max_len=3,
                         with_scale=True)
    yb, tb, rb, _ = orc.apply_case(case)
    p = case.pool
    yf, tf, rf, _ = orc.apply("f32", W.bf16_bits_to_f32(p.A), W.bf16_bits_to_f32(p.B), W.bf16_bits_to_f32(case.x),
                              W.bf16_bits_to_f32(case.y), T=case.batch.T, S=case.batch.S, K=2,
                              seg_off=case.batch.seg_off, idx=case.batch.idx, scale=case.batch.scale)
    assert np.array_equal(yb, yf) and np.array_equal(tb, tf) and np.array_equal(rb, rf)


def test_oracle_row_subset_and_threads(orc):
    case = W.random_case(10, dtype=W.BF16, n=4, r=8, d_in=32, d_out=24, S=6, K=2, min_len=0, max_len=5,
                         with_scale=True, gaps=True)
    full, tf, rf, _ = orc.apply_case(case, nthreads=1)
    rows = np.array([case.batch.T - 1, 0, 3, 3], np.int32)
    sub, ts, rs, _ = orc.apply_case(case, rows=rows, nthreads=3)
    assert np.array_equal(sub, full[rows]) and np.array_equal(ts, tf[rows]) and np.array_equal(rs, rf[rows])


def test_bf16_encoding_rne():
    """Round-to-nearest-even at the bf16 boundary (input encoding shared by both sides)."""
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0], np.float32)
    bits = W.f32_to_bf16_bits(vals)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0x8000, 0x4780]
    assert np.array_equal(W.bf16_bits_to_f32(bits[:1]), np.array([1.0], np.float32))
