"""Seeded synthetic inputs for unmerged multi-LoRA batches.

This module only draws random numbers and lays them out; it performs none of
the LoRA arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP library
(``rank_sgmv_bgmv_amd``) take their inputs from here, so a parity test feeds
the same bytes to both sides.

Shapes follow the workloads the pages describe:
  * "Serving several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
    alongside": A is r x d, B is d x r, r usually 8..128, LoRAs resident and
    grouped by request; section "Placement": a pool of 200 rank-64 LoRAs.
  * "EdgeLoRA: An Efficient Multi-Tenant LLM Serving System on Edge Devices",
    abstract: Llama3.1-8B multi-tenant batches (the Llama-3-8B shaped configs).
  * "Co-occurrence Patterns of LoRA Adapters in Production Diffusion Model
    Inference Services", abstract: heavy-tailed adapter popularity and
    multi-adapter requests (Zipf draws and stacked slots below).

Conventions (the same on both sides of every test):
  * A pool  : [n][r][d_in]  row-major; B pool: [n][d_out][r] row-major.
  * x       : [T][ldx], y: [T][ldy].
  * seg_off : int32 [S+1] (non-decreasing) or None = one token per request.
  * idx     : int32 [S][K]; -1 = empty slot / no adapter.
  * scale   : float32 [S][K] or None (= 1.0).
  * bf16 tensors are carried as uint16 bit patterns, rounded from float32 with
    round-to-nearest-even; fp32 tensors as float32.

Draw order inside one case is fixed: lengths -> idx -> scales -> A -> B -> x -> y.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------
# encoding helpers (bit-pattern conversion only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + bias) >> 16).astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)  # keep NaNs NaN (quiet)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def encode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


def decode_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact decoding of an encoded tensor to float64."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(a).astype(np.float64)


# --------------------------------------------------------------------------
# index distributions
# --------------------------------------------------------------------------
def zipf_probs(n: int, alpha: float) -> np.ndarray:
    """Truncated Zipf over ranks 1..n: P(k) proportional to k**-alpha."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-alpha)
    return w / w.sum()


class ZipfAdapters:
    """Adapter-id sampler: Zipf over popularity ranks, ranks mapped to ids by a
    seeded permutation (so the hot adapter is not always id 0)."""

    def __init__(self, rng: np.random.Generator, n: int, alpha: float = 1.1):
        self.n = n
        self.perm = rng.permutation(n).astype(np.int32)
        self.p = zipf_probs(n, alpha)

    def draw(self, rng: np.random.Generator, size: int) -> np.ndarray:
        ranks = rng.choice(self.n, size=size, p=self.p)
        return self.perm[ranks]

    def draw_distinct(self, rng: np.random.Generator, k: int) -> np.ndarray:
        out: list[int] = []
        while len(out) < k:
            a = int(self.draw(rng, 1)[0])
            if a not in out:
                out.append(a)
        return np.array(out, dtype=np.int32)


# --------------------------------------------------------------------------
# a case = one adapted linear layer's inputs for one batch
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Batch:
    T: int                      # rows of x / y
    S: int                      # requests (== T in per-token mode)
    K: int                      # slots per request
    seg_off: Optional[np.ndarray]   # int32 [S+1] or None (per-token)
    idx: np.ndarray             # int32 [S][K]
    scale: Optional[np.ndarray]     # float32 [S][K] or None

    def seg_bounds(self):
        if self.seg_off is None:
            return [(s, s + 1) for s in range(self.S)]
        return [(int(self.seg_off[s]), int(self.seg_off[s + 1])) for s in range(self.S)]


@dataclasses.dataclass
class Pool:
    dtype: str
    n: int
    r: int
    d_in: int
    d_out: int
    A: np.ndarray               # [n][r][d_in]   encoded
    B: np.ndarray               # [n][d_out][r]  encoded


@dataclasses.dataclass
class Case:
    name: str
    dtype: str
    batch: Batch
    pool: Pool
    x: np.ndarray               # [T][ldx] encoded
    y: np.ndarray               # [T][ldy] encoded (y before the LoRA delta)

    @property
    def ldx(self) -> int:
        return int(self.x.shape[1])

    @property
    def ldy(self) -> int:
        return int(self.y.shape[1])


def normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def make_pool(rng, dtype, n, r, d_in, d_out, std=0.02) -> Pool:
    A = encode(normal(rng, (n, r, d_in), std), dtype)
    B = encode(normal(rng, (n, d_out, r), std), dtype)
    return Pool(dtype, n, r, d_in, d_out, A, B)


def make_xy(rng, dtype, T, d_in, d_out, ldx=None, ldy=None):
    ldx = d_in if ldx is None else ldx
    ldy = d_out if ldy is None else ldy
    x = encode(normal(rng, (T, ldx), 1.0), dtype)
    y = encode(normal(rng, (T, ldy), 1.0), dtype)
    return x, y


def offsets_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
CONFIG_DOC = {
    "C1": "tiny SGMV fp32: d_in=d_out=256, r=8, 4 adapters, 8 requests of U{1..16} tokens, one request -1",
    "C2": "decode BGMV bf16: q_proj 4096->4096, r=16, 1000 resident adapters, 64 requests x 1 token, Zipf(1.1)",
    "C3": "prefill SGMV bf16: 4096->4096, r=64, 8 adapters, 32 segments of U{128..1024} tokens",
    "C4": "Llama-3-8B-shaped stack bf16: 32 layers x {q,o 4096->4096; k,v 4096->1024; gate,up 4096->14336; "
          "down 14336->4096}, r=32, 256 adapters per projection, 4x512 prefill + 256 decode tokens, Zipf(1.1)",
    "C5": "diffusion multi-adapter bf16: d in {1280,640}, r in {64,128}, 200 adapters, 16 requests x 4096 tokens, "
          "5 requests stack 2-3 adapters",
}

SEEDS = {"C1": 101, "C2": 102, "C3": 103, "C4": 104, "C5": 105}

# Llama-3-8B projections: name -> (d_in, d_out)
LLAMA3_8B_PROJ = [
    ("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
    ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096),
]
LLAMA3_8B_LAYERS = 32


def case_c1(seed: int = SEEDS["C1"]) -> Case:
    rng = np.random.default_rng(seed)
    S, n = 8, 4
    lengths = rng.integers(1, 17, size=S)
    idx = rng.integers(0, n, size=(S, 1)).astype(np.int32)
    idx[int(rng.integers(0, S)), 0] = -1
    batch = Batch(int(lengths.sum()), S, 1, offsets_from_lengths(lengths), idx, None)
    pool = make_pool(rng, F32, n, 8, 256, 256)
    x, y = make_xy(rng, F32, batch.T, 256, 256)
    return Case("C1", F32, batch, pool, x, y)


def batch_c2(rng, n=1000, T=64) -> Batch:
    z = ZipfAdapters(rng, n, 1.1)
    idx = z.draw(rng, T).reshape(T, 1).astype(np.int32)
    return Batch(T, T, 1, None, idx, None)


def batch_decode_stacked(rng, n=1000, T=64, K=3) -> Batch:
    """The C2 decode batch with C5's stacking: one token per request, and
    round(0.3*T) requests, chosen at random, stack 2 or 3 distinct adapters;
    every adapter drawn Zipf(1.1) over the pool."""
    z = ZipfAdapters(rng, n, 1.1)
    idx = np.full((T, K), -1, dtype=np.int32)
    stacked = set(int(s) for s in rng.choice(T, size=int(round(0.3 * T)), replace=False))
    for s in range(T):
        k = int(rng.integers(2, 4)) if s in stacked else 1
        idx[s, :k] = z.draw_distinct(rng, k)
    return Batch(T, T, K, None, idx, None)


def case_c2(seed: int = SEEDS["C2"], n: int = 1000) -> Case:
    rng = np.random.default_rng(seed)
    batch = batch_c2(rng, n)
    pool = make_pool(rng, BF16, n, 16, 4096, 4096)
    x, y = make_xy(rng, BF16, batch.T, 4096, 4096)
    return Case("C2", BF16, batch, pool, x, y)


def batch_c3(rng, S=32, n=8) -> Batch:
    """32 segments of U{128..1024} tokens, each on a uniformly drawn adapter."""
    lengths = rng.integers(128, 1025, size=S)
    idx = rng.integers(0, n, size=(S, 1)).astype(np.int32)
    return Batch(int(lengths.sum()), S, 1, offsets_from_lengths(lengths), idx, None)


def case_c3(seed: int = SEEDS["C3"]) -> Case:
    rng = np.random.default_rng(seed)
    n = 8
    batch = batch_c3(rng, 32, n)
    pool = make_pool(rng, BF16, n, 64, 4096, 4096)
    x, y = make_xy(rng, BF16, batch.T, 4096, 4096)
    return Case("C3", BF16, batch, pool, x, y)


def batch_c4(rng, n=256) -> Batch:
    """4 prefill segments of 512 tokens first, then 256 one-token decode requests;
    every request draws its adapter from Zipf(1.1) over the pool."""
    lengths = [512] * 4 + [1] * 256
    z = ZipfAdapters(rng, n, 1.1)
    idx = z.draw(rng, len(lengths)).reshape(-1, 1).astype(np.int32)
    return Batch(int(sum(lengths)), len(lengths), 1, offsets_from_lengths(lengths), idx, None)


def batch_c5(rng, n=200, S=16, L=4096, K=3) -> Batch:
    """16 requests x 4096 latent tokens; round(0.3*16)=5 requests, chosen at random,
    stack 2 or 3 distinct adapters; every adapter drawn Zipf(1.1) over the pool."""
    lengths = [L] * S
    z = ZipfAdapters(rng, n, 1.1)
    idx = np.full((S, K), -1, dtype=np.int32)
    stacked = set(int(s) for s in rng.choice(S, size=int(round(0.3 * S)), replace=False))
    for s in range(S):
        k = int(rng.integers(2, 4)) if s in stacked else 1
        idx[s, :k] = z.draw_distinct(rng, k)
    return Batch(int(sum(lengths)), S, K, offsets_from_lengths(lengths), idx, None)


def case_c5(d: int = 1280, r: int = 64, seed: int = SEEDS["C5"]) -> Case:
    rng = np.random.default_rng(seed)
    batch = batch_c5(rng)
    pool = make_pool(rng, BF16, 200, r, d, d)
    x, y = make_xy(rng, BF16, batch.T, d, d)
    return Case(f"C5_d{d}_r{r}", BF16, batch, pool, x, y)


# --------------------------------------------------------------------------
# general random cases for parity tests
# --------------------------------------------------------------------------
def random_batch(rng, *, T=None, S=8, K=1, n=4, min_len=0, max_len=16, per_token=False,
                 p_empty=0.15, with_scale=False, gaps=False, p_invalid=0.0) -> Batch:
    """A random heterogeneous batch.

    per_token: seg_off=None and S=T.  gaps: rows before seg_off[0] and after
    seg_off[S] belong to no request.  p_empty: probability that a slot is -1.
    p_invalid: probability that a slot holds an out-of-range index (the HIP
    path skips and counts these; the oracle refuses them)."""
    if per_token:
        T = S if T is None else T
        S = T
        seg_off = None
    else:
        lengths = rng.integers(min_len, max_len + 1, size=S)
        head = int(rng.integers(1, 5)) if gaps else 0
        tail = int(rng.integers(1, 5)) if gaps else 0
        seg_off = (offsets_from_lengths(lengths) + head).astype(np.int32)
        T_cov = int(seg_off[-1]) + tail
        T = T_cov if T is None else max(T, T_cov)
    idx = rng.integers(0, n, size=(S, K)).astype(np.int32)
    idx[rng.random((S, K)) < p_empty] = -1
    if p_invalid > 0:
        bad = rng.random((S, K)) < p_invalid
        nb = int(bad.sum())
        idx[bad] = np.where(rng.random(nb) < 0.5, n + rng.integers(0, 5, nb),
                            -2 - rng.integers(0, 5, nb)).astype(np.int32)
    scale = normal(rng, (S, K), 1.0) if with_scale else None
    return Batch(int(T), int(S), K, seg_off, idx, scale)


def random_case(seed, *, dtype=BF16, n=4, r=16, d_in=64, d_out=64, ldx=None, ldy=None,
                std_w=0.02, **batch_kw) -> Case:
    rng = np.random.default_rng(seed)
    batch = random_batch(rng, n=n, **batch_kw)
    pool = make_pool(rng, dtype, n, r, d_in, d_out, std_w)
    x, y = make_xy(rng, dtype, batch.T, d_in, d_out, ldx, ldy)
    return Case(f"rand{seed}", dtype, batch, pool, x, y)


# --------------------------------------------------------------------------
# structured probes (input construction only)
# --------------------------------------------------------------------------
def routing_probe(case: Case) -> Case:
    """x[t] = e_0, A_i[0][0] = 1 (all other A entries 0), B_i[o][0] = [o == i],
    y = 0.  The delta of row t is then the multi-hot vector of the adapters
    applied to it, exactly, in any precision.  Needs d_out >= n."""
    p = case.pool
    assert p.d_out >= p.n, "routing probe needs d_out >= n_adapters"
    one = encode(np.ones(1, np.float32), case.dtype)[0]
    A = np.zeros_like(p.A)
    A[:, 0, 0] = one
    B = np.zeros_like(p.B)
    ar = np.arange(p.n)
    B[ar, ar, 0] = one
    x = np.zeros_like(case.x)
    x[:, 0] = one
    y = np.zeros_like(case.y)
    pool = Pool(p.dtype, p.n, p.r, p.d_in, p.d_out, A, B)
    return Case(case.name + "_routing", case.dtype, case.batch, pool, x, y)


def integer_probe(seed, case: Case, nnz_per_row: int = 8) -> Case:
    """Small-integer inputs whose every partial sum is exact in fp32 and whose
    rank-r intermediate is exact in bf16: x in {-2..2}, each A row holds at most
    8 nonzeros in {-1, 1}, B in {-2..2}, y a small integer."""
    rng = np.random.default_rng(seed)
    p = case.pool
    A = np.zeros((p.n, p.r, p.d_in), np.float32)
    for i in range(p.n):
        for j in range(p.r):
            cols = rng.choice(p.d_in, size=min(nnz_per_row, p.d_in), replace=False)
            A[i, j, cols] = rng.choice([-1.0, 1.0], size=len(cols))
    B = rng.integers(-2, 3, size=(p.n, p.d_out, p.r)).astype(np.float32)
    x = rng.integers(-2, 3, size=case.x.shape).astype(np.float32)
    y = rng.integers(-64, 65, size=case.y.shape).astype(np.float32)
    pool = Pool(p.dtype, p.n, p.r, p.d_in, p.d_out, encode(A, case.dtype), encode(B, case.dtype))
    return Case(case.name + "_int", case.dtype, case.batch, pool, encode(x, case.dtype), encode(y, case.dtype))


def sentinel_rows(case: Case, rows: np.ndarray) -> Case:
    """Fill the given rows of y with sentinels that any write would disturb:
    -0.0 and NaNs with distinct payloads."""
    y = case.y.copy()
    if case.dtype == F32:
        u = y.view(np.uint32)
        for q, t in enumerate(rows):
            u[t, :] = np.where(np.arange(u.shape[1]) % 2 == 0, np.uint32(0x80000000),
                               np.uint32(0x7FC00000 | ((q * 131 + 7) & 0x3FFFFF)))
    else:
        for q, t in enumerate(rows):
            y[t, :] = np.where(np.arange(y.shape[1]) % 2 == 0, np.uint16(0x8000),
                               np.uint16(0x7FC0 | ((q * 13 + 1) & 0x3F)))
    return dataclasses.replace(case, y=y)
