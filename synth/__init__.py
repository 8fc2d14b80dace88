"""Seeded synthetic inputs for Dual-QK decode attention over an INT2 KV cache.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic (no transform application, quantization, selection or
attention).  Both the CPU oracle (``oracle/``) and the HIP path
(``page_set_amd``) consume exactly these buffers.

The workload shapes follow the throughput settings of "Dual-QK: Sharp Queries
and Flat Keys for Prunable 2-bit KV Caches" (§4.1 and §4.4: single-GPU decode
up to 128K context, GQA, head_dim 128).  The pages measure on real models and
benchmark suites that are not available here; seeded Gaussians stand in:

* q, k, v ~ N(0, 1), rounded to bf16 (round to nearest even).
* k gets 4 outlier channels per KV head (drawn from 1..127 without
  replacement) scaled by 10, and channel 0 offset by +3, before rounding.
* One transform pair per KV head (§3.1 fixes one pair per layer and KV
  head): T_K = bf16(R diag(u)) with R Haar-orthogonal (QR of a
  Gaussian, sign-fixed) and u ~ U[0.5, 2]; T_Q = (T_K as stored)^{-T}, computed
  in fp64 and rounded to fp32, so that (q T_Q)(k T_K)^T = q k^T (§3.1, Eq. 1).
* 128-token pages handed out in aligned blocks of eight; identity page table
  unless ``shuffle_pages`` (a seeded permutation of the blocks).
* Bucket-relative RoPE tables (§3.4, App. C.4): rotary frequencies
  base^(-i/64) stand in for a checkpoint's, with no random draws.

bf16 values are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

HEAD_DIM = 128
PAGE = 128

# stream identifiers for numpy SeedSequence spawning
_ID_Q, _ID_K, _ID_V, _ID_T, _ID_OUTLIER, _ID_LEN, _ID_PERM = 1, 2, 3, 4, 5, 6, 7
_ID_RV, _ID_D = 8, 9


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def n_keep_for_sparsity(sparsity: float, d: int = HEAD_DIM) -> int:
    """Channels kept at a given query-channel sparsity: never prune more than stated."""
    return d - int(math.floor(sparsity * d + 1e-9))


@dataclasses.dataclass
class Shape:
    batch: int
    hq: int
    hkv: int
    seq_lens: List[int]
    n_keep: int
    name: str = "custom"
    shuffle_pages: bool = False
    outliers: int = 4
    outlier_scale: float = 10.0
    ch0_offset: float = 3.0

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def max_pages(self) -> int:
        return max((L + PAGE - 1) // PAGE for L in self.seq_lens)

    @property
    def pages_per_seq(self) -> List[int]:
        return [(L + PAGE - 1) // PAGE for L in self.seq_lens]

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))


def log_uniform_lengths(n: int, lo: int, hi: int, seed: int) -> List[int]:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _ID_LEN])))
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return [int(min(hi, max(lo, math.floor(math.exp(x))))) for x in u]


def config_shape(cfg: int, seed: int = 0, sparsity: float = 0.4) -> Shape:
    """The five workloads of the decode-attention study (sizes only)."""
    nk = n_keep_for_sparsity(sparsity)
    if cfg == 0:
        return Shape(1, 8, 8, [4096], nk, name="tiny-mha-4k")
    if cfg == 1:
        return Shape(1, 32, 8, [32768], nk, name="gqa32x8-32k-b1")
    if cfg == 2:
        return Shape(16, 32, 8, [32768] * 16, nk, name="gqa32x8-32k-b16")
    if cfg == 3:
        return Shape(4, 32, 8, [131072] * 4, nk, name="gqa32x8-128k-b4")
    if cfg == 4:
        lens = log_uniform_lengths(32, 1024, 131072, seed)
        return Shape(32, 32, 8, lens, nk, name="gqa32x8-ragged-b32", shuffle_pages=True)
    raise ValueError(f"unknown config {cfg}")


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def make_transforms(hkv: int, seed: int):
    """T_K (bf16 bits, [hkv][128][128]) and T_Q (fp32, [hkv][128][128]).

    T[i][j]: i = input channel, j = output channel (row-vector convention)."""
    rng = _rng(seed, _ID_T)
    tk = np.empty((hkv, HEAD_DIM, HEAD_DIM), dtype=np.uint16)
    tq = np.empty((hkv, HEAD_DIM, HEAD_DIM), dtype=np.float32)
    for g in range(hkv):
        a = rng.standard_normal((HEAD_DIM, HEAD_DIM))
        qm, rm = np.linalg.qr(a)
        qm = qm * np.sign(np.diag(rm))[None, :]
        u = rng.uniform(0.5, 2.0, size=HEAD_DIM)
        tk[g] = f32_to_bf16_bits((qm * u[None, :]).astype(np.float32))
        tk64 = bf16_bits_to_f32(tk[g]).astype(np.float64)
        tq[g] = np.linalg.inv(tk64).T.astype(np.float32)
    return tk, tq


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def make_value_rotation(hkv: int, seed: int):
    """R_V (bf16 bits, [hkv][128][128]) and R_V^{-1} (fp32, [hkv][128][128]).

    Stands in for the calibrated value rotation composed with a Hadamard
    transform (§3.3 values paragraph, App. B.2): R_V = bf16(R H / sqrt(128))
    with R Haar-orthogonal; the inverse is that of the stored bf16 matrix,
    computed in fp64 and rounded to fp32 (the stored matrix is orthogonal
    only up to bf16 rounding)."""
    rng = _rng(seed, _ID_RV)
    hn = hadamard(HEAD_DIM) / math.sqrt(HEAD_DIM)
    rv = np.empty((hkv, HEAD_DIM, HEAD_DIM), dtype=np.uint16)
    rinv = np.empty((hkv, HEAD_DIM, HEAD_DIM), dtype=np.float32)
    for g in range(hkv):
        a = rng.standard_normal((HEAD_DIM, HEAD_DIM))
        qm, rm = np.linalg.qr(a)
        qm = qm * np.sign(np.diag(rm))[None, :]
        rv[g] = f32_to_bf16_bits((qm @ hn).astype(np.float32))
        rinv[g] = np.linalg.inv(bf16_bits_to_f32(rv[g]).astype(np.float64)).astype(np.float32)
    return rv, rinv


def make_selection_scales(hkv: int, seed: int) -> np.ndarray:
    """Per-channel selection weights 1/delta_j, fp32 [hkv][128].

    Stands in for the diagonal refinement D of §3.3 (A = A_0 D): delta_0 = 1,
    the other 127 entries log-uniform in [1/2, 2] and normalised to unit
    geometric mean (App. B.2)."""
    rng = _rng(seed, _ID_D)
    out = np.empty((hkv, HEAD_DIM), dtype=np.float32)
    for g in range(hkv):
        u = rng.uniform(math.log(0.5), math.log(2.0), size=HEAD_DIM - 1)
        u -= u.mean()
        delta = np.concatenate([[1.0], np.exp(u)])
        out[g] = (1.0 / delta).astype(np.float32)
    return out


ROPE_BUCKET = 2048


def rope_buckets(max_len: int) -> int:
    """Buckets of 2048 positions that cover max_len tokens (at least one)."""
    return max(1, -(-int(max_len) // ROPE_BUCKET))


def make_rope_tables(n_buckets: int, base: float = 10000.0):
    """Anchor tables of bucket-relative RoPE (§3.4, App. C.4), fp32 [n_buckets][64].

    Stands in for a checkpoint's rotary frequencies: theta_i = base^(-i/64)
    for the channel pair (i, i + 64), bucket k's anchor a_k = 2048 k, and the
    entries cos(a_k theta_i) and -sin(a_k theta_i) (the rotation back by the
    anchor), computed in fp64 and rounded to fp32.  No random draws."""
    i = np.arange(HEAD_DIM // 2, dtype=np.float64)
    theta = base ** (-i / (HEAD_DIM // 2))
    ang = (ROPE_BUCKET * np.arange(n_buckets, dtype=np.float64))[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), (-np.sin(ang)).astype(np.float32)


def outlier_channels(hkv: int, n: int, seed: int) -> np.ndarray:
    rng = _rng(seed, _ID_OUTLIER)
    out = np.zeros((hkv, n), dtype=np.int64)
    for g in range(hkv):
        out[g] = rng.choice(np.arange(1, HEAD_DIM), size=n, replace=False)
    return out


def make_q(shape: Shape, seed: int) -> np.ndarray:
    rng = _rng(seed, _ID_Q)
    x = rng.standard_normal((shape.batch, shape.hq, HEAD_DIM), dtype=np.float32)
    return f32_to_bf16_bits(x)


def make_kv_seq(shape: Shape, seed: int, b: int, outl: Optional[np.ndarray] = None):
    """bf16 K and V of sequence b: each [L_b][hkv][128]."""
    L = shape.seq_lens[b]
    rk = _rng(seed, _ID_K, b)
    rv = _rng(seed, _ID_V, b)
    k = rk.standard_normal((L, shape.hkv, HEAD_DIM), dtype=np.float32)
    v = rv.standard_normal((L, shape.hkv, HEAD_DIM), dtype=np.float32)
    if outl is None:
        outl = outlier_channels(shape.hkv, shape.outliers, seed)
    for g in range(shape.hkv):
        if shape.outliers:
            k[:, g, outl[g]] *= np.float32(shape.outlier_scale)
    k[:, :, 0] += np.float32(shape.ch0_offset)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def make_page_table(shape: Shape, seed: int):
    """int32 [batch][max_pages] page table (unused slots = -1) and pool size.

    The pool is handed out in aligned blocks of eight pages (the cache keeps
    the key rows of a block's eight pages side by side): sequence b gets
    ceil(pages_b / 8) blocks and its logical page i sits in slot i % 8 of its
    block i // 8.  ``shuffle_pages`` permutes the blocks of the pool."""
    K = 8
    pps = shape.pages_per_seq
    nblk = [(n + K - 1) // K for n in pps]
    total_blocks = int(sum(nblk))
    blocks = np.arange(total_blocks, dtype=np.int32)
    if shape.shuffle_pages:
        blocks = _rng(seed, _ID_PERM).permutation(total_blocks).astype(np.int32)
    pt = np.full((shape.batch, shape.max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pps):
        mine = blocks[off:off + nblk[b]]
        i = np.arange(n)
        pt[b, :n] = K * mine[i // K] + i % K
        off += nblk[b]
    return pt, K * total_blocks


@dataclasses.dataclass
class Problem:
    shape: Shape
    seed: int
    q: np.ndarray            # bf16 bits [B][Hq][128]
    t_k: np.ndarray          # bf16 bits [Hkv][128][128]
    t_q: np.ndarray          # fp32 [Hkv][128][128]
    page_table: np.ndarray   # int32 [B][max_pages]
    num_pages: int
    seq_lens: np.ndarray     # int32 [B]
    cu_tokens: np.ndarray    # int32 [B+1]
    outliers: np.ndarray     # int64 [Hkv][n]
    k: Optional[np.ndarray] = None  # bf16 bits [total_tokens][Hkv][128]
    v: Optional[np.ndarray] = None

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)

    def kv_seq(self, b: int):
        if self.k is not None:
            s, e = int(self.cu_tokens[b]), int(self.cu_tokens[b + 1])
            return self.k[s:e], self.v[s:e]
        return make_kv_seq(self.shape, self.seed, b, self.outliers)


def make_problem(shape: Shape, seed: int = 0, materialize_kv: bool = True) -> Problem:
    tk, tq = make_transforms(shape.hkv, seed)
    outl = outlier_channels(shape.hkv, shape.outliers, seed) if shape.outliers else np.zeros((shape.hkv, 0), np.int64)
    pt, total_pages = make_page_table(shape, seed)
    lens = np.asarray(shape.seq_lens, dtype=np.int32)
    cu = np.zeros(shape.batch + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    prob = Problem(shape, seed, make_q(shape, seed), tk, tq, pt, total_pages, lens, cu, outl)
    if materialize_kv:
        ks, vs = [], []
        for b in range(shape.batch):
            kb, vb = make_kv_seq(shape, seed, b, outl)
            ks.append(kb)
            vs.append(vb)
        prob.k = np.concatenate(ks, axis=0)
        prob.v = np.concatenate(vs, axis=0)
    return prob
