"""CPU oracle for Dual-QK decode attention over a 2-bit KV cache.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``page_set_amd``) never imports it and shares no code with it.

Written from "Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV
Caches" (Whang, Oh, Kim, Seo).  The arithmetic lives in ``oracle.c`` (plain C,
``-ffp-contract=off``); this module only marshals numpy arrays.

Pins (tests/test_oracle_*.py, run without a GPU):

=====================  ==========================================================
function               pinned by
=====================  ==========================================================
f16 / bf16 rounding    the enumerated binary16 grid (numpy) and torch's bf16 cast
quantize_group         brute-force nearest level, [min,max] coverage, s/2 bound,
                       s^2/12 error statistics, hand-derived golden bytes
key_transform          fp64 matmul; dot-product invariance of §3.1 Eq. 1
pack_cache             golden page with hand-derived bytes; layout read back by an
                       independent numpy decoder; page-permutation invariance
select_channels        fp64 reference q T_Q within the fma-chain bound; full
                       sort; nestedness; g = 1 reduces to top-k |q'|
decode_attn            textbook softmax attention (numpy, fp64) on the decoded
                       cache with unselected channels zeroed; tiny brute force;
                       n_keep = 128 dense reduction; unquantized transform
                       identity; App. C.2 pruning-variance statistics
decode_bf16            textbook attention (numpy, fp64)
bytes (bytes.py)       the bits-per-element figures printed in Table 1
=====================  ==========================================================

Parity unpinned: the accuracy tables of the paper (need models and datasets).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

HEAD_DIM = 128
PAGE = 128

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        _lib.orc_f16_value.argtypes = [ctypes.c_uint16]
        _lib.orc_f16_value.restype = f64
        _lib.orc_f16_round_down.argtypes = [ctypes.c_float]
        _lib.orc_f16_round_down.restype = ctypes.c_uint16
        _lib.orc_f16_round_up.argtypes = [ctypes.c_float]
        _lib.orc_f16_round_up.restype = ctypes.c_uint16
        _lib.orc_bf16_round_nearest.argtypes = [ctypes.c_float]
        _lib.orc_bf16_round_nearest.restype = ctypes.c_uint16
        _lib.orc_quantize_group.argtypes = [P, i32, P, P, P]
        _lib.orc_quantize_group.restype = None
        _lib.orc_dequant.argtypes = [i32, ctypes.c_uint16, ctypes.c_uint16]
        _lib.orc_dequant.restype = ctypes.c_float
        _lib.orc_key_transform.argtypes = [P, P, i64, i32, P]
        _lib.orc_key_transform.restype = None
        _lib.orc_pack_cache.argtypes = [P, P, i32, i32, P, P, i32, P, P, P, P, P]
        _lib.orc_pack_cache.restype = None
        _lib.orc_select_channels.argtypes = [P, P, i32, i32, i32, i32, P, P]
        _lib.orc_select_channels.restype = i32
        _lib.orc_decode_attn.argtypes = [P, P, P, P, P, i32, P, P, i32, i32, i32, P, i32, P, f64, P, P]
        _lib.orc_decode_attn.restype = i32
        _lib.orc_decode_bf16.argtypes = [P, P, i32, P, i32, i32, P, i32, P, f64, P, P]
        _lib.orc_decode_bf16.restype = i32
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats
def f16_value(bits: int) -> float:
    return _load().orc_f16_value(int(bits))


def f16_round_down(x: float) -> int:
    return int(_load().orc_f16_round_down(float(x)))


def f16_round_up(x: float) -> int:
    return int(_load().orc_f16_round_up(float(x)))


def bf16_round_nearest(x: float) -> int:
    return int(_load().orc_bf16_round_nearest(float(x)))


# ---------------------------------------------------------------- quantizer
def quantize_group(x: np.ndarray):
    """(scale bits, zero bits, codes) of one group of fp32 values."""
    x = _c(x, np.float32)
    codes = np.zeros(x.size, dtype=np.uint8)
    s = ctypes.c_uint16()
    z = ctypes.c_uint16()
    _load().orc_quantize_group(_p(x), int(x.size), ctypes.byref(s), ctypes.byref(z), _p(codes))
    return int(s.value), int(z.value), codes


def dequant(code: int, s_bits: int, z_bits: int) -> float:
    return float(_load().orc_dequant(int(code), int(s_bits), int(z_bits)))


# ---------------------------------------------------------------- transform
def key_transform(k_bf16: np.ndarray, t_k_bf16: np.ndarray) -> np.ndarray:
    """k' = k T_K per token and KV head.  k [T][Hkv][128] bf16 bits -> fp32."""
    k = _c(k_bf16, np.uint16)
    tk = _c(t_k_bf16, np.uint16)
    T, hkv = k.shape[0], k.shape[1]
    out = np.empty((T, hkv, HEAD_DIM), dtype=np.float32)
    _load().orc_key_transform(_p(k), _p(tk), T, hkv, _p(out))
    return out


# ---------------------------------------------------------------- cache
class Cache:
    """Host copy of the paged INT2 cache (see oracle.c for the layout)."""

    def __init__(self, num_pages: int, hkv: int):
        self.num_pages, self.hkv = num_pages, hkv
        self.k_codes = np.zeros((num_pages, hkv, HEAD_DIM, 32), dtype=np.uint8)
        self.k_meta = np.zeros((num_pages, hkv, HEAD_DIM, 2), dtype=np.uint16)
        self.k_ch0 = np.zeros((num_pages, hkv, PAGE), dtype=np.uint16)
        self.v_codes = np.zeros((num_pages, hkv, PAGE, 32), dtype=np.uint8)
        self.v_meta = np.zeros((num_pages, hkv, 2, 4, PAGE), dtype=np.uint16)

    def arrays(self):
        return self.k_codes, self.k_meta, self.k_ch0, self.v_codes, self.v_meta


def pack_cache(kprime: np.ndarray, v_bf16: np.ndarray, cu_tokens, page_table, num_pages: int,
               cache: Optional[Cache] = None) -> Cache:
    kp = _c(kprime, np.float32)
    v = _c(v_bf16, np.uint16)
    cu = _c(cu_tokens, np.int32)
    pt = _c(page_table, np.int32)
    hkv = kp.shape[1]
    if cache is None:
        cache = Cache(num_pages, hkv)
    _load().orc_pack_cache(_p(kp), _p(v), hkv, len(cu) - 1, _p(cu), _p(pt), pt.shape[1],
                           *[_p(a) for a in cache.arrays()])
    return cache


def quantize_append(k_bf16, v_bf16, t_k_bf16, cu_tokens, page_table, num_pages: int,
                    cache: Optional[Cache] = None):
    """Transform keys with T_K and pack keys and values; returns (cache, k')."""
    kp = key_transform(k_bf16, t_k_bf16)
    return pack_cache(kp, v_bf16, cu_tokens, page_table, num_pages, cache), kp


# ---------------------------------------------------------------- decode
def select_channels(q_bf16, t_q, hkv: int, n_keep: int):
    q = _c(q_bf16, np.uint16)
    tq = _c(t_q, np.float32)
    B, hq = q.shape[0], q.shape[1]
    qp = np.empty((B, hq, HEAD_DIM), dtype=np.float32)
    sel = np.empty((B, hkv, n_keep), dtype=np.int32)
    rc = _load().orc_select_channels(_p(q), _p(tq), B, hq, hkv, n_keep, _p(qp), _p(sel))
    if rc:
        raise ValueError(f"select_channels: bad shape (rc={rc})")
    return qp, sel


def decode_attn(cache: Cache, q_prime, sel_idx, page_table, seq_lens, sm_scale: float):
    qp = _c(q_prime, np.float32)
    sel = _c(sel_idx, np.int32)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    B, hq = qp.shape[0], qp.shape[1]
    n_keep = sel.shape[2]
    out = np.empty((B, hq, HEAD_DIM), dtype=np.float64)
    lse = np.empty((B, hq), dtype=np.float64)
    rc = _load().orc_decode_attn(*[_p(a) for a in cache.arrays()], cache.hkv, _p(qp), _p(sel), n_keep, B, hq,
                                 _p(pt), pt.shape[1], _p(sl), float(sm_scale), _p(out), _p(lse))
    if rc:
        raise ValueError(f"decode_attn failed (rc={rc})")
    return out, lse


def decode_bf16(kb, vb, q_bf16, page_table, seq_lens, sm_scale: float):
    kb = _c(kb, np.uint16)
    vb = _c(vb, np.uint16)
    q = _c(q_bf16, np.uint16)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    B, hq = q.shape[0], q.shape[1]
    out = np.empty((B, hq, HEAD_DIM), dtype=np.float64)
    lse = np.empty((B, hq), dtype=np.float64)
    rc = _load().orc_decode_bf16(_p(kb), _p(vb), kb.shape[1], _p(q), B, hq, _p(pt), pt.shape[1], _p(sl),
                                 float(sm_scale), _p(out), _p(lse))
    if rc:
        raise ValueError(f"decode_bf16 failed (rc={rc})")
    return out, lse


def paged_bf16(k_bf16, v_bf16, cu_tokens, page_table, num_pages: int):
    """Lay raw bf16 K/V [T][Hkv][128] out in the baseline's paged layout
    [P][Hkv][128 tok][128 ch] (unused slots zero)."""
    hkv = k_bf16.shape[1]
    kb = np.zeros((num_pages, hkv, PAGE, HEAD_DIM), dtype=np.uint16)
    vb = np.zeros_like(kb)
    for b in range(len(cu_tokens) - 1):
        s, e = int(cu_tokens[b]), int(cu_tokens[b + 1])
        for pi in range((e - s + PAGE - 1) // PAGE):
            p = int(page_table[b, pi])
            t0, t1 = s + pi * PAGE, min(e, s + (pi + 1) * PAGE)
            kb[p, :, : t1 - t0, :] = np.transpose(k_bf16[t0:t1], (1, 0, 2))
            vb[p, :, : t1 - t0, :] = np.transpose(v_bf16[t0:t1], (1, 0, 2))
    return kb, vb
