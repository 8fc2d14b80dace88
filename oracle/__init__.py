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
decode_bf16            attention computed from the raw unpaged bf16 keys and
                       values (numpy, fp64); 3-token pure-Python brute force;
                       scale 0 gives the value mean; page permutation and
                       tail-garbage invariance (tests/test_oracle_bf16.py)
paged_bf16             token t of sequence b lands at [page_table[b][t//128]][g]
                       [t%128], checked element by element
prefill_tiered         tier membership counted token by token; INT2 pages equal
                       pack_cache of the shifted token range; tier bytes equal
                       bf16(k') and v slot by slot (tests/test_oracle_tiers.py)
append_token           token-by-token appends from any length reproduce the
                       prefill of the final length byte for byte
decode_tiered          textbook attention (numpy, fp64) over the three token
                       sources decoded independently; all-BF16 sequences reduce
                       to attention on bf16 k', v; with every tier token moved
                       into pages it equals decode_attn on the same tokens
quantize_group_clip    clip 1 equals quantize_group; brute-force nearest level
                       of the clipped grid inside it, saturation outside; the
                       clipped range from the group extremes by hand
select_channels_base   unit scales equal select_channels; equals plain
                       selection with the base transform T_Q diag(sel_scale)
                       formed explicitly (fp64), up to near-ties
pack_cache_vrot        identity rotation and clip 1 equal pack_cache; a
                       within-group channel permutation as R_V permutes the
                       value codes of pack_cache exactly
value_unrotate         permutation R_V: rotate, pack, decode and unrotate give
                       decode_attn of the unrotated cache exactly; a Haar
                       rotation and its inverse return the input (fp64 bound)
                       (tests/test_oracle_vrot.py)
pack_cache_tokgrid     every token's codes are the nearest levels of its own
                       grid, which covers channels 1..127 tightly; channel 0
                       outside the range (changing it moves nothing else); the
                       layout read back by an independent numpy decoder
decode_attn_tokgrid    textbook attention (torch, fp64) over the cache decoded
                       by that reader; tiny brute force; with every token's
                       channels alike it equals decode_attn on a per-channel
                       pack of the same keys (tests/test_oracle_tokgrid.py)
key_transform_rope     identity tables equal key_transform exactly; with T_K = I
                       the rotation matches a complex fp64 rotation of each
                       channel pair (i, i + 64) within bf16 rounding; scores of
                       query and key rotated by one bucket's table equal the
                       unrotated ones (App. C.4); relative-position identity of
                       absolute RoPE (fp64)
select_channels_rope   identity tables give select_channels in every bucket;
                       each bucket equals select_channels of the query rotated
                       by an independent fp64 complex rotation (up to near-ties)
decode_attn_rope       textbook attention (torch, fp64) with each token scored
                       by its own bucket's masked query, one softmax over all;
                       equal buckets equal decode_attn exactly
                       (tests/test_oracle_rope.py)
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
        _lib.orc_bf16_round_array.argtypes = [P, i64, P]
        _lib.orc_bf16_round_array.restype = None
        f32 = ctypes.c_float
        _lib.orc_quantize_group_clip.argtypes = [P, i32, f32, P, P, P]
        _lib.orc_quantize_group_clip.restype = None
        _lib.orc_pack_cache_vrot.argtypes = [P, P, f32, i32, i32, P, P, i32, P, P, P, P, P]
        _lib.orc_pack_cache_vrot.restype = None
        _lib.orc_value_unrotate.argtypes = [P, P, i32, i32, i32, P]
        _lib.orc_value_unrotate.restype = i32
        _lib.orc_select_channels_base.argtypes = [P, P, P, i32, i32, i32, i32, P, P]
        _lib.orc_select_channels_base.restype = i32
        _lib.orc_pack_cache_tokgrid.argtypes = [P, P, i32, i32, P, P, i32, P, P, P, P, P]
        _lib.orc_pack_cache_tokgrid.restype = None
        _lib.orc_decode_attn_tokgrid.argtypes = [P, P, P, P, P, i32, P, P, i32, i32, i32, P, i32, P, f64, P, P]
        _lib.orc_decode_attn_tokgrid.restype = i32
        _lib.orc_key_transform_rope.argtypes = [P, P, i32, P, i32, P, P, P]
        _lib.orc_key_transform_rope.restype = None
        _lib.orc_select_channels_rope.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P, P]
        _lib.orc_select_channels_rope.restype = i32
        _lib.orc_decode_attn_rope.argtypes = [P, P, P, P, P, i32, P, P, i32, i32, i32, i32, P, i32, P, f64, P, P]
        _lib.orc_decode_attn_rope.restype = i32
        _lib.orc_tier_pages.argtypes = [i64]
        _lib.orc_tier_pages.restype = i64
        _lib.orc_decode_tiered.argtypes = [P, P, P, P, P, i32, P, P, P, P, P, P, i32, i32, i32, P, i32, P, f64, P,
                                           P]
        _lib.orc_decode_tiered.restype = i32
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


def quantize_group_clip(x: np.ndarray, clip: float):
    """quantize_group on the clipped range [clip * min, clip * max] (fp32 products)."""
    x = _c(x, np.float32)
    codes = np.zeros(x.size, dtype=np.uint8)
    s = ctypes.c_uint16()
    z = ctypes.c_uint16()
    _load().orc_quantize_group_clip(_p(x), int(x.size), float(clip), ctypes.byref(s), ctypes.byref(z), _p(codes))
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
    """Host copy of the paged INT2 cache (see oracle.c for the layout).

    Key rows and key metadata are stored in aligned blocks of eight pages, so
    the page pool holds a multiple of eight pages (rounded up here);
    ``k_rows(p)`` and ``k_meta_page(p)`` are writable views of one page."""

    BLOCK = 8

    def __init__(self, num_pages: int, hkv: int):
        K = self.BLOCK
        num_pages = -(-int(num_pages) // K) * K
        self.num_pages, self.hkv = num_pages, hkv
        nb = num_pages // K
        self.k_codes = np.zeros((nb, hkv, HEAD_DIM, K, 32), dtype=np.uint8)
        self.k_meta = np.zeros((nb, hkv, HEAD_DIM, K, 2), dtype=np.uint16)
        self.k_ch0 = np.zeros((num_pages, hkv, PAGE), dtype=np.uint16)
        self.v_codes = np.zeros((num_pages, hkv, PAGE, 32), dtype=np.uint8)
        self.v_meta = np.zeros((num_pages, hkv, 2, 4, PAGE), dtype=np.uint16)

    def arrays(self):
        return self.k_codes, self.k_meta, self.k_ch0, self.v_codes, self.v_meta

    def k_rows(self, p: int) -> np.ndarray:
        """[Hkv][128 ch][32] key rows of physical page p (a view)."""
        return self.k_codes[p // self.BLOCK, :, :, p % self.BLOCK]

    def k_meta_page(self, p: int) -> np.ndarray:
        """[Hkv][128 ch][2] key (scale, zero) of physical page p (a view)."""
        return self.k_meta[p // self.BLOCK, :, :, p % self.BLOCK]

    def page_major(self):
        """All five buffers indexed by physical page first:
        k_codes [P][Hkv][128][32], k_meta [P][Hkv][128][2], the rest as stored."""
        P = self.num_pages
        kc = np.ascontiguousarray(self.k_codes.transpose(0, 3, 1, 2, 4)).reshape(P, self.hkv, HEAD_DIM, 32)
        km = np.ascontiguousarray(self.k_meta.transpose(0, 3, 1, 2, 4)).reshape(P, self.hkv, HEAD_DIM, 2)
        return kc, km, self.k_ch0, self.v_codes, self.v_meta

    def set_page_major(self, kc, km, k0, vc, vm):
        K = self.BLOCK
        nb = self.num_pages // K
        self.k_codes[...] = kc.reshape(nb, K, self.hkv, HEAD_DIM, 32).transpose(0, 2, 3, 1, 4)
        self.k_meta[...] = km.reshape(nb, K, self.hkv, HEAD_DIM, 2).transpose(0, 2, 3, 1, 4)
        self.k_ch0[...], self.v_codes[...], self.v_meta[...] = k0, vc, vm


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


def pack_cache_tokgrid(kprime: np.ndarray, v_bf16: np.ndarray, cu_tokens, page_table, num_pages: int,
                       cache: Optional[Cache] = None) -> Cache:
    """pack_cache with one key grid per token and KV head over channels 1..127
    (per-token (scale, zero) pairs in k_meta, [P/8][Hkv][8][128][2])."""
    kp = _c(kprime, np.float32)
    v = _c(v_bf16, np.uint16)
    cu = _c(cu_tokens, np.int32)
    pt = _c(page_table, np.int32)
    hkv = kp.shape[1]
    if cache is None:
        cache = Cache(num_pages, hkv)
    _load().orc_pack_cache_tokgrid(_p(kp), _p(v), hkv, len(cu) - 1, _p(cu), _p(pt), pt.shape[1],
                                   *[_p(a) for a in cache.arrays()])
    return cache


def quantize_append_tokgrid(k_bf16, v_bf16, t_k_bf16, cu_tokens, page_table, num_pages: int,
                            cache: Optional[Cache] = None):
    """quantize_append with per-token key grids; returns (cache, k')."""
    kp = key_transform(k_bf16, t_k_bf16)
    return pack_cache_tokgrid(kp, v_bf16, cu_tokens, page_table, num_pages, cache), kp


def value_transform(v_bf16: np.ndarray, r_v_bf16: np.ndarray) -> np.ndarray:
    """v' = v R_V per token and KV head (the same row-vector product as k T_K)."""
    return key_transform(v_bf16, r_v_bf16)


def pack_cache_vrot(kprime: np.ndarray, vprime: np.ndarray, clip: float, cu_tokens, page_table, num_pages: int,
                    cache: Optional[Cache] = None) -> Cache:
    """pack_cache with fp32 rotated values and clipped value grids."""
    kp = _c(kprime, np.float32)
    vp = _c(vprime, np.float32)
    cu = _c(cu_tokens, np.int32)
    pt = _c(page_table, np.int32)
    hkv = kp.shape[1]
    if cache is None:
        cache = Cache(num_pages, hkv)
    _load().orc_pack_cache_vrot(_p(kp), _p(vp), float(clip), hkv, len(cu) - 1, _p(cu), _p(pt), pt.shape[1],
                                *[_p(a) for a in cache.arrays()])
    return cache


def quantize_append_vrot(k_bf16, v_bf16, t_k_bf16, r_v_bf16, clip: float, cu_tokens, page_table, num_pages: int,
                         cache: Optional[Cache] = None):
    """Keys as quantize_append; values rotated by R_V and clipped.  Returns (cache, k', v')."""
    kp = key_transform(k_bf16, t_k_bf16)
    vp = value_transform(v_bf16, r_v_bf16)
    return pack_cache_vrot(kp, vp, clip, cu_tokens, page_table, num_pages, cache), kp, vp


def value_unrotate(o, r_v_inv, hkv: int) -> np.ndarray:
    """out = o R_V^{-1} per query head (fp64 in, fp64 out)."""
    o = _c(o, np.float64)
    r = _c(r_v_inv, np.float32)
    B, hq = o.shape[0], o.shape[1]
    out = np.empty_like(o)
    rc = _load().orc_value_unrotate(_p(o), _p(r), B, hq, hkv, _p(out))
    if rc:
        raise ValueError(f"value_unrotate: bad shape (rc={rc})")
    return out


# ---------------------------------------------------------------- decode
def select_channels_base(q_bf16, t_q, sel_scale, hkv: int, n_keep: int):
    """select_channels ranking channels by the base-coordinate energy (q' * sel_scale)^2."""
    q = _c(q_bf16, np.uint16)
    tq = _c(t_q, np.float32)
    sc = _c(sel_scale, np.float32)
    B, hq = q.shape[0], q.shape[1]
    qp = np.empty((B, hq, HEAD_DIM), dtype=np.float32)
    sel = np.empty((B, hkv, n_keep), dtype=np.int32)
    rc = _load().orc_select_channels_base(_p(q), _p(tq), _p(sc), B, hq, hkv, n_keep, _p(qp), _p(sel))
    if rc:
        raise ValueError(f"select_channels_base: bad shape (rc={rc})")
    return qp, sel


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


def decode_attn_tokgrid(cache: Cache, q_prime, sel_idx, page_table, seq_lens, sm_scale: float):
    """decode_attn over a cache with per-token key grids."""
    qp = _c(q_prime, np.float32)
    sel = _c(sel_idx, np.int32)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    B, hq = qp.shape[0], qp.shape[1]
    out = np.empty((B, hq, HEAD_DIM), dtype=np.float64)
    lse = np.empty((B, hq), dtype=np.float64)
    rc = _load().orc_decode_attn_tokgrid(*[_p(a) for a in cache.arrays()], cache.hkv, _p(qp), _p(sel),
                                         sel.shape[2], B, hq, _p(pt), pt.shape[1], _p(sl), float(sm_scale),
                                         _p(out), _p(lse))
    if rc:
        raise ValueError(f"decode_attn_tokgrid failed (rc={rc})")
    return out, lse


# ---------------------------------------------------------------- bucket-relative RoPE
ROPE_BUCKET = 2048


def key_transform_rope(k_bf16, t_k_bf16, cu_tokens, rope_cos, rope_sin) -> np.ndarray:
    """k' = bf16(k rotated by its bucket's table) T_K: token t of sequence b
    (bucket (t - cu_tokens[b]) // 2048) uses rope_cos/rope_sin [n_buckets][64]."""
    k = _c(k_bf16, np.uint16)
    tk = _c(t_k_bf16, np.uint16)
    cu = _c(cu_tokens, np.int32)
    cs = _c(rope_cos, np.float32)
    sn = _c(rope_sin, np.float32)
    lens = np.diff(cu)
    if len(lens) and int(lens.max()) > cs.shape[0] * ROPE_BUCKET:
        raise ValueError("key_transform_rope: a sequence is longer than its bucket tables cover")
    T, hkv = k.shape[0], k.shape[1]
    out = np.empty((T, hkv, HEAD_DIM), dtype=np.float32)
    _load().orc_key_transform_rope(_p(k), _p(tk), len(cu) - 1, _p(cu), hkv, _p(cs), _p(sn), _p(out))
    return out


def quantize_append_rope(k_bf16, v_bf16, t_k_bf16, rope_cos, rope_sin, cu_tokens, page_table, num_pages: int,
                         cache: Optional[Cache] = None):
    """quantize_append with every key stored in its bucket frame; returns (cache, k')."""
    kp = key_transform_rope(k_bf16, t_k_bf16, cu_tokens, rope_cos, rope_sin)
    return pack_cache(kp, v_bf16, cu_tokens, page_table, num_pages, cache), kp


def select_channels_rope(q_bf16, t_q, rope_cos, rope_sin, hkv: int, n_keep: int):
    """Per-bucket selection: q' [B][n_buckets][Hq][128], sel [B][n_buckets][Hkv][n_keep]."""
    q = _c(q_bf16, np.uint16)
    tq = _c(t_q, np.float32)
    cs = _c(rope_cos, np.float32)
    sn = _c(rope_sin, np.float32)
    B, hq, nb = q.shape[0], q.shape[1], cs.shape[0]
    qp = np.empty((B, nb, hq, HEAD_DIM), dtype=np.float32)
    sel = np.empty((B, nb, hkv, n_keep), dtype=np.int32)
    rc = _load().orc_select_channels_rope(_p(q), _p(tq), _p(cs), _p(sn), nb, B, hq, hkv, n_keep, _p(qp), _p(sel))
    if rc:
        raise ValueError(f"select_channels_rope: bad shape (rc={rc})")
    return qp, sel


def decode_attn_rope(cache: Cache, q_prime, sel_idx, page_table, seq_lens, sm_scale: float):
    """decode_attn where token t scores with q_prime[b][t // 2048] and sel_idx[b][t // 2048]."""
    qp = _c(q_prime, np.float32)
    sel = _c(sel_idx, np.int32)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    B, nb, hq = qp.shape[0], qp.shape[1], qp.shape[2]
    out = np.empty((B, hq, HEAD_DIM), dtype=np.float64)
    lse = np.empty((B, hq), dtype=np.float64)
    rc = _load().orc_decode_attn_rope(*[_p(a) for a in cache.arrays()], cache.hkv, _p(qp), _p(sel), sel.shape[3],
                                      nb, B, hq, _p(pt), pt.shape[1], _p(sl), float(sm_scale), _p(out), _p(lse))
    if rc:
        raise ValueError(f"decode_attn_rope failed (rc={rc})")
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


# ---------------------------------------------------------------- BF16 tiers
# The first 64 and the most recent 256 tokens of a sequence stay in BF16 for
# keys and values (Dual-QK §3.3), scored under the same channel mask and in
# one softmax with the INT2 pages (§3.4).  Reading: tokens [0, 64) are the
# sink (slot t); INT2 page i holds tokens [64 + 128 i, 64 + 128 i + 128) and
# there are P = floor((L - 320) / 128) of them (0 below 320), so a page is
# packed once all its tokens are older than the 256 most recent; tokens
# [64 + 128 P, L) are the tail (256..383 of them once L >= 320), in slot
# (t - 64) mod 384.  Tier keys are the fp32 k' of key_transform rounded to
# bf16 (round to nearest even); tier values are the bf16 inputs; the tail
# also keeps the raw bf16 keys, from which its oldest page is packed.
SINK, RECENT, TAIL_SLOTS = 64, 256, 384


def tier_pages(L: int) -> int:
    """INT2 pages of a sequence of L tokens."""
    return int(_load().orc_tier_pages(int(L)))


class Tiers:
    """BF16 tiers of a batch: sink_k, sink_v [B][Hkv][64][128]; tail_k,
    tail_v, tail_kraw [B][Hkv][384][128]; all bf16 bits (uint16)."""

    def __init__(self, batch: int, hkv: int):
        self.batch, self.hkv = batch, hkv
        self.sink_k = np.zeros((batch, hkv, SINK, HEAD_DIM), np.uint16)
        self.sink_v = np.zeros_like(self.sink_k)
        self.tail_k = np.zeros((batch, hkv, TAIL_SLOTS, HEAD_DIM), np.uint16)
        self.tail_v = np.zeros_like(self.tail_k)
        self.tail_kraw = np.zeros_like(self.tail_k)

    def arrays(self):
        return self.sink_k, self.sink_v, self.tail_k, self.tail_v, self.tail_kraw


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (the oracle's scalar rule)."""
    flat = np.ascontiguousarray(x, np.float32).ravel()
    out = np.empty(flat.size, np.uint16)
    _load().orc_bf16_round_array(_p(flat), flat.size, _p(out))
    return out.reshape(np.shape(x))


def _put_tier_token(tiers: Tiers, b: int, t: int, kprime_t, k_t, v_t):
    """Token t of sequence b (k' fp32 [Hkv][128], raw k and v bf16 bits) into its tier slot."""
    kb = _bf16_bits(kprime_t)
    if t < SINK:
        tiers.sink_k[b, :, t] = kb
        tiers.sink_v[b, :, t] = v_t
    else:
        slot = (t - SINK) % TAIL_SLOTS
        tiers.tail_k[b, :, slot] = kb
        tiers.tail_v[b, :, slot] = v_t
        tiers.tail_kraw[b, :, slot] = k_t


def prefill_tiered(k_bf16, v_bf16, t_k_bf16, cu_tokens, page_table, num_pages: int):
    """Whole sequences into the tiered layout; returns (cache, tiers)."""
    k = _c(k_bf16, np.uint16)
    v = _c(v_bf16, np.uint16)
    cu = _c(cu_tokens, np.int32)
    pt = _c(page_table, np.int32)
    B, hkv = len(cu) - 1, k.shape[1]
    kp = key_transform(k, t_k_bf16)
    cache = Cache(num_pages, hkv)
    tiers = Tiers(B, hkv)
    ks, vs, cu2, rows = [], [], [0], []
    for b in range(B):
        t0, L = int(cu[b]), int(cu[b + 1] - cu[b])
        P = tier_pages(L)
        for t in list(range(min(L, SINK))) + list(range(SINK + PAGE * P, L)):
            _put_tier_token(tiers, b, t, kp[t0 + t], k[t0 + t], v[t0 + t])
        ks.append(kp[t0 + SINK:t0 + SINK + PAGE * P])
        vs.append(v[t0 + SINK:t0 + SINK + PAGE * P])
        cu2.append(cu2[-1] + PAGE * P)
        rows.append(pt[b])
    if cu2[-1] > 0:
        pack_cache(np.concatenate(ks), np.concatenate(vs), np.array(cu2, np.int32), np.stack(rows), num_pages,
                   cache)
    return cache, tiers


def append_token(cache: Cache, tiers: Tiers, k_new, v_new, t_k_bf16, seq_lens_before, page_table):
    """One new token per sequence (k_new, v_new bf16 [B][Hkv][128]) at position
    seq_lens_before[b]; when the new length completes a page's age, that page
    is packed from the tail's raw keys and values into page_table[b][i]."""
    k = _c(k_new, np.uint16)
    v = _c(v_new, np.uint16)
    pt = _c(page_table, np.int32)
    kp = key_transform(k, t_k_bf16)
    for b in range(k.shape[0]):
        t = int(seq_lens_before[b])
        _put_tier_token(tiers, b, t, kp[b], k[b], v[b])
        P0, P1 = tier_pages(t), tier_pages(t + 1)
        if P1 > P0:
            slots = [(PAGE * P0 + i) % TAIL_SLOTS for i in range(PAGE)]
            kr = np.ascontiguousarray(tiers.tail_kraw[b][:, slots].transpose(1, 0, 2))
            vr = np.ascontiguousarray(tiers.tail_v[b][:, slots].transpose(1, 0, 2))
            quantize_append(kr, vr, t_k_bf16, np.array([0, PAGE], np.int32), pt[b:b + 1, P0:P0 + 1],
                            cache.num_pages, cache)


def decode_tiered(cache: Cache, tiers: Tiers, q_prime, sel_idx, page_table, seq_lens, sm_scale: float):
    qp = _c(q_prime, np.float32)
    sel = _c(sel_idx, np.int32)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    B, hq = qp.shape[0], qp.shape[1]
    n_keep = sel.shape[2]
    out = np.empty((B, hq, HEAD_DIM), dtype=np.float64)
    lse = np.empty((B, hq), dtype=np.float64)
    ta = [_c(a, np.uint16) for a in (tiers.sink_k, tiers.sink_v, tiers.tail_k, tiers.tail_v)]
    rc = _load().orc_decode_tiered(*[_p(a) for a in cache.arrays()], cache.hkv, *[_p(a) for a in ta], _p(qp),
                                   _p(sel), n_keep, B, hq, _p(pt), pt.shape[1], _p(sl), float(sm_scale), _p(out),
                                   _p(lse))
    if rc:
        raise ValueError(f"decode_tiered failed (rc={rc})")
    return out, lse
