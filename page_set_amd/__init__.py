"""Python binding of libdqk (include/dqk.h): argument marshalling only.

Every step of the decode path runs in the HIP kernels of ``libdqk.so``; torch
is used for device memory and streams.  Importing this package does not need
a GPU, but every entry point raises if the library is missing: there is no
CPU fallback.

Names mirror the C ABI.  Tensors are torch CUDA (HIP) tensors; bf16 data may be
passed as ``torch.bfloat16`` or as ``torch.int16``/``torch.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdqk.so")
HEAD_DIM = 128
PAGE = 128

DQK_OK, DQK_ERR_NULL, DQK_ERR_SHAPE, DQK_ERR_ALIGN = 0, -1, -2, -3
DQK_ERR_UNSUPPORTED, DQK_ERR_WORKSPACE, DQK_ERR_HIP = -4, -5, -6

_lib = None


class DqkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().dqk_status_string(status).decode()
        if status == DQK_ERR_HIP:
            msg += f" (hipError {lib().dqk_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


class dqk_cache(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("k_codes", ctypes.c_void_p), ("k_meta", ctypes.c_void_p), ("k_ch0", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_meta", ctypes.c_void_p)]


class dqk_tiers(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("sink_k", ctypes.c_void_p), ("sink_v", ctypes.c_void_p), ("tail_k", ctypes.c_void_p),
                ("tail_v", ctypes.c_void_p), ("tail_kraw", ctypes.c_void_p)]


TIER_SINK, TIER_RECENT, TIER_TAIL_SLOTS = 64, 256, 384


def lib():
    """The loaded libdqk (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libdqk.so not found at {LIB_PATH}; build it with page_set_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.dqk_status_string.argtypes = [ctypes.c_int]
        L.dqk_status_string.restype = ctypes.c_char_p
        L.dqk_last_hip_error.argtypes = []
        L.dqk_last_hip_error.restype = ctypes.c_int
        L.dqk_quantize_append.argtypes = [ctypes.POINTER(dqk_cache), P, P, P, i32, P, i64, P, i32, P, P]
        L.dqk_quantize_append.restype = ctypes.c_int
        L.dqk_select_channels.argtypes = [P, P, i32, i32, i32, i32, P, P, P]
        L.dqk_select_channels.restype = ctypes.c_int
        L.dqk_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.dqk_decode_workspace_size.restype = sz
        L.dqk_decode_attn.argtypes = [ctypes.POINTER(dqk_cache), P, P, i32, i32, i32, P, i32, P, ctypes.c_float, i32,
                                      P, sz, P, P, P]
        L.dqk_decode_attn.restype = ctypes.c_int
        L.dqk_select_decode_attn.argtypes = [ctypes.POINTER(dqk_cache), P, P, i32, i32, i32, P, i32, P,
                                             ctypes.c_float, i32, P, sz, P, P, P, P, P]
        L.dqk_select_decode_attn.restype = ctypes.c_int
        L.dqk_select_decode_attn_vrot.argtypes = [ctypes.POINTER(dqk_cache), P, P, P, P, i32, i32, i32, P, i32, P,
                                                  ctypes.c_float, i32, P, sz, P, P, P, P, P]
        L.dqk_select_decode_attn_vrot.restype = ctypes.c_int
        L.dqk_decode_attn_noalloc.argtypes = [ctypes.POINTER(dqk_cache), P, P, i32, i32, i32, P, i32, P,
                                              ctypes.c_float, i32, P, P, P]
        L.dqk_decode_attn_noalloc.restype = ctypes.c_int
        L.dqk_decode_noalloc_max_bytes.argtypes = []
        L.dqk_decode_noalloc_max_bytes.restype = sz
        L.dqk_decode_attn_bf16.argtypes = [P, P, i32, i32, P, i32, i32, P, i32, P, ctypes.c_float, i32, P, sz, P, P,
                                           P]
        L.dqk_decode_attn_bf16.restype = ctypes.c_int
        T = ctypes.POINTER(dqk_tiers)
        L.dqk_prefill_tiered.argtypes = [ctypes.POINTER(dqk_cache), T, P, P, P, i32, P, i64, P, i32, P]
        L.dqk_prefill_tiered.restype = ctypes.c_int
        L.dqk_append_token.argtypes = [ctypes.POINTER(dqk_cache), T, P, P, P, i32, P, P, i32, P]
        L.dqk_append_token.restype = ctypes.c_int
        L.dqk_decode_tiered_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.dqk_decode_tiered_workspace_size.restype = sz
        L.dqk_decode_attn_tiered.argtypes = [ctypes.POINTER(dqk_cache), T, P, P, i32, i32, i32, P, i32, P,
                                             ctypes.c_float, i32, P, sz, P, P, P]
        L.dqk_decode_attn_tiered.restype = ctypes.c_int
        L.dqk_select_decode_attn_tiered.argtypes = [ctypes.POINTER(dqk_cache), T, P, P, i32, i32, i32, P, i32, P,
                                                    ctypes.c_float, i32, P, sz, P, P, P, P, P]
        L.dqk_select_decode_attn_tiered.restype = ctypes.c_int
        L.dqk_quantize_append_vrot.argtypes = [ctypes.POINTER(dqk_cache), P, P, P, P, ctypes.c_float, i32, P, i64,
                                               P, i32, P, P, P]
        L.dqk_quantize_append_vrot.restype = ctypes.c_int
        L.dqk_select_channels_base.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P]
        L.dqk_select_channels_base.restype = ctypes.c_int
        L.dqk_value_unrotate.argtypes = [P, P, i32, i32, i32, P, P]
        L.dqk_value_unrotate.restype = ctypes.c_int
        L.dqk_quantize_append_tokgrid.argtypes = [ctypes.POINTER(dqk_cache), P, P, P, i32, P, i64, P, i32, P, P]
        L.dqk_quantize_append_tokgrid.restype = ctypes.c_int
        L.dqk_decode_attn_tokgrid.argtypes = [ctypes.POINTER(dqk_cache), P, P, i32, i32, i32, P, i32, P,
                                              ctypes.c_float, i32, P, sz, P, P, P]
        L.dqk_decode_attn_tokgrid.restype = ctypes.c_int
        L.dqk_select_decode_attn_tokgrid.argtypes = [ctypes.POINTER(dqk_cache), P, P, i32, i32, i32, P, i32, P,
                                                     ctypes.c_float, i32, P, sz, P, P, P, P, P]
        L.dqk_select_decode_attn_tokgrid.restype = ctypes.c_int
        L.dqk_quantize_append_rope.argtypes = [ctypes.POINTER(dqk_cache), P, P, P, P, P, i32, i32, P, i64, P, i32,
                                               P, P]
        L.dqk_quantize_append_rope.restype = ctypes.c_int
        L.dqk_select_channels_rope.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P, P, P]
        L.dqk_select_channels_rope.restype = ctypes.c_int
        L.dqk_decode_rope_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.dqk_decode_rope_workspace_size.restype = sz
        L.dqk_decode_attn_rope.argtypes = [ctypes.POINTER(dqk_cache), P, P, i32, i32, i32, i32, P, i32, P,
                                           ctypes.c_float, i32, P, sz, P, P, P]
        L.dqk_decode_attn_rope.restype = ctypes.c_int
        L.dqk_select_decode_attn_rope.argtypes = [ctypes.POINTER(dqk_cache), P, P, P, P, i32, i32, i32, i32, P, i32,
                                                  P, ctypes.c_float, i32, P, sz, P, P, P, P, P]
        L.dqk_select_decode_attn_rope.restype = ctypes.c_int
        L.dqk_stream_read.argtypes = [P, sz, P, P]
        L.dqk_stream_read.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int, where: str):
    if rc != DQK_OK:
        raise DqkError(rc, where)


class Cache:
    """Device buffers of the paged INT2 cache (layout in include/dqk.h).  The
    page pool is a whole number of aligned 8-page blocks (rounded up here)."""

    BLOCK = 8

    def __init__(self, num_pages: int, num_kv_heads: int, device="cuda"):
        import torch
        K = self.BLOCK
        self.num_pages, self.num_kv_heads = -(-int(num_pages) // K) * K, int(num_kv_heads)
        P, H = self.num_pages, self.num_kv_heads
        self.k_codes = torch.zeros((P // K, H, HEAD_DIM, K, 32), dtype=torch.uint8, device=device)
        self.k_meta = torch.zeros((P // K, H, HEAD_DIM, K, 2), dtype=torch.int16, device=device)
        self.k_ch0 = torch.zeros((P, H, PAGE), dtype=torch.int16, device=device)
        self.v_codes = torch.zeros((P, H, PAGE, 32), dtype=torch.uint8, device=device)
        self.v_meta = torch.zeros((P, H, 2, 4, PAGE), dtype=torch.int16, device=device)

    def arrays(self):
        return self.k_codes, self.k_meta, self.k_ch0, self.v_codes, self.v_meta

    def struct(self) -> dqk_cache:
        return dqk_cache(self.num_kv_heads, self.num_pages, *[a.data_ptr() for a in self.arrays()])

    def nbytes(self) -> int:
        return sum(a.numel() * a.element_size() for a in self.arrays())

    def page_major(self):
        """Copies of the five buffers indexed by physical page first (key rows
        [P][Hkv][128][32], key metadata [P][Hkv][128][2]); for tests."""
        P, H = self.num_pages, self.num_kv_heads
        kc = self.k_codes.permute(0, 3, 1, 2, 4).reshape(P, H, HEAD_DIM, 32)
        km = self.k_meta.permute(0, 3, 1, 2, 4).reshape(P, H, HEAD_DIM, 2)
        return kc, km, self.k_ch0, self.v_codes, self.v_meta


class Tiers:
    """Device buffers of the BF16 tiers (layout in include/dqk.h):
    sink_k, sink_v [B][Hkv][64][128]; tail_k, tail_v, tail_kraw [B][Hkv][384][128]; bf16 bits."""

    def __init__(self, batch: int, num_kv_heads: int, device="cuda"):
        import torch
        self.batch, self.num_kv_heads = int(batch), int(num_kv_heads)
        B, H = self.batch, self.num_kv_heads
        self.sink_k = torch.zeros((B, H, TIER_SINK, HEAD_DIM), dtype=torch.int16, device=device)
        self.sink_v = torch.zeros_like(self.sink_k)
        self.tail_k = torch.zeros((B, H, TIER_TAIL_SLOTS, HEAD_DIM), dtype=torch.int16, device=device)
        self.tail_v = torch.zeros_like(self.tail_k)
        self.tail_kraw = torch.zeros_like(self.tail_k)

    def arrays(self):
        return self.sink_k, self.sink_v, self.tail_k, self.tail_v, self.tail_kraw

    def struct(self) -> dqk_tiers:
        return dqk_tiers(self.batch, self.num_kv_heads, *[a.data_ptr() for a in self.arrays()])


def dqk_prefill_tiered(cache: Cache, tiers: Tiers, k, v, t_k, cu_tokens, page_table, stream=None):
    n_seqs = cu_tokens.numel() - 1
    s, t = cache.struct(), tiers.struct()
    rc = lib().dqk_prefill_tiered(ctypes.byref(s), ctypes.byref(t), _ptr(k), _ptr(v), _ptr(t_k), n_seqs,
                                  _ptr(cu_tokens), int(k.shape[0]), _ptr(page_table), int(page_table.shape[1]),
                                  _stream(stream))
    _check(rc, "dqk_prefill_tiered")


def dqk_append_token(cache: Cache, tiers: Tiers, k_new, v_new, t_k, lens_before, page_table, stream=None):
    s, t = cache.struct(), tiers.struct()
    rc = lib().dqk_append_token(ctypes.byref(s), ctypes.byref(t), _ptr(k_new), _ptr(v_new), _ptr(t_k),
                                int(k_new.shape[0]), _ptr(lens_before), _ptr(page_table), int(page_table.shape[1]),
                                _stream(stream))
    _check(rc, "dqk_append_token")


def dqk_decode_tiered_workspace_size(batch: int, hq: int, hkv: int, max_pages: int, num_splits: int = 0) -> int:
    return int(lib().dqk_decode_tiered_workspace_size(batch, hq, hkv, max_pages, num_splits))


def dqk_decode_attn_tiered(cache: Cache, tiers: Tiers, q_prime, sel_idx, page_table, seq_lens, sm_scale: float,
                           num_splits: int = 0, workspace=None, out=None, lse=None, want_lse: bool = True,
                           stream=None):
    import torch
    B, hq = int(q_prime.shape[0]), int(q_prime.shape[1])
    n_keep = int(sel_idx.shape[2])
    max_pages = int(page_table.shape[1])
    dev = q_prime.device
    if workspace is None:
        n = dqk_decode_tiered_workspace_size(B, hq, cache.num_kv_heads, max_pages, num_splits)
        workspace = torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    s, t = cache.struct(), tiers.struct()
    rc = lib().dqk_decode_attn_tiered(ctypes.byref(s), ctypes.byref(t), _ptr(q_prime), _ptr(sel_idx), n_keep, B, hq,
                                      _ptr(page_table), max_pages, _ptr(seq_lens), float(sm_scale), int(num_splits),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                                      _ptr(lse), _stream(stream))
    _check(rc, "dqk_decode_attn_tiered")
    return out, lse


def dqk_select_decode_attn_tiered(cache: Cache, tiers: Tiers, q, t_q, n_keep: int, page_table, seq_lens,
                                  sm_scale: float, num_splits: int = 0, workspace=None, out=None, lse=None,
                                  want_lse: bool = True, q_prime=None, sel_idx=None, stream=None):
    """Selection and tiered decode in one call; returns (out, lse, q_prime, sel_idx)."""
    import torch
    B, hq = int(q.shape[0]), int(q.shape[1])
    hkv = cache.num_kv_heads
    max_pages = int(page_table.shape[1])
    dev = q.device
    if workspace is None:
        n = dqk_decode_tiered_workspace_size(B, hq, hkv, max_pages, num_splits)
        workspace = torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    if q_prime is None:
        q_prime = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty((B, hkv, n_keep), dtype=torch.int32, device=dev)
    s, t = cache.struct(), tiers.struct()
    rc = lib().dqk_select_decode_attn_tiered(ctypes.byref(s), ctypes.byref(t), _ptr(q), _ptr(t_q), int(n_keep), B,
                                             hq, _ptr(page_table), max_pages, _ptr(seq_lens), float(sm_scale),
                                             int(num_splits), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                                             _ptr(q_prime), _ptr(sel_idx), _stream(stream))
    _check(rc, "dqk_select_decode_attn_tiered")
    return out, lse, q_prime, sel_idx


def dqk_quantize_append(cache: Cache, k, v, t_k, cu_tokens, page_table, kprime_dbg=None, stream=None):
    n_seqs = cu_tokens.numel() - 1
    s = cache.struct()
    rc = lib().dqk_quantize_append(ctypes.byref(s), _ptr(k), _ptr(v), _ptr(t_k), n_seqs, _ptr(cu_tokens),
                                   int(k.shape[0]), _ptr(page_table), int(page_table.shape[1]), _ptr(kprime_dbg),
                                   _stream(stream))
    _check(rc, "dqk_quantize_append")


def dqk_quantize_append_tokgrid(cache: Cache, k, v, t_k, cu_tokens, page_table, kprime_dbg=None, stream=None):
    n_seqs = cu_tokens.numel() - 1
    s = cache.struct()
    rc = lib().dqk_quantize_append_tokgrid(ctypes.byref(s), _ptr(k), _ptr(v), _ptr(t_k), n_seqs, _ptr(cu_tokens),
                                           int(k.shape[0]), _ptr(page_table), int(page_table.shape[1]),
                                           _ptr(kprime_dbg), _stream(stream))
    _check(rc, "dqk_quantize_append_tokgrid")


def dqk_select_channels(q, t_q, hkv: int, n_keep: int, q_prime=None, sel_idx=None, stream=None):
    import torch
    B, hq = int(q.shape[0]), int(q.shape[1])
    if q_prime is None:
        q_prime = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if sel_idx is None:
        sel_idx = torch.empty((B, hkv, n_keep), dtype=torch.int32, device=q.device)
    rc = lib().dqk_select_channels(_ptr(q), _ptr(t_q), B, hq, hkv, n_keep, _ptr(q_prime), _ptr(sel_idx),
                                   _stream(stream))
    _check(rc, "dqk_select_channels")
    return q_prime, sel_idx


def dqk_quantize_append_vrot(cache: Cache, k, v, t_k, r_v, clip: float, cu_tokens, page_table, kprime_dbg=None,
                             vprime_dbg=None, stream=None):
    n_seqs = cu_tokens.numel() - 1
    s = cache.struct()
    rc = lib().dqk_quantize_append_vrot(ctypes.byref(s), _ptr(k), _ptr(v), _ptr(t_k), _ptr(r_v), float(clip), n_seqs,
                                        _ptr(cu_tokens), int(k.shape[0]), _ptr(page_table), int(page_table.shape[1]),
                                        _ptr(kprime_dbg), _ptr(vprime_dbg), _stream(stream))
    _check(rc, "dqk_quantize_append_vrot")


def dqk_select_channels_base(q, t_q, sel_scale, hkv: int, n_keep: int, q_prime=None, sel_idx=None, stream=None):
    import torch
    B, hq = int(q.shape[0]), int(q.shape[1])
    if q_prime is None:
        q_prime = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if sel_idx is None:
        sel_idx = torch.empty((B, hkv, n_keep), dtype=torch.int32, device=q.device)
    rc = lib().dqk_select_channels_base(_ptr(q), _ptr(t_q), _ptr(sel_scale), B, hq, hkv, n_keep, _ptr(q_prime),
                                        _ptr(sel_idx), _stream(stream))
    _check(rc, "dqk_select_channels_base")
    return q_prime, sel_idx


def dqk_value_unrotate(o_rot, r_v_inv, hkv: int, out=None, stream=None):
    """out = o_rot R_V^-1 per query head (out must not overlap o_rot); returns out."""
    import torch
    B, hq = int(o_rot.shape[0]), int(o_rot.shape[1])
    if out is None:
        out = torch.empty_like(o_rot)
    rc = lib().dqk_value_unrotate(_ptr(o_rot), _ptr(r_v_inv), B, hq, hkv, _ptr(out), _stream(stream))
    _check(rc, "dqk_value_unrotate")
    return out


def dqk_decode_workspace_size(batch: int, hq: int, hkv: int, max_pages: int, num_splits: int = 0) -> int:
    return int(lib().dqk_decode_workspace_size(batch, hq, hkv, max_pages, num_splits))


def _workspace(batch, hq, hkv, max_pages, num_splits, device):
    import torch
    n = dqk_decode_workspace_size(batch, hq, hkv, max_pages, num_splits)
    return torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device=device)


def dqk_decode_attn(cache: Cache, q_prime, sel_idx, page_table, seq_lens, sm_scale: float, num_splits: int = 0,
                    workspace=None, out=None, lse=None, want_lse: bool = True, stream=None, token_grid: bool = False):
    """Decode over the INT2 cache; token_grid: the cache was written by
    dqk_quantize_append_tokgrid (calls dqk_decode_attn_tokgrid)."""
    import torch
    B, hq = int(q_prime.shape[0]), int(q_prime.shape[1])
    n_keep = int(sel_idx.shape[2])
    max_pages = int(page_table.shape[1])
    dev = q_prime.device
    if workspace is None:
        workspace = _workspace(B, hq, cache.num_kv_heads, max_pages, num_splits, dev)
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    s = cache.struct()
    name = "dqk_decode_attn_tokgrid" if token_grid else "dqk_decode_attn"
    rc = getattr(lib(), name)(ctypes.byref(s), _ptr(q_prime), _ptr(sel_idx), n_keep, B, hq, _ptr(page_table),
                              max_pages, _ptr(seq_lens), float(sm_scale), int(num_splits), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream))
    _check(rc, name)
    return out, lse


def dqk_select_decode_attn(cache: Cache, q, t_q, n_keep: int, page_table, seq_lens, sm_scale: float,
                           num_splits: int = 0, workspace=None, out=None, lse=None, want_lse: bool = True,
                           q_prime=None, sel_idx=None, stream=None, token_grid: bool = False):
    """Selection and decode in one call; returns (out, lse, q_prime, sel_idx).
    token_grid: the cache holds per-token key grids."""
    import torch
    B, hq = int(q.shape[0]), int(q.shape[1])
    hkv = cache.num_kv_heads
    max_pages = int(page_table.shape[1])
    dev = q.device
    if workspace is None:
        workspace = _workspace(B, hq, hkv, max_pages, num_splits, dev)
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    if q_prime is None:
        q_prime = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty((B, hkv, n_keep), dtype=torch.int32, device=dev)
    s = cache.struct()
    name = "dqk_select_decode_attn_tokgrid" if token_grid else "dqk_select_decode_attn"
    rc = getattr(lib(), name)(ctypes.byref(s), _ptr(q), _ptr(t_q), int(n_keep), B, hq, _ptr(page_table),
                              max_pages, _ptr(seq_lens), float(sm_scale), int(num_splits), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                              _ptr(q_prime), _ptr(sel_idx), _stream(stream))
    _check(rc, name)
    return out, lse, q_prime, sel_idx


def dqk_select_decode_attn_vrot(cache: Cache, q, t_q, sel_scale, r_v_inv, n_keep: int, page_table, seq_lens,
                                sm_scale: float, num_splits: int = 0, workspace=None, out=None, lse=None,
                                want_lse: bool = True, q_prime=None, sel_idx=None, stream=None):
    """Base selection, decode and merge with the inverse value rotation in one
    call; returns (out, lse, q_prime, sel_idx)."""
    import torch
    B, hq = int(q.shape[0]), int(q.shape[1])
    hkv = cache.num_kv_heads
    max_pages = int(page_table.shape[1])
    dev = q.device
    if workspace is None:
        workspace = _workspace(B, hq, hkv, max_pages, num_splits, dev)
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    if q_prime is None:
        q_prime = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty((B, hkv, n_keep), dtype=torch.int32, device=dev)
    s = cache.struct()
    rc = lib().dqk_select_decode_attn_vrot(ctypes.byref(s), _ptr(q), _ptr(t_q), _ptr(sel_scale), _ptr(r_v_inv),
                                           int(n_keep), B, hq, _ptr(page_table), max_pages, _ptr(seq_lens),
                                           float(sm_scale), int(num_splits), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                                           _ptr(q_prime), _ptr(sel_idx), _stream(stream))
    _check(rc, "dqk_select_decode_attn_vrot")
    return out, lse, q_prime, sel_idx


# ---- bucket-relative RoPE: tables rope_cos / rope_sin fp32 [n_buckets][64]
def dqk_quantize_append_rope(cache: Cache, k, v, t_k, rope_cos, rope_sin, cu_tokens, page_table, kprime_dbg=None,
                             stream=None):
    n_seqs = cu_tokens.numel() - 1
    s = cache.struct()
    rc = lib().dqk_quantize_append_rope(ctypes.byref(s), _ptr(k), _ptr(v), _ptr(t_k), _ptr(rope_cos), _ptr(rope_sin),
                                        int(rope_cos.shape[0]), n_seqs, _ptr(cu_tokens), int(k.shape[0]),
                                        _ptr(page_table), int(page_table.shape[1]), _ptr(kprime_dbg),
                                        _stream(stream))
    _check(rc, "dqk_quantize_append_rope")


def dqk_select_channels_rope(q, t_q, rope_cos, rope_sin, hkv: int, n_keep: int, q_prime=None, sel_idx=None,
                             stream=None):
    """Per-bucket selection; returns q_prime [B][n_buckets][Hq][128], sel_idx [B][n_buckets][Hkv][n_keep]."""
    import torch
    B, hq, nb = int(q.shape[0]), int(q.shape[1]), int(rope_cos.shape[0])
    if q_prime is None:
        q_prime = torch.empty((B, nb, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if sel_idx is None:
        sel_idx = torch.empty((B, nb, hkv, n_keep), dtype=torch.int32, device=q.device)
    rc = lib().dqk_select_channels_rope(_ptr(q), _ptr(t_q), _ptr(rope_cos), _ptr(rope_sin), nb, B, hq, hkv, n_keep,
                                        _ptr(q_prime), _ptr(sel_idx), _stream(stream))
    _check(rc, "dqk_select_channels_rope")
    return q_prime, sel_idx


def dqk_decode_rope_workspace_size(batch: int, hq: int, hkv: int, n_buckets: int, num_splits: int = 0) -> int:
    return int(lib().dqk_decode_rope_workspace_size(batch, hq, hkv, n_buckets, num_splits))


def _rope_outputs(B, hq, nb, hkv, num_splits, want_lse, workspace, out, lse, dev):
    import torch
    if workspace is None:
        n = dqk_decode_rope_workspace_size(B, hq, hkv, nb, num_splits)
        workspace = torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    return workspace, out, lse


def dqk_decode_attn_rope(cache: Cache, q_prime, sel_idx, page_table, seq_lens, sm_scale: float, num_splits: int = 0,
                         workspace=None, out=None, lse=None, want_lse: bool = True, stream=None):
    """Decode over a cache written by dqk_quantize_append_rope, with
    q_prime / sel_idx as dqk_select_channels_rope returns them."""
    B, nb, hq = int(q_prime.shape[0]), int(q_prime.shape[1]), int(q_prime.shape[2])
    n_keep = int(sel_idx.shape[3])
    workspace, out, lse = _rope_outputs(B, hq, nb, cache.num_kv_heads, num_splits, want_lse, workspace, out, lse,
                                        q_prime.device)
    s = cache.struct()
    rc = lib().dqk_decode_attn_rope(ctypes.byref(s), _ptr(q_prime), _ptr(sel_idx), n_keep, nb, B, hq,
                                    _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens), float(sm_scale),
                                    int(num_splits), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _ptr(out), _ptr(lse), _stream(stream))
    _check(rc, "dqk_decode_attn_rope")
    return out, lse


def dqk_select_decode_attn_rope(cache: Cache, q, t_q, rope_cos, rope_sin, n_keep: int, page_table, seq_lens,
                                sm_scale: float, num_splits: int = 0, workspace=None, out=None, lse=None,
                                want_lse: bool = True, q_prime=None, sel_idx=None, stream=None):
    """Per-bucket selection, decode and bucket merge in one call; returns
    (out, lse, q_prime, sel_idx)."""
    import torch
    B, hq, nb = int(q.shape[0]), int(q.shape[1]), int(rope_cos.shape[0])
    hkv = cache.num_kv_heads
    dev = q.device
    workspace, out, lse = _rope_outputs(B, hq, nb, hkv, num_splits, want_lse, workspace, out, lse, dev)
    if q_prime is None:
        q_prime = torch.empty((B, nb, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty((B, nb, hkv, n_keep), dtype=torch.int32, device=dev)
    s = cache.struct()
    rc = lib().dqk_select_decode_attn_rope(ctypes.byref(s), _ptr(q), _ptr(t_q), _ptr(rope_cos), _ptr(rope_sin),
                                           int(n_keep), nb, B, hq, _ptr(page_table), int(page_table.shape[1]),
                                           _ptr(seq_lens), float(sm_scale), int(num_splits), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                                           _ptr(q_prime), _ptr(sel_idx), _stream(stream))
    _check(rc, "dqk_select_decode_attn_rope")
    return out, lse, q_prime, sel_idx


def prepared(name: str, *args):
    """A zero-argument callable that invokes C entry point `name` with the
    given arguments, marshalled once (torch tensors become their device
    addresses, a Cache or Tiers its struct, None NULL, streams their handles), and
    raises on a non-zero status.  For tight launch loops; the tensors must
    outlive the callable."""
    import torch
    L = lib()
    fn = getattr(L, name)
    conv, keep = [], []
    for a in args:
        if isinstance(a, (Cache, Tiers)):
            st = a.struct()
            keep.append(st)
            conv.append(ctypes.byref(st))
        elif isinstance(a, torch.Tensor):
            conv.append(a.data_ptr())
        elif isinstance(a, torch.cuda.Stream):
            conv.append(a.cuda_stream)
        else:
            conv.append(a)
    conv = tuple(conv)

    def call():
        rc = fn(*conv)
        if rc != DQK_OK:
            raise DqkError(rc, name)

    call.keep = keep
    return call


def dqk_decode_attn_noalloc(cache: Cache, q_prime, sel_idx, page_table, seq_lens, sm_scale: float,
                            num_splits: int = 0, out=None, lse=None, want_lse: bool = True, stream=None):
    """dqk_decode_attn through the entry point that allocates nothing on the
    device (its partials live in the library's own scratch array); out / lse
    are allocated here only when not given."""
    import torch
    B, hq = int(q_prime.shape[0]), int(q_prime.shape[1])
    n_keep = int(sel_idx.shape[2])
    max_pages = int(page_table.shape[1])
    dev = q_prime.device
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    s = cache.struct()
    rc = lib().dqk_decode_attn_noalloc(ctypes.byref(s), _ptr(q_prime), _ptr(sel_idx), n_keep, B, hq, _ptr(page_table),
                                       max_pages, _ptr(seq_lens), float(sm_scale), int(num_splits), _ptr(out),
                                       _ptr(lse), _stream(stream))
    _check(rc, "dqk_decode_attn_noalloc")
    return out, lse


def dqk_decode_attn_bf16(k_pages, v_pages, q, page_table, seq_lens, sm_scale: float, num_splits: int = 0,
                         workspace=None, out=None, lse=None, want_lse: bool = True, stream=None):
    import torch
    num_pages, hkv = int(k_pages.shape[0]), int(k_pages.shape[1])
    B, hq = int(q.shape[0]), int(q.shape[1])
    max_pages = int(page_table.shape[1])
    dev = q.device
    if workspace is None:
        workspace = _workspace(B, hq, hkv, max_pages, num_splits, dev)
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    rc = lib().dqk_decode_attn_bf16(_ptr(k_pages), _ptr(v_pages), hkv, num_pages, _ptr(q), B, hq, _ptr(page_table),
                                    max_pages, _ptr(seq_lens), float(sm_scale), int(num_splits), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                                    _stream(stream))
    _check(rc, "dqk_decode_attn_bf16")
    return out, lse


def dqk_stream_read(src, sink, stream=None):
    """Measurement helper: plain streaming read of all of `src` (device tensor,
    a multiple of 16 KiB); `sink` is a device uint32/int32 tensor of 4096 entries."""
    rc = lib().dqk_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream))
    _check(rc, "dqk_stream_read")
