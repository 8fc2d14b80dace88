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
        L.dqk_decode_attn_bf16.argtypes = [P, P, i32, i32, P, i32, i32, P, i32, P, ctypes.c_float, i32, P, sz, P, P,
                                           P]
        L.dqk_decode_attn_bf16.restype = ctypes.c_int
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
    """Device buffers of the paged INT2 cache (layout in include/dqk.h)."""

    def __init__(self, num_pages: int, num_kv_heads: int, device="cuda"):
        import torch
        self.num_pages, self.num_kv_heads = int(num_pages), int(num_kv_heads)
        P, H = self.num_pages, self.num_kv_heads
        self.k_codes = torch.zeros((P, H, HEAD_DIM, 32), dtype=torch.uint8, device=device)
        self.k_meta = torch.zeros((P, H, HEAD_DIM, 2), dtype=torch.int16, device=device)
        self.k_ch0 = torch.zeros((P, H, PAGE), dtype=torch.int16, device=device)
        self.v_codes = torch.zeros((P, H, PAGE, 32), dtype=torch.uint8, device=device)
        self.v_meta = torch.zeros((P, H, 2, 4, PAGE), dtype=torch.int16, device=device)

    def arrays(self):
        return self.k_codes, self.k_meta, self.k_ch0, self.v_codes, self.v_meta

    def struct(self) -> dqk_cache:
        return dqk_cache(self.num_kv_heads, self.num_pages, *[a.data_ptr() for a in self.arrays()])

    def nbytes(self) -> int:
        return sum(a.numel() * a.element_size() for a in self.arrays())


def dqk_quantize_append(cache: Cache, k, v, t_k, cu_tokens, page_table, kprime_dbg=None, stream=None):
    n_seqs = cu_tokens.numel() - 1
    s = cache.struct()
    rc = lib().dqk_quantize_append(ctypes.byref(s), _ptr(k), _ptr(v), _ptr(t_k), n_seqs, _ptr(cu_tokens),
                                   int(k.shape[0]), _ptr(page_table), int(page_table.shape[1]), _ptr(kprime_dbg),
                                   _stream(stream))
    _check(rc, "dqk_quantize_append")


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


def dqk_decode_workspace_size(batch: int, hq: int, hkv: int, max_pages: int, num_splits: int = 0) -> int:
    return int(lib().dqk_decode_workspace_size(batch, hq, hkv, max_pages, num_splits))


def _workspace(batch, hq, hkv, max_pages, num_splits, device):
    import torch
    n = dqk_decode_workspace_size(batch, hq, hkv, max_pages, num_splits)
    return torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device=device)


def dqk_decode_attn(cache: Cache, q_prime, sel_idx, page_table, seq_lens, sm_scale: float, num_splits: int = 0,
                    workspace=None, out=None, lse=None, want_lse: bool = True, stream=None):
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
    rc = lib().dqk_decode_attn(ctypes.byref(s), _ptr(q_prime), _ptr(sel_idx), n_keep, B, hq, _ptr(page_table),
                               max_pages, _ptr(seq_lens), float(sm_scale), int(num_splits), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream))
    _check(rc, "dqk_decode_attn")
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
