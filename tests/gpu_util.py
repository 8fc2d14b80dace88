"""Helpers for the GPU parity tests: move seeded inputs and caches between
numpy (oracle side) and device tensors (libdqk side)."""
import numpy as np
import torch

import oracle
import page_set_amd as pa

TOL = 2e-3   # max relative error per (sequence, head) row, fp32 accumulate


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def upload(prob):
    d = dict(q=dev(prob.q), t_q=dev(prob.t_q), t_k=dev(prob.t_k), page_table=dev(prob.page_table),
             seq_lens=dev(prob.seq_lens), cu=dev(prob.cu_tokens))
    if prob.k is not None:
        d["k"] = dev(prob.k)
        d["v"] = dev(prob.v)
    return d


def cache_to_device(c: oracle.Cache) -> pa.Cache:
    g = pa.Cache(c.num_pages, c.hkv)
    for src, dst in zip(c.arrays(), g.arrays()):
        dst.copy_(dev(src))
    return g


def cache_to_host(g: pa.Cache) -> oracle.Cache:
    c = oracle.Cache(g.num_pages, g.num_kv_heads)
    for src, dst in zip(g.arrays(), c.arrays()):
        dst[...] = host(src, dst.dtype)
    return c


def row_rel_err(got, want):
    """max_c |got - want| / max_c |want| for every (b, h) row."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    num = np.abs(got - want).max(axis=-1)
    den = np.abs(want).max(axis=-1)
    return num / np.maximum(den, 1e-30)
