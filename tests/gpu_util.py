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


def lse_bound(cache, qp, sel, page_table, seq_lens, sm_scale, lse_ref):
    """Allowed |lse_gpu - lse_oracle| per (b, h) row.

    The kernels form each logit as an fp32 sum over the selected channels of
    products whose query-side operand carries at least 21 significant bits
    (q' * scale split into two binary16 limbs), so every logit is off by at
    most about n * 2^-24 + 2^-21 <= 2^-16 times the sum of the absolute
    values of its terms (n <= 128).  The log-sum-exp is a softmax-weighted
    mean of the logits, so its error is bounded by the largest logit error,
    plus the fp32 rounding of exp2/log2 and of the merge (2^-20 |lse|)."""
    from tests import cachefmt as cf
    B, hq = qp.shape[0], qp.shape[1]
    hkv = sel.shape[1]
    grp = hq // hkv
    out = np.zeros((B, hq))
    for b in range(B):
        L = int(seq_lens[b])
        for g in range(hkv):
            kh, _ = cf.gather_seq(cache, page_table, b, L, g)
            mask = np.zeros(128)
            mask[sel[b, g]] = 1.0
            qa = np.abs(qp[b, g * grp:(g + 1) * grp].astype(np.float64)) * mask
            out[b, g * grp:(g + 1) * grp] = (np.abs(kh.astype(np.float64)) @ qa.T).max(0) * sm_scale
    return 2.0 ** -16 * out + 2.0 ** -20 * np.abs(lse_ref)


def assert_lse(lse, lse_ref, bound):
    err = np.abs(np.asarray(lse, np.float64) - lse_ref)
    assert (err <= bound).all(), f"lse error {err.max():.3e} above the derived bound (worst ratio {(err / bound).max():.2f})"
