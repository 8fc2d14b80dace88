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


def lse_bound(cache, qp, sel, page_table, seq_lens, sm_scale, lse_ref, gather=None):
    """Allowed |lse_gpu - lse_oracle| per (b, h) row.

    The kernels form each logit as an fp32 sum over the selected channels of
    products whose query-side operand carries at least 21 significant bits
    (q' * scale split into two binary16 limbs), so every logit is off by at
    most about n * 2^-24 + 2^-21 <= 2^-16 times the sum of the absolute
    values of its terms (n <= 128).  The log-sum-exp is a softmax-weighted
    mean of the logits, so its error is bounded by the largest logit error,
    plus the fp32 rounding of exp2/log2 and of the merge (2^-20 |lse|)."""
    from tests import cachefmt as cf
    gather = gather or cf.gather_seq
    B, hq = qp.shape[0], qp.shape[1]
    hkv = sel.shape[1]
    grp = hq // hkv
    out = np.zeros((B, hq))
    for b in range(B):
        L = int(seq_lens[b])
        for g in range(hkv):
            kh, _ = gather(cache, page_table, b, L, g)
            mask = np.zeros(128)
            mask[sel[b, g]] = 1.0
            qa = np.abs(qp[b, g * grp:(g + 1) * grp].astype(np.float64)) * mask
            out[b, g * grp:(g + 1) * grp] = (np.abs(kh.astype(np.float64)) @ qa.T).max(0) * sm_scale
    return 2.0 ** -16 * out + 2.0 ** -20 * np.abs(lse_ref)


def assert_lse(lse, lse_ref, bound):
    err = np.abs(np.asarray(lse, np.float64) - lse_ref)
    assert (err <= bound).all(), f"lse error {err.max():.3e} above the derived bound (worst ratio {(err / bound).max():.2f})"


def split_bound(cache, qp, sel, page_table, seq_lens, sm_scale, gather=None):
    """Allowed |o(one split count) - o(another)| per (b, h, channel) for the
    group-4 MFMA decode.

    Each split rounds the probabilities P_t = 2^(x_t - m + 14), m its own
    integer running maximum, to binary16, and the products A_t = P_t s'_t
    (s' = s 2^-E, E the split's running scale exponent) to binary16 again;
    u = 2^-11 is the unit roundoff of each.  With p_t the exact softmax
    weights, one split's output differs from the exact sum by at most
      sum_t p_t (u |z_t + 1.5 s_t| + 2u |s_t| |c_t - 1.5|)   centred value terms
      + u |o_c|                                              the sum of P (normalisation)
      + 2^-15 sum_t p_t |v_t|                                fp32 accumulation
      + 2^-24 max_t s_t                                      subnormal P s'
      + L 2^-38 max_t |v_t|                                  subnormal P,
    two splits by twice that."""
    from tests import cachefmt as cf
    gather = gather or cf.gather_seq
    u = 2.0 ** -11
    B, hq = qp.shape[0], qp.shape[1]
    hkv = sel.shape[1]
    grp = hq // hkv
    bound = np.zeros((B, hq, 128))
    for b in range(B):
        L = int(seq_lens[b])
        for g in range(hkv):
            kh, vh = gather(cache, page_table, b, L, g)
            codes, sc, zp = cf.gather_vparts(cache, page_table, b, L, g)
            mask = np.zeros(128)
            mask[sel[b, g]] = 1.0
            q = qp[b, g * grp:(g + 1) * grp].astype(np.float64) * mask
            x = (kh.astype(np.float64) @ q.T) * sm_scale            # [L][grp]
            p = np.exp(x - x.max(0))
            p /= p.sum(0)
            v = vh.astype(np.float64)
            s64, z64 = sc.astype(np.float64), zp.astype(np.float64)
            centred = u * np.abs(z64 + 1.5 * s64) + 2 * u * np.abs(s64) * np.abs(codes - 1.5)
            o = p.T @ v                                              # [grp][128]
            one = (p.T @ centred + u * np.abs(o) + 2.0 ** -15 * (p.T @ np.abs(v))
                   + 2.0 ** -24 * np.abs(s64).max() + L * 2.0 ** -38 * np.abs(v).max(0))
            bound[b, g * grp:(g + 1) * grp] = 2 * one
    return bound
