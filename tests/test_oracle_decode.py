"""Pins of the oracle's paged decode attention (§3.2, §3.3, §3.4)."""
import math

import numpy as np
import pytest
import torch

import synth
from tests import cachefmt as cf


def _sdpa(q, k, v, scale):
    """Textbook softmax attention through torch's library routine (fp64, CPU).
    q [H][d], k [L][d], v [L][d] -> [H][d]"""
    qt = torch.from_numpy(np.ascontiguousarray(q, np.float64))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(v, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0, :].numpy()


def _build(orc, shape, seed):
    prob = synth.make_problem(shape, seed=seed)
    cache, kp = orc.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = orc.select_channels(prob.q, prob.t_q, shape.hkv, shape.n_keep)
    return prob, cache, kp, qp, sel


@pytest.mark.parametrize("n_keep", [128, 77, 1])
@pytest.mark.parametrize("hq,hkv,lens", [(8, 8, [300, 5]), (32, 8, [129, 256]), (4, 1, [1000])])
def test_decode_equals_library_attention_on_decoded_cache(orc, n_keep, hq, hkv, lens):
    """Pruning restricts the dot product to the selected channels, i.e. it is
    textbook attention with the unselected query channels zeroed; at n_keep=128
    it is plain dense attention over the dequantized cache."""
    shape = synth.Shape(len(lens), hq, hkv, lens, n_keep, shuffle_pages=True)
    prob, cache, kp, qp, sel = _build(orc, shape, 21)
    out, lse = orc.decode_attn(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    grp = hq // hkv
    for b in range(shape.batch):
        for g in range(hkv):
            kh, vh = cf.gather_seq(cache, prob.page_table, b, int(prob.seq_lens[b]), g)
            mask = np.zeros(128)
            mask[sel[b, g]] = 1.0
            qm = qp[b, g * grp:(g + 1) * grp].astype(np.float64) * mask
            want = _sdpa(qm, kh, vh, prob.sm_scale)
            np.testing.assert_allclose(out[b, g * grp:(g + 1) * grp], want, rtol=1e-10, atol=1e-12)
            logits = (qm @ kh.astype(np.float64).T) * prob.sm_scale
            want_lse = np.log(np.exp(logits - logits.max(1, keepdims=True)).sum(1)) + logits.max(1)
            np.testing.assert_allclose(lse[b, g * grp:(g + 1) * grp], want_lse, rtol=1e-12)


@pytest.mark.parametrize("L", [1, 5, 127, 128, 129, 256])
@pytest.mark.parametrize("hq,n_keep", [(1, 1), (1, 128), (4, 2), (4, 77)])
def test_decode_tiny_brute_force(orc, L, hq, n_keep):
    """Pure-Python enumeration straight from the definitions."""
    shape = synth.Shape(1, hq, 1, [L], n_keep)
    prob, cache, kp, qp, sel = _build(orc, shape, 100 + L)
    out, lse = orc.decode_attn(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    for h in range(hq):
        logits = []
        for t in range(L):
            p, s = int(prob.page_table[0, t // 128]), t % 128
            acc = 0.0
            for j in sel[0, 0]:
                if j == 0:
                    kv = float(cf.bf16(cache.k_ch0[p, 0, s]))
                else:
                    code = (int(cache.k_rows(p)[0, j, s // 4]) >> (2 * (s % 4))) & 3
                    km = cache.k_meta_page(p)[0, j]
                    kv = float(np.float32(code) * cf.f16(km[0]) + cf.f16(km[1]))
                acc += float(qp[0, h, j]) * kv
            logits.append(acc / math.sqrt(128))
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        tot = sum(w)
        for c in range(0, 128, 17):
            o = 0.0
            for t in range(L):
                p, s = int(prob.page_table[0, t // 128]), t % 128
                code = (int(cache.v_codes[p, 0, s, c // 4]) >> (2 * (c % 4))) & 3
                sc = cf.f16(cache.v_meta[p, 0, 0, c // 32, s])
                zc = cf.f16(cache.v_meta[p, 0, 1, c // 32, s])
                o += w[t] * float(np.float32(code) * sc + zc)
            assert abs(out[0, h, c] - o / tot) <= 1e-12 * max(1.0, abs(o / tot))
        assert abs(lse[0, h] - (m + math.log(tot))) <= 1e-12 * abs(m + math.log(tot)) + 1e-12
    if L == 1:
        # a single token: the output is its value row, lse is its logit
        np.testing.assert_allclose(out[0], np.repeat(cf.decode_v(cache, 0, 0)[:1], hq, 0), rtol=1e-7)


def test_decode_invariant_to_page_permutation_and_slot_garbage(orc):
    shape = synth.Shape(2, 8, 2, [300, 129], 77)
    prob, cache, kp, qp, sel = _build(orc, shape, 31)
    out1, lse1 = orc.decode_attn(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    perm = np.random.default_rng(1).permutation(prob.num_pages)
    c2 = orc.Cache(prob.num_pages, shape.hkv)
    moved = []
    for a_src in cache.page_major():
        a_dst = np.empty_like(a_src)
        a_dst[perm] = a_src
        moved.append(a_dst)
    c2.set_page_major(*moved)
    pt2 = np.where(prob.page_table >= 0, perm[np.maximum(prob.page_table, 0)], -1).astype(np.int32)
    # garbage in every slot past each sequence's end
    rng = np.random.default_rng(2)
    for b in range(2):
        L = int(prob.seq_lens[b])
        p = int(pt2[b, (L - 1) // 128])
        s = L % 128
        if s:
            c2.v_codes[p, :, s:] = rng.integers(0, 256, c2.v_codes[p, :, s:].shape, dtype=np.uint8)
            c2.k_ch0[p, :, s:] = rng.integers(0, 0x3F00, c2.k_ch0[p, :, s:].shape).astype(np.uint16)
            rows = c2.k_rows(p)[:, :, s // 4 + 1:]
            c2.k_rows(p)[:, :, s // 4 + 1:] = rng.integers(0, 256, rows.shape, dtype=np.uint8)
    out2, lse2 = orc.decode_attn(c2, qp, sel, pt2, prob.seq_lens, prob.sm_scale)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


def test_decode_close_to_unquantized_attention(orc):
    """Sanity (not parity): with no pruning the INT2 cache stays close to
    attention on the raw bf16 inputs, which the dual transform leaves
    unchanged before compression (§3.1 Eq. 1)."""
    shape = synth.Shape(1, 8, 2, [2048], 128)
    prob, cache, kp, qp, sel = _build(orc, shape, 41)
    out, _ = orc.decode_attn(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    q = synth.bf16_bits_to_f32(prob.q).astype(np.float64)
    k = synth.bf16_bits_to_f32(prob.k).astype(np.float64)
    v = synth.bf16_bits_to_f32(prob.v).astype(np.float64)
    for g in range(2):
        want = _sdpa(q[0, 4 * g:4 * g + 4], k[:, g], v[:, g], prob.sm_scale)
        o = out[0, 4 * g:4 * g + 4]
        cos = (o * want).sum() / np.sqrt((o * o).sum() * (want * want).sum())
        assert cos > 0.5   # INT2 on unstructured Gaussian data gives ~0.7


def test_pruned_logit_variance_matches_appendix_c2(orc):
    """App. C.2: for keys with i.i.d. channels of variance sigma^2, the omitted
    part of the logit has variance sigma^2 * sum_{j not in M} q_j^2.  One
    token per page makes every key grid a single point, so dequantized keys
    equal the inputs to binary16 precision and the statistic is visible
    through the per-sequence lse (= the logit for a one-token context)."""
    n, sigma = 4096, 0.7
    rng = np.random.default_rng(5)
    kprime = (rng.standard_normal((n, 1, 128)) * sigma).astype(np.float32)
    v = np.zeros((n, 1, 128), np.uint16)
    cu = np.arange(n + 1, dtype=np.int32)
    pt = np.arange(n, dtype=np.int32)[:, None]
    cache = orc.pack_cache(kprime, v, cu, pt, n)
    qp = np.tile(rng.standard_normal(128).astype(np.float32), (n, 1))[:, None, :]
    lens = np.ones(n, np.int32)
    full = np.tile(np.arange(128, dtype=np.int32), (n, 1))[:, None, :]
    k = 77
    keep = np.sort(np.argsort(-np.abs(qp[0, 0]))[:k]).astype(np.int32)
    part = np.tile(keep, (n, 1))[:, None, :]
    _, lse_full = orc.decode_attn(cache, qp, full, pt, lens, 1.0)
    _, lse_part = orc.decode_attn(cache, qp, part, pt, lens, 1.0)
    omitted = np.setdiff1d(np.arange(128), keep)
    want = sigma ** 2 * float((qp[0, 0, omitted].astype(np.float64) ** 2).sum())
    got = np.var(lse_full[:, 0] - lse_part[:, 0])
    assert abs(got / want - 1) < 0.1
