"""Pins of the oracle's unpruned BF16 decode attention (the baseline the
Dual-QK paper measures its throughput against, §4.4 and Table 1's BF16 row).

The oracle function reads a paged bf16 cache; these tests check it against
attention computed directly from the raw, unpaged bf16 keys and values
(gathered here with plain numpy, never through the oracle's own pager), so a
transposed key, a dropped softmax scale or a page-table slip fails one of
them.
"""
import math

import numpy as np
import pytest

import synth


def _raw_attention(prob, b, h, scale):
    """softmax(q k^T * scale) v in fp64 for query head h of sequence b, from the
    raw token-major inputs [T][Hkv][128] (no pages involved)."""
    grp = prob.shape.hq // prob.shape.hkv
    g = h // grp
    s, e = int(prob.cu_tokens[b]), int(prob.cu_tokens[b + 1])
    q = synth.bf16_bits_to_f32(prob.q[b, h]).astype(np.float64)
    k = synth.bf16_bits_to_f32(prob.k[s:e, g]).astype(np.float64)
    v = synth.bf16_bits_to_f32(prob.v[s:e, g]).astype(np.float64)
    logits = (k @ q) * scale
    m = logits.max()
    w = np.exp(logits - m)
    return (w @ v) / w.sum(), m + math.log(w.sum())


def _run(orc, prob, scale=None):
    scale = prob.sm_scale if scale is None else scale
    kb, vb = orc.paged_bf16(prob.k, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    return orc.decode_bf16(kb, vb, prob.q, prob.page_table, prob.seq_lens, scale)


@pytest.mark.parametrize("L", [1, 5, 128, 129])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 1), (4, 4), (8, 2)])
def test_bf16_decode_equals_raw_attention(orc, L, hq, hkv):
    shape = synth.Shape(2, hq, hkv, [L, L + 300], 128, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=60 + L + hq)
    out, lse = _run(orc, prob)
    for b in range(2):
        for h in range(hq):
            want, want_lse = _raw_attention(prob, b, h, prob.sm_scale)
            np.testing.assert_allclose(out[b, h], want, rtol=1e-12, atol=1e-13)
            assert abs(lse[b, h] - want_lse) <= 1e-12 * max(1.0, abs(want_lse))


def test_bf16_decode_tiny_brute_force(orc):
    """Pure-Python loops over tokens and channels for a 3-token context."""
    shape = synth.Shape(1, 2, 1, [3], 128)
    prob = synth.make_problem(shape, seed=71)
    out, lse = _run(orc, prob)
    q = synth.bf16_bits_to_f32(prob.q).astype(np.float64)
    k = synth.bf16_bits_to_f32(prob.k).astype(np.float64)
    v = synth.bf16_bits_to_f32(prob.v).astype(np.float64)
    for h in range(2):
        logits = [sum(q[0, h, c] * k[t, 0, c] for c in range(128)) / math.sqrt(128) for t in range(3)]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        for c in range(128):
            want = sum(w[t] * v[t, 0, c] for t in range(3)) / sum(w)
            assert abs(out[0, h, c] - want) <= 1e-12 * max(1.0, abs(want))
        assert abs(lse[0, h] - (m + math.log(sum(w)))) <= 1e-12


def test_bf16_decode_uses_the_given_scale(orc):
    """The scale multiplies the logits: scale 0 gives the plain mean of the
    values (uniform weights) and lse = log L."""
    shape = synth.Shape(1, 4, 1, [200], 128)
    prob = synth.make_problem(shape, seed=72)
    out, lse = _run(orc, prob, scale=0.0)
    v = synth.bf16_bits_to_f32(prob.v[:, 0]).astype(np.float64)
    np.testing.assert_allclose(out[0], np.repeat(v.mean(0)[None], 4, 0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0], math.log(200), rtol=1e-14)
    out2, _ = _run(orc, prob, scale=0.5)
    want, _ = _raw_attention(prob, 0, 2, 0.5)
    np.testing.assert_allclose(out2[0, 2], want, rtol=1e-12, atol=1e-13)


def test_bf16_decode_page_permutation_and_tail_garbage(orc):
    """Moving pages in the physical pool (page table updated) changes nothing,
    and neither does garbage in the slots past each sequence's end."""
    shape = synth.Shape(2, 8, 2, [300, 129], 128)
    prob = synth.make_problem(shape, seed=73)
    kb, vb = orc.paged_bf16(prob.k, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    out1, lse1 = orc.decode_bf16(kb, vb, prob.q, prob.page_table, prob.seq_lens, prob.sm_scale)
    perm = np.random.default_rng(3).permutation(prob.num_pages)
    kb2, vb2 = np.empty_like(kb), np.empty_like(vb)
    kb2[perm], vb2[perm] = kb, vb
    pt2 = np.where(prob.page_table >= 0, perm[np.maximum(prob.page_table, 0)], -1).astype(np.int32)
    rng = np.random.default_rng(4)
    for b in range(2):
        L = int(prob.seq_lens[b])
        p = int(pt2[b, (L - 1) // 128])
        s = L % 128
        if s:
            kb2[p, :, s:] = rng.integers(0, 0x4000, kb2[p, :, s:].shape).astype(np.uint16)
            vb2[p, :, s:] = rng.integers(0, 0x4000, vb2[p, :, s:].shape).astype(np.uint16)
    out2, lse2 = orc.decode_bf16(kb2, vb2, prob.q, pt2, prob.seq_lens, prob.sm_scale)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


def test_paged_bf16_layout(orc):
    """The pager puts token t of sequence b, KV head g at [page_table[b][t // 128]][g][t % 128]."""
    shape = synth.Shape(2, 4, 2, [130, 7], 128, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=74)
    kb, vb = orc.paged_bf16(prob.k, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    for b in range(2):
        s = int(prob.cu_tokens[b])
        for t in range(int(prob.seq_lens[b])):
            p = int(prob.page_table[b, t // 128])
            np.testing.assert_array_equal(kb[p, :, t % 128], prob.k[s + t])
            np.testing.assert_array_equal(vb[p, :, t % 128], prob.v[s + t])
