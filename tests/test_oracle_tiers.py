"""Pins of the oracle's protected BF16 tiers (Dual-QK §3.3: the first 64 and
the most recent 256 tokens in BF16 for keys and values, same channel mask;
§3.4: one softmax over every token)."""
import math

import numpy as np
import pytest
import torch

import synth
from tests import cachefmt as cf


def _bf16_bits_torch(x):
    """fp32 -> bf16 bits through torch's cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("L", [1, 63, 64, 65, 319, 320, 321, 447, 448, 449, 575, 576, 1000, 5000])
def test_tier_membership(orc, L):
    """Every token sits in exactly one place; INT2 tokens are older than the
    256 most recent and come in whole pages, as many as fit; the tail holds
    the rest (fewer than 256 + 128 tokens)."""
    P = orc.tier_pages(L)
    sink = list(range(min(L, 64)))
    int2 = list(range(64, 64 + 128 * P))
    tail = list(range(64 + 128 * P, L)) if L > 64 else []
    assert sorted(sink + int2 + tail) == list(range(L))
    assert all(t < L - 256 for t in int2)
    # one more page would take a token among the 256 most recent
    assert 64 + 128 * (P + 1) > L - 256
    assert len(tail) < 256 + 128
    if L >= 320:
        assert len(tail) >= 256
    # tail slots are distinct
    assert len({(t - 64) % 384 for t in tail}) == len(tail)


def _problem(shape, seed):
    return synth.make_problem(shape, seed=seed)


@pytest.mark.parametrize("lens", [[5, 700], [320, 449, 64]])
def test_prefill_tiered_layout(orc, lens):
    """Tier slots hold bf16(k') (torch's rounding) and the inputs; INT2 page
    i of a sequence decodes to the quantized tokens 64 + 128 i .. + 127."""
    shape = synth.Shape(len(lens), 8, 2, lens, 77, shuffle_pages=True)
    prob = _problem(shape, 41)
    cache, tiers = orc.prefill_tiered(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    kp = orc.key_transform(prob.k, prob.t_k)
    for b, L in enumerate(lens):
        t0 = int(prob.cu_tokens[b])
        P = orc.tier_pages(L)
        for t in range(L):
            if t < 64:
                np.testing.assert_array_equal(tiers.sink_k[b, :, t], _bf16_bits_torch(kp[t0 + t]))
                np.testing.assert_array_equal(tiers.sink_v[b, :, t], prob.v[t0 + t])
            elif t >= 64 + 128 * P:
                s = (t - 64) % 384
                np.testing.assert_array_equal(tiers.tail_k[b, :, s], _bf16_bits_torch(kp[t0 + t]))
                np.testing.assert_array_equal(tiers.tail_v[b, :, s], prob.v[t0 + t])
                np.testing.assert_array_equal(tiers.tail_kraw[b, :, s], prob.k[t0 + t])
        for i in range(P):
            p = int(prob.page_table[b, i])
            for g in range(shape.hkv):
                # values: each (token, group) quantized on its own
                vt = synth.bf16_bits_to_f32(prob.v[t0 + 64 + 128 * i:t0 + 64 + 128 * (i + 1), g])
                for tok in (0, 77, 127):
                    s_bits, z_bits, codes = orc.quantize_group(vt[tok, 32:64])
                    assert cf.v_codes(cache, p, g)[tok, 32:64].tolist() == list(codes)
                    assert int(cache.v_meta[p, g, 0, 1, tok]) == s_bits and int(cache.v_meta[p, g, 1, 1, tok]) == z_bits
                # keys: channel 5 over the page's 128 tokens
                s_bits, z_bits, codes = orc.quantize_group(kp[t0 + 64 + 128 * i:t0 + 64 + 128 * (i + 1), g, 5])
                assert cf.k_codes(cache, p, g)[5].tolist() == list(codes)


@pytest.mark.parametrize("L0,L1", [(0, 70), (100, 720), (447, 449), (1000, 1300)])
def test_append_token_reproduces_prefill(orc, L0, L1):
    """Appending tokens one at a time from L0 to L1 gives the same INT2 pages
    and the same live tier slots as a prefill of L1 tokens."""
    shape = synth.Shape(2, 8, 2, [L1, L1 - 1], 77)
    prob = _problem(shape, 43)
    want_c, want_t = orc.prefill_tiered(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    starts = [min(L0, L) for L in shape.seq_lens]
    pre_lens = np.array(starts, np.int32)
    pre_cu = np.concatenate([[0], np.cumsum(pre_lens)]).astype(np.int32)
    ks = np.concatenate([prob.k[prob.cu_tokens[b]:prob.cu_tokens[b] + starts[b]] for b in range(2)])
    vs = np.concatenate([prob.v[prob.cu_tokens[b]:prob.cu_tokens[b] + starts[b]] for b in range(2)])
    if pre_cu[-1] > 0:
        cache, tiers = orc.prefill_tiered(ks, vs, prob.t_k, pre_cu, prob.page_table, prob.num_pages)
    else:
        cache, tiers = orc.Cache(prob.num_pages, shape.hkv), orc.Tiers(2, shape.hkv)
    lens = pre_lens.copy()
    while (lens < np.array(shape.seq_lens)).any():
        active = lens < np.array(shape.seq_lens)
        kn = np.zeros((2, shape.hkv, 128), np.uint16)
        vn = np.zeros_like(kn)
        for b in range(2):
            t = int(lens[b]) if active[b] else int(lens[b]) - 1
            kn[b] = prob.k[prob.cu_tokens[b] + t]
            vn[b] = prob.v[prob.cu_tokens[b] + t]
        # a finished sequence re-appends its last token at its last position:
        # same bytes, no page completes (the page count depends on the length only)
        before = np.where(active, lens, lens - 1).astype(np.int32)
        orc.append_token(cache, tiers, kn, vn, prob.t_k, before, prob.page_table)
        lens = lens + active
    for a, w in zip(cache.arrays(), want_c.arrays()):
        np.testing.assert_array_equal(a, w)
    for b, L in enumerate(shape.seq_lens):
        P = orc.tier_pages(L)
        live = [(t - 64) % 384 for t in range(64 + 128 * P, L)]
        np.testing.assert_array_equal(tiers.sink_k[b, :, :min(L, 64)], want_t.sink_k[b, :, :min(L, 64)])
        np.testing.assert_array_equal(tiers.sink_v[b, :, :min(L, 64)], want_t.sink_v[b, :, :min(L, 64)])
        for arr, warr in zip((tiers.tail_k, tiers.tail_v, tiers.tail_kraw),
                             (want_t.tail_k, want_t.tail_v, want_t.tail_kraw)):
            np.testing.assert_array_equal(arr[b][:, live], warr[b][:, live])


def _tier_tokens(orc, tiers, b, g, L):
    """(k', v) fp64 [n][128] of the BF16 tokens of sequence b, in token order."""
    P = orc.tier_pages(L)
    ks, vs = [], []
    for t in list(range(min(L, 64))) + list(range(64 + 128 * P, L) if L > 64 else []):
        if t < 64:
            ks.append(cf.bf16(tiers.sink_k[b, g, t]))
            vs.append(cf.bf16(tiers.sink_v[b, g, t]))
        else:
            s = (t - 64) % 384
            ks.append(cf.bf16(tiers.tail_k[b, g, s]))
            vs.append(cf.bf16(tiers.tail_v[b, g, s]))
    return np.array(ks, np.float64), np.array(vs, np.float64)


@pytest.mark.parametrize("lens,hq,hkv,n_keep", [([5, 300], 8, 2, 77), ([449, 1000], 32, 8, 52),
                                                 ([2000], 4, 1, 128)])
def test_decode_tiered_equals_textbook_attention(orc, lens, hq, hkv, n_keep):
    """The three token sources decoded independently (numpy readers of the
    INT2 pages and of the bf16 tiers), then textbook softmax attention in
    fp64 with the unselected channels zeroed."""
    shape = synth.Shape(len(lens), hq, hkv, lens, n_keep, shuffle_pages=True)
    prob = _problem(shape, 47)
    cache, tiers = orc.prefill_tiered(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = orc.select_channels(prob.q, prob.t_q, hkv, n_keep)
    out, lse = orc.decode_tiered(cache, tiers, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    grp = hq // hkv
    for b, L in enumerate(lens):
        P = orc.tier_pages(L)
        for g in range(hkv):
            kt, vt = _tier_tokens(orc, tiers, b, g, L)
            n_sink = min(L, 64)
            if P:
                ki, vi = cf.gather_seq(cache, prob.page_table, b, 128 * P, g)
                k = np.concatenate([kt[:n_sink], ki, kt[n_sink:]])
                v = np.concatenate([vt[:n_sink], vi, vt[n_sink:]])
            else:
                k, v = kt, vt
            assert k.shape[0] == L
            mask = np.zeros(128)
            mask[sel[b, g]] = 1.0
            qm = qp[b, g * grp:(g + 1) * grp].astype(np.float64) * mask
            x = qm @ k.T * prob.sm_scale
            m = x.max(1, keepdims=True)
            w = np.exp(x - m)
            want = (w @ v) / w.sum(1, keepdims=True)
            np.testing.assert_allclose(out[b, g * grp:(g + 1) * grp], want, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[b, g * grp:(g + 1) * grp], (m[:, 0] + np.log(w.sum(1))), rtol=1e-12)


def test_decode_tiered_splits_into_int2_and_bf16_parts(orc):
    """log-sum-exp decomposition: the tiered output combines decode_attn over
    the INT2 pages alone with attention over the BF16 tokens alone."""
    lens = [1300, 500]
    shape = synth.Shape(2, 8, 2, lens, 77, shuffle_pages=True)
    prob = _problem(shape, 53)
    cache, tiers = orc.prefill_tiered(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = orc.select_channels(prob.q, prob.t_q, 2, 77)
    out, lse = orc.decode_tiered(cache, tiers, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    n_int2 = np.array([128 * orc.tier_pages(L) for L in lens], np.int32)
    oa, la = orc.decode_attn(cache, qp, sel, prob.page_table, n_int2, prob.sm_scale)
    for b, L in enumerate(lens):
        for h in range(8):
            g = h // 4
            kt, vt = _tier_tokens(orc, tiers, b, g, L)
            mask = np.zeros(128)
            mask[sel[b, g]] = 1.0
            x = (qp[b, h].astype(np.float64) * mask) @ kt.T * prob.sm_scale
            lb = x.max() + math.log(np.exp(x - x.max()).sum())
            ob = np.exp(x - lb) @ vt
            M = max(la[b, h], lb)
            wa, wb = math.exp(la[b, h] - M), math.exp(lb - M)
            np.testing.assert_allclose(out[b, h], (wa * oa[b, h] + wb * ob) / (wa + wb), rtol=1e-9, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], M + math.log(wa + wb), rtol=1e-12)


@pytest.mark.parametrize("L", [1, 3, 70])
def test_decode_tiered_tiny_brute_force(orc, L):
    """All tokens in BF16 (no page yet): pure-Python enumeration."""
    shape = synth.Shape(1, 2, 1, [L], 5)
    prob = _problem(shape, 59 + L)
    cache, tiers = orc.prefill_tiered(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = orc.select_channels(prob.q, prob.t_q, 1, 5)
    out, lse = orc.decode_tiered(cache, tiers, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    for h in range(2):
        logits = []
        for t in range(L):
            row = tiers.sink_k[0, 0, t] if t < 64 else tiers.tail_k[0, 0, (t - 64) % 384]
            logits.append(sum(float(qp[0, h, j]) * float(cf.bf16(row[j])) for j in sel[0, 0]) / math.sqrt(128))
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        for c in (0, 64, 127):
            o = sum(w[t] * float(cf.bf16((tiers.sink_v[0, 0, t] if t < 64 else
                                          tiers.tail_v[0, 0, (t - 64) % 384])[c])) for t in range(L))
            assert abs(out[0, h, c] - o / sum(w)) <= 1e-12 * max(1.0, abs(o / sum(w)))
