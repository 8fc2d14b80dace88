"""Pins of the oracle's bucket-relative RoPE (Dual-QK paper, §3.4 and App.
C.4: each stored key is moved from its absolute position to the frame of its
2048-token bucket's anchor before the key transform; for every bucket the
current query gets the same anchor adjustment before the query transform and
its own channel mask; one softmax spans all tokens).

The rotation is checked against complex multiplication in fp64 (channel pair
(i, i + 64) as the number x_i + i x_{i+64}, turned back by the anchor angle),
written here from the definition of RoPE, not from the oracle."""
import numpy as np
import pytest
import torch

import synth
from tests import cachefmt as cf

U = 2.0 ** -24
BUCKET = 2048


def _angles(n_buckets, base=10000.0):
    i = np.arange(64, dtype=np.float64)
    theta = base ** (-2.0 * i / 128.0)
    return (BUCKET * np.arange(n_buckets, dtype=np.float64))[:, None] * theta[None, :]


def _turn(x, ang):
    """x [..., 128] fp64 turned by angle ang [64] per channel pair (i, i + 64)."""
    z = (x[..., :64] + 1j * x[..., 64:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def _eye_tk(hkv):
    return np.broadcast_to(synth.f32_to_bf16_bits(np.eye(128, dtype=np.float32)), (hkv, 128, 128)).copy()


def _identity_tables(nb):
    return np.ones((nb, 64), np.float32), np.zeros((nb, 64), np.float32)


def test_tables_are_the_anchor_rotations():
    cs, sn = synth.make_rope_tables(5)
    ang = _angles(5)
    np.testing.assert_allclose(cs, np.cos(ang), atol=1e-7)
    np.testing.assert_allclose(sn, -np.sin(ang), atol=1e-7)
    assert (cs[0] == 1).all() and (sn[0] == 0).all()


def test_identity_tables_reduce_to_the_plain_transforms(orc):
    shape = synth.Shape(2, 8, 2, [4100, 300], 77)
    prob = synth.make_problem(shape, seed=60)
    cs, sn = _identity_tables(3)
    kp = orc.key_transform(prob.k, prob.t_k)
    kr = orc.key_transform_rope(prob.k, prob.t_k, prob.cu_tokens, cs, sn)
    np.testing.assert_array_equal(kp, kr)
    qp, sel = orc.select_channels(prob.q, prob.t_q, 2, 77)
    qr, sr = orc.select_channels_rope(prob.q, prob.t_q, cs, sn, 2, 77)
    for k in range(3):
        np.testing.assert_array_equal(qr[:, k], qp)
        np.testing.assert_array_equal(sr[:, k], sel)


def test_keys_are_turned_back_by_their_bucket_anchor(orc):
    """T_K = I: k' is bf16 of the key turned by -a_k theta_i, with bucket
    k = position // 2048 counted from each sequence's start."""
    lens = [5000, 300, 2049]
    shape = synth.Shape(3, 4, 2, lens, 77)
    prob = synth.make_problem(shape, seed=61)
    nb = 3
    cs, sn = synth.make_rope_tables(nb)
    kp = orc.key_transform_rope(prob.k, _eye_tk(2), prob.cu_tokens, cs, sn).astype(np.float64)
    x = synth.bf16_bits_to_f32(prob.k).astype(np.float64)
    ang = _angles(nb)
    pos = np.concatenate([np.arange(L) for L in lens])
    want = np.empty_like(x)
    for k in range(nb):
        m = pos // BUCKET == k
        want[m] = _turn(x[m], -ang[k])
    pair = np.abs(x[..., :64]) + np.abs(x[..., 64:])
    slack = np.concatenate([pair, pair], axis=-1) * 4 * U
    assert (np.abs(kp - want) <= 2.0 ** -8 * np.abs(want) + slack).all()
    # the first bucket is not turned at all; tokens 2047 and 2048 use different anchors
    np.testing.assert_array_equal(kp[:2048], x[:2048])
    assert not np.allclose(kp[2048], x[2048], rtol=1e-3)


def test_scores_are_invariant_and_relative(orc):
    """App. C.4: with q and k rotary-embedded at absolute positions m and n,
    turning both back by the same anchor leaves the score q(m) . k(n), which
    depends on n - m only.  T_K = I, T_Q = I, n_keep = 128."""
    rng = np.random.default_rng(62)
    L, hkv, hq = 4600, 1, 2
    m = L - 1
    nb = synth.rope_buckets(L)
    theta = 10000.0 ** (-2.0 * np.arange(64) / 128.0)
    q0 = rng.standard_normal((hq, 128))
    k0 = rng.standard_normal((L, hkv, 128))
    q_abs = _turn(q0, m * theta)                                   # RoPE at position m
    k_abs = _turn(k0, np.arange(L)[:, None, None] * theta)          # RoPE at position n
    qb = synth.f32_to_bf16_bits(q_abs.astype(np.float32))[None]
    kb = synth.f32_to_bf16_bits(k_abs.astype(np.float32))
    cs, sn = synth.make_rope_tables(nb)
    cu = np.array([0, L], np.int32)
    kp = orc.key_transform_rope(kb, _eye_tk(hkv), cu, cs, sn).astype(np.float64)
    qp, sel = orc.select_channels_rope(qb, np.broadcast_to(np.eye(128, dtype=np.float32), (hkv, 128, 128)).copy(),
                                       cs, sn, hkv, 128)
    assert (sel == np.arange(128)).all()
    n = np.arange(L)
    rel = np.stack([(q0[h] * _turn(k0[:, 0], (n - m)[:, None] * theta)).sum(-1) for h in range(hq)])
    got = np.stack([(qp[0, n // BUCKET, h].astype(np.float64) * kp[:, 0]).sum(-1) for h in range(hq)])
    scale = np.stack([(np.abs(q0[h]).sum() * np.abs(k0[:, 0]).max(-1)) for h in range(hq)])
    assert (np.abs(got - rel) <= 2.0 ** -6 * scale[:, None]).all()


@pytest.mark.parametrize("hq,hkv,n_keep", [(8, 2, 77), (4, 4, 1), (32, 8, 128)])
def test_bucket_selection_is_plain_selection_of_the_turned_query(orc, hq, hkv, n_keep):
    shape = synth.Shape(2, hq, hkv, [128, 128], n_keep)
    prob = synth.make_problem(shape, seed=63, materialize_kv=False)
    nb = 4
    cs, sn = synth.make_rope_tables(nb)
    qp, sel = orc.select_channels_rope(prob.q, prob.t_q, cs, sn, hkv, n_keep)
    assert qp.shape == (2, nb, hq, 128) and sel.shape == (2, nb, hkv, n_keep)
    q64 = synth.bf16_bits_to_f32(prob.q).astype(np.float64)
    ang = _angles(nb)
    grp = hq // hkv
    for b in range(2):
        for k in range(nb):
            qt = _turn(q64[b], -ang[k])
            S = np.zeros((hkv, 128))
            for h in range(hq):
                tq = prob.t_q[h // grp].astype(np.float64)
                ref = qt[h] @ tq
                bound = (136 * U) * (np.abs(np.concatenate([np.abs(q64[b, h, :64]) + np.abs(q64[b, h, 64:])] * 2))
                                     @ np.abs(tq)) + 1e-30
                assert (np.abs(qp[b, k, h] - ref) <= bound).all()
                S[h // grp] += qp[b, k, h].astype(np.float64) ** 2
            for g in range(hkv):
                idx = sel[b, k, g]
                assert (np.diff(idx) > 0).all()
                order = sorted(range(128), key=lambda j: (-S[g, j], j))
                want, got = set(order[:n_keep]), set(idx.tolist())
                thr = S[g, order[n_keep - 1]]
                for j in got ^ want:
                    assert abs(S[g, j] - thr) <= 8 * U * thr * grp
    # masks really differ across buckets
    assert (sel[:, 0] != sel[:, 1]).any() or n_keep == 128


def _sdpa_rows(q, k, v, scale):
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k)
    vt = torch.from_numpy(v)
    logits = (qt * kt).sum(-1) * scale          # q is per token here
    return torch.softmax(logits, 0) @ vt, torch.logsumexp(logits, 0)


@pytest.mark.parametrize("n_keep", [77, 128])
def test_decode_is_one_softmax_over_per_bucket_scores(orc, n_keep):
    lens = [4100, 2049, 7]
    shape = synth.Shape(3, 8, 2, lens, n_keep, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=64)
    nb = synth.rope_buckets(max(lens))
    cs, sn = synth.make_rope_tables(nb)
    cache, _ = orc.quantize_append_rope(prob.k, prob.v, prob.t_k, cs, sn, prob.cu_tokens, prob.page_table,
                                        prob.num_pages)
    qp, sel = orc.select_channels_rope(prob.q, prob.t_q, cs, sn, 2, n_keep)
    out, lse = orc.decode_attn_rope(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    grp = 4
    for b, L in enumerate(lens):
        bk = np.arange(L) // BUCKET
        for g in range(2):
            kh, vh = cf.gather_seq(cache, prob.page_table, b, L, g)
            mask = np.zeros((nb, 128))
            for k in range(nb):
                mask[k, sel[b, k, g]] = 1.0
            for h in range(g * grp, (g + 1) * grp):
                qtok = qp[b, bk, h].astype(np.float64) * mask[bk]
                o, l = _sdpa_rows(qtok, kh.astype(np.float64), vh.astype(np.float64), prob.sm_scale)
                np.testing.assert_allclose(out[b, h], o.numpy(), rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(lse[b, h], l.item(), rtol=1e-12)


def test_equal_buckets_reduce_to_plain_decode(orc):
    lens = [4100, 300]
    shape = synth.Shape(2, 8, 2, lens, 77)
    prob = synth.make_problem(shape, seed=65)
    cache, _ = orc.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = orc.select_channels(prob.q, prob.t_q, 2, 77)
    nb = 3
    qr = np.repeat(qp[:, None], nb, axis=1)
    sr = np.repeat(sel[:, None], nb, axis=1)
    o1, l1 = orc.decode_attn(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    o2, l2 = orc.decode_attn_rope(cache, qr, sr, prob.page_table, prob.seq_lens, prob.sm_scale)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_rejects_tokens_past_the_buckets(orc):
    lens = [2049]
    shape = synth.Shape(1, 4, 1, lens, 77)
    prob = synth.make_problem(shape, seed=66)
    cs, sn = synth.make_rope_tables(1)
    with pytest.raises(ValueError):
        orc.key_transform_rope(prob.k, prob.t_k, prob.cu_tokens, cs, sn)
    cache, _ = orc.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = orc.select_channels_rope(prob.q, prob.t_q, cs, sn, 1, 77)
    with pytest.raises(ValueError):
        orc.decode_attn_rope(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
