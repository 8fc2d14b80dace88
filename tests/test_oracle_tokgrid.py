"""Pins of the oracle's per-token key grid (Dual-QK paper, §3.3: one
asymmetric INT2 grid per token and KV head over channels 1..127, channel 0
kept in bf16 outside the range)."""
import numpy as np
import pytest
import torch

import synth
from tests import cachefmt as cf


def ulp32(x):
    return np.spacing(np.abs(np.float32(x))).astype(np.float64)


def _build(orc, shape, seed):
    prob = synth.make_problem(shape, seed=seed)
    cache, kp = orc.quantize_append_tokgrid(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table,
                                            prob.num_pages)
    return prob, cache, kp


@pytest.mark.parametrize("lens", [[300, 5], [128, 129]])
def test_token_codes_are_the_nearest_levels_of_their_own_grid(orc, lens):
    shape = synth.Shape(len(lens), 8, 2, lens, 77, shuffle_pages=True)
    prob, cache, kp = _build(orc, shape, 40)
    for b, L in enumerate(lens):
        t0 = int(prob.cu_tokens[b])
        for pi in range((L + 127) // 128):
            p = int(prob.page_table[b, pi])
            nvalid = min(128, L - 128 * pi)
            for g in range(2):
                s, z = cf.k_token_meta(cache, p, g)
                codes = cf.k_codes(cache, p, g)                     # [ch][tok]
                assert not codes[0].any()                           # row 0 unused
                assert not codes[:, nvalid:].any() and not s[nvalid:].any() and not z[nvalid:].any()
                for t in range(nvalid):
                    x = kp[t0 + 128 * pi + t, g, 1:].astype(np.float64)
                    st, zt = float(s[t]), float(z[t])
                    mn, mx = x.min(), x.max()
                    assert zt <= mn and (mn - zt) < max(2 ** -24, abs(mn) * 2 ** -10) * 1.0000001
                    assert 3 * st >= (mx - zt) * (1 - 2 ** -23)
                    levels = zt + st * np.arange(4)
                    for xi, c in zip(x, codes[1:, t]):
                        dist = np.abs(xi - levels)
                        best = np.flatnonzero(dist == dist.min()).max()
                        if best != c:
                            mid = zt + (min(best, c) + 0.5) * st
                            assert abs(xi - mid) <= 2 * ulp32(max(abs(mid), abs(zt) + 3 * st))


def test_channel0_is_outside_the_token_range(orc):
    """Scaling channel 0 of k' by 1000 changes only the bf16 channel-0 copy:
    every token's grid and every code of channels 1..127 stay as they were."""
    shape = synth.Shape(1, 4, 1, [256], 77)
    prob = synth.make_problem(shape, seed=41)
    kp = orc.key_transform(prob.k, prob.t_k)
    a = orc.pack_cache_tokgrid(kp, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    kp2 = kp.copy()
    kp2[:, :, 0] *= 1000.0
    b = orc.pack_cache_tokgrid(kp2, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    for nm in ("k_codes", "k_meta", "v_codes", "v_meta"):
        np.testing.assert_array_equal(getattr(a, nm), getattr(b, nm))
    assert (a.k_ch0 != b.k_ch0).any()


def _sdpa(q, k, v, scale):
    qt = torch.from_numpy(np.ascontiguousarray(q, np.float64))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(v, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, :, 0, :].numpy()


@pytest.mark.parametrize("n_keep", [128, 77, 1])
@pytest.mark.parametrize("hq,hkv,lens", [(8, 8, [300, 5]), (32, 8, [129, 256]), (4, 1, [1000])])
def test_decode_is_library_attention_on_the_decoded_cache(orc, n_keep, hq, hkv, lens):
    shape = synth.Shape(len(lens), hq, hkv, lens, n_keep, shuffle_pages=True)
    prob, cache, _ = _build(orc, shape, 42)
    qp, sel = orc.select_channels(prob.q, prob.t_q, hkv, n_keep)
    out, lse = orc.decode_attn_tokgrid(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    grp = hq // hkv
    for b in range(shape.batch):
        for g in range(hkv):
            kh, vh = cf.gather_seq_tokgrid(cache, prob.page_table, b, int(prob.seq_lens[b]), g)
            mask = np.zeros(128)
            mask[sel[b, g]] = 1.0
            qm = qp[b, g * grp:(g + 1) * grp].astype(np.float64) * mask
            np.testing.assert_allclose(out[b, g * grp:(g + 1) * grp], _sdpa(qm, kh, vh, prob.sm_scale),
                                       rtol=1e-10, atol=1e-12)
            logits = (qm @ kh.astype(np.float64).T) * prob.sm_scale
            want = np.log(np.exp(logits - logits.max(1, keepdims=True)).sum(1)) + logits.max(1)
            np.testing.assert_allclose(lse[b, g * grp:(g + 1) * grp], want, rtol=1e-12)


@pytest.mark.parametrize("L", [1, 5, 129])
def test_decode_tiny_brute_force(orc, L):
    shape = synth.Shape(1, 4, 1, [L], 3)
    prob, cache, kp = _build(orc, shape, 43 + L)
    qp, sel = orc.select_channels(prob.q, prob.t_q, 1, 3)
    out, _ = orc.decode_attn_tokgrid(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    for h in range(4):
        logits = []
        for t in range(L):
            p, slot = int(prob.page_table[0, t // 128]), t % 128
            s, z = cf.k_token_meta(cache, p, 0)
            acc = 0.0
            for j in sel[0, 0]:
                if j == 0:
                    kv = float(cf.bf16(cache.k_ch0[p, 0, slot]))
                else:
                    c = (int(cache.k_codes[p >> 3, 0, j, p & 7, slot >> 2]) >> (2 * (slot & 3))) & 3
                    kv = float(np.float32(c) * s[slot] + z[slot])
                acc += float(qp[0, h, j]) * kv
            logits.append(acc * prob.sm_scale)
        w = np.exp(np.array(logits) - max(logits))
        w /= w.sum()
        _, vh = cf.gather_seq(cache, prob.page_table, 0, L, 0)
        np.testing.assert_allclose(out[0, h], w @ vh.astype(np.float64), rtol=1e-9, atol=1e-12)


def test_equal_ranges_reduce_to_the_per_channel_grid(orc):
    """When every token's channels 1..127 and every channel's tokens span the
    same values, the per-token and the per-channel grids coincide, so the two
    packs decode to the same keys and the two decodes agree exactly."""
    shape = synth.Shape(2, 8, 2, [256, 384], 77)
    prob = synth.make_problem(shape, seed=44)
    T = int(prob.cu_tokens[-1])
    vals = np.array([-1.5, 2.25, 0.125, 1.0], np.float32)
    t = np.arange(T)[:, None, None]
    j = np.arange(128)[None, None, :]
    kp = np.broadcast_to(vals[(t + 3 * j) % 4], (T, 2, 128)).astype(np.float32).copy()
    kp[:, :, 0] = np.random.default_rng(0).standard_normal((T, 2)).astype(np.float32)
    a = orc.pack_cache(kp, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    b = orc.pack_cache_tokgrid(kp, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    np.testing.assert_array_equal(a.k_codes, b.k_codes)
    qp, sel = orc.select_channels(prob.q, prob.t_q, 2, 77)
    oa, la = orc.decode_attn(a, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    ob, lb = orc.decode_attn_tokgrid(b, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)
    # and the metadata really is laid out differently
    assert (a.k_meta != b.k_meta).any()
