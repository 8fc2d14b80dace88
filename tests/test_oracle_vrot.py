"""Pins of the oracle's value rotation, value clipping and base-coordinate
selection (Dual-QK paper: §3.3 values paragraph and diagonal refinement,
§3.4 inverse value rotation after aggregation, App. B.2 value quantization,
App. C.2 selection in base coordinates)."""
import numpy as np
import pytest
import torch

import synth
from tests import cachefmt as cf

CLIP = 0.92


def ulp32(x):
    return np.spacing(np.abs(np.float32(x))).astype(np.float64)


def _groups(rng, n_groups, size):
    out = []
    for i in range(n_groups):
        kind = i % 5
        if kind == 0:
            x = rng.standard_normal(size)
        elif kind == 1:
            x = rng.uniform(-1, 1, size) * 10.0 ** rng.integers(-6, 4)
        elif kind == 2:
            x = rng.standard_normal(size) * 0.01 + rng.uniform(-50, 50)
        elif kind == 3:
            x = rng.standard_normal(size) ** 3                      # heavy tails: clipping bites
        else:
            x = rng.integers(-3, 4, size).astype(np.float64) * 0.5
        out.append(x.astype(np.float32))
    return out


# ----------------------------------------------------------------- clipped grid
def test_clip_one_is_the_plain_quantizer(orc):
    rng = np.random.default_rng(1)
    for x in _groups(rng, 200, 32):
        a = orc.quantize_group(x)
        b = orc.quantize_group_clip(x, 1.0)
        assert a[0] == b[0] and a[1] == b[1]
        np.testing.assert_array_equal(a[2], b[2])


@pytest.mark.parametrize("size", [1, 32, 128])
def test_clipped_grid_covers_the_clipped_range_and_codes_are_nearest(orc, size):
    """The grid is fitted to [0.92 min, 0.92 max] (not to [min, max]); every
    value, inside the range or beyond it, takes the nearest of the four
    levels (ties up), so values past a clipped end saturate to code 0 or 3."""
    rng = np.random.default_rng(20 + size)
    saturated = 0
    for x in _groups(rng, 150, size):
        sb, zb, codes = orc.quantize_group_clip(x, CLIP)
        s, z = orc.f16_value(sb), orc.f16_value(zb)
        lo = float(np.float32(CLIP) * np.float32(x.min()))
        hi = float(np.float32(CLIP) * np.float32(x.max()))
        # z: binary16 at or below the clipped minimum, within one binary16 step
        assert z <= lo and (lo - z) < max(2 ** -24, abs(lo) * 2 ** -10) * 1.0000001
        # 3s reaches the clipped maximum and is the smallest binary16 that does (up to fp32 rounding)
        assert 3 * s >= (hi - z) * (1 - 2 ** -23)
        assert 3 * s <= (hi - z) * (1 + 2 ** -9) + 3 * 2 ** -24
        levels = z + s * np.arange(4)
        for xi, c in zip(x.astype(np.float64), codes):
            dist = np.abs(xi - levels)
            best = np.flatnonzero(dist == dist.min()).max()
            if best != c:
                mid = z + (min(best, c) + 0.5) * s
                assert abs(xi - mid) <= 2 * ulp32(max(abs(mid), abs(z) + 3 * s)), (xi, c, best, s, z)
            if xi < z or xi > z + 3 * s:
                saturated += 1
                assert c == (0 if xi < z else 3)
    assert saturated > 0


def test_clipping_lowers_the_error_of_gaussian_groups(orc):
    """Sanity (not a pin): on Gaussian 32-channel groups the clipped INT2 grid
    has a lower mean squared error than the full-range one."""
    rng = np.random.default_rng(4)
    err = {1.0: 0.0, CLIP: 0.0}
    for _ in range(300):
        x = rng.standard_normal(32).astype(np.float32)
        for clip in err:
            sb, zb, codes = orc.quantize_group_clip(x, clip)
            xh = np.array([orc.dequant(int(c), sb, zb) for c in codes])
            err[clip] += float(np.mean((x - xh) ** 2))
    assert err[CLIP] < err[1.0]


# ----------------------------------------------------------------- base selection
def test_unit_scales_are_plain_selection(orc):
    shape = synth.Shape(3, 32, 8, [128] * 3, 77)
    prob = synth.make_problem(shape, seed=2, materialize_kv=False)
    ones = np.ones((shape.hkv, 128), np.float32)
    for nk in (1, 52, 77, 128):
        qa, sa = orc.select_channels(prob.q, prob.t_q, shape.hkv, nk)
        qb, sb = orc.select_channels_base(prob.q, prob.t_q, ones, shape.hkv, nk)
        np.testing.assert_array_equal(qa, qb)
        np.testing.assert_array_equal(sa, sb)


@pytest.mark.parametrize("hq,hkv,n_keep", [(32, 8, 77), (8, 8, 52), (16, 2, 103)])
def test_base_selection_is_selection_with_the_base_transform(orc, hq, hkv, n_keep):
    """A_0 = A D^-1 formed explicitly (fp64, rounded to fp32) and used as the
    query transform of plain selection picks the same channels as selection
    on q' = q A weighted by 1/delta, except at near-ties; the returned q' is
    the scoring one, q A (App. C.2)."""
    shape = synth.Shape(4, hq, hkv, [128] * 4, n_keep)
    prob = synth.make_problem(shape, seed=3, materialize_kv=False)
    w = synth.make_selection_scales(hkv, seed=3)
    a0 = (prob.t_q.astype(np.float64) * w.astype(np.float64)[:, None, :]).astype(np.float32)
    qb, sb = orc.select_channels_base(prob.q, prob.t_q, w, hkv, n_keep)
    qa, _ = orc.select_channels(prob.q, prob.t_q, hkv, n_keep)
    np.testing.assert_array_equal(qb, qa)
    q0, s0 = orc.select_channels(prob.q, a0, hkv, n_keep)
    grp = hq // hkv
    q64 = synth.bf16_bits_to_f32(prob.q).astype(np.float64)
    mismatches = 0
    for b in range(shape.batch):
        for g in range(hkv):
            if set(sb[b, g]) == set(s0[b, g]):
                continue
            base = q64[b, g * grp:(g + 1) * grp] @ a0[g].astype(np.float64)
            e = (base ** 2).sum(0)
            kth = np.sort(e)[::-1][n_keep - 1]
            for j in set(sb[b, g]) ^ set(s0[b, g]):
                mismatches += 1
                assert abs(e[j] - kth) <= 1e-5 * kth, (b, g, j)
    assert mismatches <= 2


def test_base_selection_differs_from_plain_selection(orc):
    """The weights matter: with the refinement folded in, ranking on q' alone
    picks other channels for most (sequence, KV head) pairs."""
    shape = synth.Shape(4, 32, 8, [128] * 4, 77)
    prob = synth.make_problem(shape, seed=4, materialize_kv=False)
    w = synth.make_selection_scales(8, seed=4)
    _, sa = orc.select_channels(prob.q, prob.t_q, 8, 77)
    _, sb = orc.select_channels_base(prob.q, prob.t_q, w, 8, 77)
    differ = sum(set(sa[b, g]) != set(sb[b, g]) for b in range(4) for g in range(8))
    assert differ >= 24


# ----------------------------------------------------------------- rotated pack
def _identity_bf16(hkv):
    return np.broadcast_to(synth.f32_to_bf16_bits(np.eye(128, dtype=np.float32)), (hkv, 128, 128)).copy()


def _group_permutation(rng):
    """A channel permutation that keeps every 32-channel group in place."""
    perm = np.concatenate([32 * q + rng.permutation(32) for q in range(4)])
    return perm


def test_identity_rotation_without_clipping_is_the_plain_pack(orc):
    shape = synth.Shape(2, 8, 2, [300, 77], 77, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=7)
    plain, kp = orc.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    rot, kp2, vp = orc.quantize_append_vrot(prob.k, prob.v, prob.t_k, _identity_bf16(2), 1.0, prob.cu_tokens,
                                            prob.page_table, prob.num_pages)
    np.testing.assert_array_equal(vp, synth.bf16_bits_to_f32(prob.v))
    for a, b in zip(plain.arrays(), rot.arrays()):
        np.testing.assert_array_equal(a, b)


def test_permutation_rotation_permutes_value_codes(orc):
    """R_V = a permutation within 32-channel groups: v' = v R_V moves value
    channel perm[j] to channel j, so the rotated pack holds the plain pack's
    codes moved the same way, with the same group metadata; keys unchanged."""
    rng = np.random.default_rng(8)
    shape = synth.Shape(2, 8, 2, [256, 130], 77)
    prob = synth.make_problem(shape, seed=8)
    perms = [_group_permutation(rng) for _ in range(2)]
    rv = np.zeros((2, 128, 128), np.float32)
    for g in range(2):
        rv[g, perms[g], np.arange(128)] = 1.0
    plain, _ = orc.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    rot, _, vp = orc.quantize_append_vrot(prob.k, prob.v, prob.t_k, synth.f32_to_bf16_bits(rv), 1.0,
                                          prob.cu_tokens, prob.page_table, prob.num_pages)
    v = synth.bf16_bits_to_f32(prob.v)
    for g in range(2):
        np.testing.assert_array_equal(vp[:, g, :], v[:, g, perms[g]])
    for name in ("k_codes", "k_meta", "k_ch0", "v_meta"):
        np.testing.assert_array_equal(getattr(plain, name), getattr(rot, name))
    for p in range(prob.num_pages):
        for g in range(2):
            np.testing.assert_array_equal(cf.v_codes(rot, p, g), cf.v_codes(plain, p, g)[:, perms[g]])


def test_clipped_pack_uses_clipped_value_grids(orc):
    """Every (token, group) of the rotated pack equals the clipped quantizer
    run on that token's 32 rotated values; the keys are not clipped."""
    shape = synth.Shape(1, 4, 1, [200], 77)
    prob = synth.make_problem(shape, seed=9)
    rv, _ = synth.make_value_rotation(1, seed=9)
    rot, kp, vp = orc.quantize_append_vrot(prob.k, prob.v, prob.t_k, rv, CLIP, prob.cu_tokens, prob.page_table,
                                           prob.num_pages)
    plain, _ = orc.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    for name in ("k_codes", "k_meta", "k_ch0"):
        np.testing.assert_array_equal(getattr(plain, name), getattr(rot, name))
    for t in range(200):
        p, slot = int(prob.page_table[0, t // 128]), t % 128
        codes = cf.v_codes(rot, p, 0)[slot]
        for q in range(4):
            sb, zb, c = orc.quantize_group_clip(vp[t, 0, 32 * q:32 * q + 32], CLIP)
            assert rot.v_meta[p, 0, 0, q, slot] == sb and rot.v_meta[p, 0, 1, q, slot] == zb
            np.testing.assert_array_equal(codes[32 * q:32 * q + 32], c)


# ----------------------------------------------------------------- unrotation
def test_unrotate_inverts_the_rotation_per_kv_head(orc):
    """out = o R_V^-1 with KV head h // (hq/hkv)'s matrix: applied to o R_V it
    returns o (up to the fp32 storage of the inverse)."""
    rng = np.random.default_rng(10)
    rv, rinv = synth.make_value_rotation(2, seed=10)
    r = synth.bf16_bits_to_f32(rv).astype(np.float64)
    o = rng.standard_normal((3, 8, 128))
    rotated = np.stack([np.stack([o[b, h] @ r[h // 4] for h in range(8)]) for b in range(3)])
    back = orc.value_unrotate(rotated, rinv, 2)
    np.testing.assert_allclose(back, o, rtol=0, atol=1e-6 * np.abs(o).max())
    # the other KV head's inverse does not undo it
    swapped = orc.value_unrotate(rotated, rinv[::-1].copy(), 2)
    assert np.abs(swapped - o).max() > 0.1


def test_permutation_rotation_end_to_end_is_the_plain_decode(orc):
    """Rotate (a within-group permutation), pack, decode, unrotate with its
    inverse: the same output as the plain path, exactly."""
    rng = np.random.default_rng(11)
    shape = synth.Shape(2, 8, 2, [300, 129], 77, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=11)
    rv = np.zeros((2, 128, 128), np.float32)
    for g in range(2):
        rv[g, _group_permutation(rng), np.arange(128)] = 1.0
    rinv = np.ascontiguousarray(rv.transpose(0, 2, 1))
    plain, _ = orc.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    rot, _, _ = orc.quantize_append_vrot(prob.k, prob.v, prob.t_k, synth.f32_to_bf16_bits(rv), 1.0,
                                         prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = orc.select_channels(prob.q, prob.t_q, 2, 77)
    want, lw = orc.decode_attn(plain, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    o_rot, lr = orc.decode_attn(rot, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    got = orc.value_unrotate(o_rot, rinv, 2)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(lr, lw)


def test_rotated_decode_is_attention_over_unrotated_dequantized_values(orc):
    """n_keep = 128: decode + unrotate equals textbook softmax attention
    (torch's library routine, fp64) over (q', K^', V^' R_V^-1) decoded
    independently from the cache bytes."""
    shape = synth.Shape(1, 8, 2, [333], 128)
    prob = synth.make_problem(shape, seed=12)
    rv, rinv = synth.make_value_rotation(2, seed=12)
    cache, _, _ = orc.quantize_append_vrot(prob.k, prob.v, prob.t_k, rv, CLIP, prob.cu_tokens, prob.page_table,
                                           prob.num_pages)
    qp, sel = orc.select_channels(prob.q, prob.t_q, 2, 128)
    o_rot, _ = orc.decode_attn(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    got = orc.value_unrotate(o_rot, rinv, 2)
    for g in range(2):
        kh, vh = cf.gather_seq(cache, prob.page_table, 0, 333, g)
        vu = vh.astype(np.float64) @ rinv[g].astype(np.float64)
        qt = torch.from_numpy(qp[0, 4 * g:4 * g + 4].astype(np.float64))[None, :, None, :]
        kt = torch.from_numpy(kh.astype(np.float64))[None, None].expand(1, 4, -1, -1)
        vt = torch.from_numpy(vu)[None, None].expand(1, 4, -1, -1)
        want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=prob.sm_scale)[0, :, 0].numpy()
        np.testing.assert_allclose(got[0, 4 * g:4 * g + 4], want, rtol=1e-9, atol=1e-12)


def test_rotation_flattens_value_outliers(orc):
    """Sanity (not a pin): with a few large value channels, rotating before
    the INT2 grid (and rotating back) reconstructs values with a lower error
    than the plain per-group grid."""
    shape = synth.Shape(1, 4, 1, [256], 77)
    prob = synth.make_problem(shape, seed=13)
    v = synth.bf16_bits_to_f32(prob.v).copy()
    v[:, 0, [5, 40, 77]] *= 20.0
    vb = synth.f32_to_bf16_bits(v)
    rv, rinv = synth.make_value_rotation(1, seed=13)
    plain, _ = orc.quantize_append(prob.k, vb, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    rot, _, _ = orc.quantize_append_vrot(prob.k, vb, prob.t_k, rv, CLIP, prob.cu_tokens, prob.page_table,
                                         prob.num_pages)
    _, v_plain = cf.gather_seq(plain, prob.page_table, 0, 256, 0)
    _, v_rot = cf.gather_seq(rot, prob.page_table, 0, 256, 0)
    ref = synth.bf16_bits_to_f32(vb)[:, 0].astype(np.float64)
    e_plain = np.mean((v_plain - ref) ** 2)
    e_rot = np.mean((v_rot.astype(np.float64) @ rinv[0].astype(np.float64) - ref) ** 2)
    assert e_rot < e_plain
