"""Pins of the oracle's key transform, INT2 quantizer and cache packing."""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from tests import cachefmt as cf

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def ulp32(x):
    return np.spacing(np.abs(np.float32(x))).astype(np.float64)


# ----------------------------------------------------------------- golden page
def test_golden_page_bytes(orc):
    g = json.load(open(os.path.join(GOLD, "pack_page_small.json")))
    n = g["n_valid"]
    kp = np.zeros((n, 1, 128), dtype=np.float32)
    for ch, vals in g["kprime"].items():
        kp[:, 0, int(ch)] = np.array(vals, dtype=np.float32)
    v = np.zeros((n, 1, 128), dtype=np.float32)
    v[:, 0, :32] = np.arange(32) % 4
    vb = synth.f32_to_bf16_bits(v)
    cache = orc.pack_cache(kp, vb, [0, n], np.zeros((1, 1), np.int32), 1)
    e = g["expect"]
    np.testing.assert_array_equal(cache.k_ch0[0, 0, :n], e["k_ch0_bits"])
    assert not cache.k_ch0[0, 0, n:].any()
    for ch, row in e["k_rows"].items():
        j = int(ch)
        assert list(cache.k_rows(0)[0, j, :2]) == row["bytes01"], ch
        assert not cache.k_rows(0)[0, j, 2:].any()
        assert cache.k_meta_page(0)[0, j, 0] == row["scale_bits"], ch
        assert cache.k_meta_page(0)[0, j, 1] == row["zero_bits"], ch
    assert not cache.k_rows(0)[0, 0].any() and not cache.k_meta_page(0)[0, 0].any()
    # the other three slots of the page's block are untouched
    assert not cache.k_codes[0, 0, :, 1:].any() and not cache.k_meta[0, 0, :, 1:].any()
    for t in range(n):
        assert list(cache.v_codes[0, 0, t]) == e["v_token_bytes"]
        assert list(cache.v_meta[0, 0, 0, :, t]) == e["v_scale_bits"]
        assert list(cache.v_meta[0, 0, 1, :, t]) == e["v_zero_bits"]
    assert not cache.v_codes[0, 0, n:].any() and not cache.v_meta[0, 0, :, :, n:].any()


# ----------------------------------------------------------------- quantizer
def _groups(rng, n_groups, size):
    out = []
    for i in range(n_groups):
        kind = i % 5
        if kind == 0:
            x = rng.standard_normal(size)
        elif kind == 1:
            x = rng.uniform(-1, 1, size) * 10.0 ** rng.integers(-6, 4)
        elif kind == 2:
            x = rng.standard_normal(size) * 0.01 + rng.uniform(-50, 50)   # large offset, small spread
        elif kind == 3:
            x = np.full(size, rng.standard_normal())                        # constant
        else:
            x = rng.integers(-3, 4, size).astype(np.float64) * 0.5           # exactly on levels/thresholds
        out.append(x.astype(np.float32))
    return out


@pytest.mark.parametrize("size", [1, 2, 32, 128])
def test_quantizer_nearest_level_and_bounds(orc, size):
    rng = np.random.default_rng(10 + size)
    for x in _groups(rng, 120, size):
        sb, zb, codes = orc.quantize_group(x)
        s, z = orc.f16_value(sb), orc.f16_value(zb)
        mn, mx = float(x.min()), float(x.max())
        # z is the binary16 round-down of the minimum, s >= (max - z)/3 up to fp32 rounding
        assert z <= mn and (mn - z) < max(2 ** -24, abs(mn) * 2 ** -10) * 1.0000001
        assert 3 * s >= (mx - z) * (1 - 2 ** -23)
        assert codes.max() <= 3
        levels = z + s * np.arange(4)                       # exact in fp64
        for xi, c in zip(x.astype(np.float64), codes):
            dist = np.abs(xi - levels)
            best = np.flatnonzero(dist == dist.min()).max()   # ties to the upper level
            if best != c:
                # only allowed where x is within fp32 rounding of the midpoint
                mid = z + (min(best, c) + 0.5) * s
                assert abs(xi - mid) <= 2 * ulp32(max(abs(mid), abs(z) + 3 * s)), (xi, c, best, s, z)
            xh = orc.dequant(int(c), sb, zb)
            assert abs(xi - xh) <= s / 2 + 2 * ulp32(max(abs(xi), abs(z) + 3 * s))


def test_quantizer_error_statistics(orc):
    """Uniform-noise model of rounding error: mean squared error ~ s^2/12."""
    rng = np.random.default_rng(3)
    ratios = []
    for _ in range(400):
        x = rng.uniform(-2, 3, 128).astype(np.float32)
        sb, zb, codes = orc.quantize_group(x)
        s = orc.f16_value(sb)
        xh = np.array([orc.dequant(int(c), sb, zb) for c in codes])
        ratios.append(np.mean((x - xh) ** 2) / (s * s / 12))
    assert 0.85 < np.mean(ratios) < 1.15


# ----------------------------------------------------------------- key transform
def test_key_transform_matches_fp64_matmul(orc):
    shape = synth.Shape(1, 4, 2, [300], 77)
    prob = synth.make_problem(shape, seed=5)
    kp = orc.key_transform(prob.k, prob.t_k)
    k64 = synth.bf16_bits_to_f32(prob.k).astype(np.float64)
    t64 = synth.bf16_bits_to_f32(prob.t_k).astype(np.float64)
    ref = np.einsum("tgi,gij->tgj", k64, t64).astype(np.float32)
    diff = np.abs(kp.astype(np.float64) - ref.astype(np.float64))
    assert (diff <= ulp32(ref)).all()
    assert (diff == 0).mean() > 0.999


def test_dual_transform_preserves_dot_products(orc):
    """(q T_Q)(k T_K)^T = q k^T when T_Q = T_K^{-T} (Eq. 1 of §3.1): checked
    through the oracle's own q' (select) and k' (key transform) against the
    closed-form rounding bound."""
    shape = synth.Shape(2, 8, 2, [64, 64], 128)
    prob = synth.make_problem(shape, seed=6)
    qp, _ = orc.select_channels(prob.q, prob.t_q, shape.hkv, 128)
    kp = orc.key_transform(prob.k, prob.t_k)
    q64 = synth.bf16_bits_to_f32(prob.q).astype(np.float64)
    k64 = synth.bf16_bits_to_f32(prob.k).astype(np.float64)
    tq = prob.t_q.astype(np.float64)
    tk = synth.bf16_bits_to_f32(prob.t_k).astype(np.float64)
    n, u = 128, 2.0 ** -24
    gam = n * u / (1 - n * u)
    grp = shape.hq // shape.hkv
    for b in range(shape.batch):
        for h in range(shape.hq):
            g = h // grp
            kk = k64[prob.cu_tokens[b]:prob.cu_tokens[b + 1], g]
            kkp = kp[prob.cu_tokens[b]:prob.cu_tokens[b + 1], g].astype(np.float64)
            lhs = kkp @ qp[b, h].astype(np.float64)
            rhs = kk @ q64[b, h]
            # error of q' (fp32 chain), of k' (one rounding), of T_Q's fp32 storage, of the dot itself
            bound = (gam + 2 * u) * (np.abs(kk) @ (np.abs(tk[g]) @ (np.abs(tq[g]).T @ np.abs(q64[b, h])))) + 1e-9
            tq_err = np.abs(tq[g] - np.linalg.inv(tk[g]).T)
            bound += np.abs(kk) @ (np.abs(tk[g]) @ (tq_err.T @ np.abs(q64[b, h])))
            assert (np.abs(lhs - rhs) <= bound).all()


# ----------------------------------------------------------------- packing
def test_pack_layout_reads_back(orc):
    """An independent reader of the layout recovers every input within the
    grid's half step; channel 0 is the bf16 rounding of k'[:, 0]; slots past
    the sequence end are zero; ragged sequences in a shuffled pool."""
    shape = synth.Shape(3, 4, 2, [130, 128, 5], 77, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=7)
    cache, kp = orc.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    vf = synth.bf16_bits_to_f32(prob.v)
    for b in range(shape.batch):
        L = int(prob.seq_lens[b])
        s0 = int(prob.cu_tokens[b])
        for g in range(shape.hkv):
            kh, vh = cf.gather_seq(cache, prob.page_table, b, L, g)
            kref = kp[s0:s0 + L, g]
            ch0 = torch.from_numpy(kref[:, 0].copy()).to(torch.bfloat16).float().numpy()
            np.testing.assert_array_equal(kh[:, 0], ch0)
            for pi in range((L + 127) // 128):
                p = int(prob.page_table[b, pi])
                sl = slice(pi * 128, min(L, pi * 128 + 128))
                s = cf.f16(cache.k_meta_page(p)[g, 1:, 0])
                err = np.abs(kh[sl, 1:] - kref[sl, 1:])
                assert (err <= s / 2 + 4 * ulp32(np.abs(kref[sl, 1:]) + 3 * s)).all()
                nval = sl.stop - sl.start
                assert not cf.k_codes(cache, p, g)[:, nval:].any()
                assert not cache.v_codes[p, g, nval:].any()
                assert not cache.k_ch0[p, g, nval:].any()
            vs = cf.f16(np.stack([cache.v_meta[int(prob.page_table[b, t // 128]), g, 0, :, t % 128] for t in range(L)]))
            err = np.abs(vh - vf[s0:s0 + L, g])
            assert (err <= np.repeat(vs, 32, axis=1) / 2 + 4 * ulp32(np.abs(vf[s0:s0 + L, g]) + 3 * np.repeat(vs, 32, axis=1))).all()


def test_pack_is_page_permutation_equivariant(orc):
    shape = synth.Shape(2, 4, 2, [256, 200], 77)
    prob = synth.make_problem(shape, seed=8)
    kp = orc.key_transform(prob.k, prob.t_k)
    c1 = orc.pack_cache(kp, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    perm = np.random.default_rng(0).permutation(prob.num_pages).astype(np.int32)
    pt2 = np.where(prob.page_table >= 0, perm[np.maximum(prob.page_table, 0)], -1).astype(np.int32)
    c2 = orc.pack_cache(kp, prob.v, prob.cu_tokens, pt2, prob.num_pages)
    for a1, a2 in zip(c1.page_major(), c2.page_major()):
        np.testing.assert_array_equal(a1, a2[perm])
