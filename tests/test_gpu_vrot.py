"""GPU parity of rotated values, clipped value grids and base-coordinate
selection: libdqk (through the C ABI) against the CPU oracle on the same
seeded inputs.  Bit-exact on q', selected indices and packed bytes (given the
GPU's own v' = v R_V); within the fp32 summation bound on v' and on the
inverse rotation; within 2e-3 max relative error per output row end to end."""
import numpy as np
import pytest
import torch

import oracle
import page_set_amd as pa
import synth
from tests import cachefmt as cf
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CLIP = 0.92
GAM = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)
NAMES = ["k_codes", "k_meta", "k_ch0", "v_codes", "v_meta"]


def _say(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------- selection
@pytest.mark.parametrize("B,hq,hkv,nk", [(4, 32, 8, 77), (1, 8, 8, 52), (3, 16, 2, 103), (2, 64, 1, 77),
                                         (2, 8, 8, 128), (4, 32, 8, 1), (2, 24, 2, 77)])
def test_select_base_bit_exact(B, hq, hkv, nk):
    _say("select base", B, hq, hkv, nk)
    shape = synth.Shape(B, hq, hkv, [128] * B, nk)
    prob = synth.make_problem(shape, seed=300 + hq + nk, materialize_kv=False)
    w = synth.make_selection_scales(hkv, seed=300 + nk)
    d = gu.upload(prob)
    qp, sel = pa.dqk_select_channels_base(d["q"], d["t_q"], gu.dev(w), hkv, nk)
    torch.cuda.synchronize()
    qp_ref, sel_ref = oracle.select_channels_base(prob.q, prob.t_q, w, hkv, nk)
    np.testing.assert_array_equal(gu.host(qp).view(np.uint32), qp_ref.view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel), sel_ref)


# ----------------------------------------------------------------- append
def _identity(hkv):
    return np.broadcast_to(synth.f32_to_bf16_bits(np.eye(128, dtype=np.float32)), (hkv, 128, 128)).copy()


def test_identity_rotation_without_clipping_is_the_plain_append():
    _say("vrot identity")
    shape = synth.Shape(3, 8, 2, [1153, 128, 77], 77, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=31)
    d = gu.upload(prob)
    c1 = pa.Cache(prob.num_pages, shape.hkv)
    c2 = pa.Cache(prob.num_pages, shape.hkv)
    vdbg = torch.full((prob.k.shape[0], shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    pa.dqk_quantize_append(c1, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"])
    pa.dqk_quantize_append_vrot(c2, d["k"], d["v"], d["t_k"], gu.dev(_identity(2)), 1.0, d["cu"], d["page_table"],
                                vprime_dbg=vdbg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.host(vdbg), synth.bf16_bits_to_f32(prob.v))
    for nm, a, b in zip(NAMES, gu.cache_to_host(c1).arrays(), gu.cache_to_host(c2).arrays()):
        np.testing.assert_array_equal(a, b, err_msg=nm)


def test_permutation_rotation_permutes_the_plain_value_codes():
    """R_V = a channel permutation inside each 32-channel group: bf16-exact, so
    v' is v with its channels moved and the GPU pack must hold the plain GPU
    pack's value codes moved the same way (same metadata, same keys)."""
    _say("vrot permutation")
    rng = np.random.default_rng(32)
    shape = synth.Shape(2, 32, 8, [700, 129], 77, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=32)
    perms = [np.concatenate([32 * q + rng.permutation(32) for q in range(4)]) for _ in range(8)]
    rv = np.zeros((8, 128, 128), np.float32)
    for g in range(8):
        rv[g, perms[g], np.arange(128)] = 1.0
    d = gu.upload(prob)
    c1 = pa.Cache(prob.num_pages, 8)
    c2 = pa.Cache(prob.num_pages, 8)
    pa.dqk_quantize_append(c1, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"])
    pa.dqk_quantize_append_vrot(c2, d["k"], d["v"], d["t_k"], gu.dev(synth.f32_to_bf16_bits(rv)), 1.0, d["cu"],
                                d["page_table"])
    torch.cuda.synchronize()
    plain, rot = gu.cache_to_host(c1), gu.cache_to_host(c2)
    for nm in ("k_codes", "k_meta", "k_ch0", "v_meta"):
        np.testing.assert_array_equal(getattr(plain, nm), getattr(rot, nm), err_msg=nm)
    for b in range(2):
        for pi in range((int(prob.seq_lens[b]) + 127) // 128):
            p = int(prob.page_table[b, pi])
            for g in range(8):
                np.testing.assert_array_equal(cf.v_codes(rot, p, g), cf.v_codes(plain, p, g)[:, perms[g]])


VROT_APPEND_CASES = [
    ("one-page-tail", synth.Shape(1, 8, 2, [5], 77)),
    ("ragged-shuffled", synth.Shape(4, 8, 2, [130, 128, 5, 257], 77, shuffle_pages=True)),
    ("cfg0-4k", synth.config_shape(0)),
    ("gqa-ragged", synth.Shape(2, 32, 8, [1000, 3000], 77, shuffle_pages=True)),
]


@pytest.mark.parametrize("name,shape", VROT_APPEND_CASES, ids=[c[0] for c in VROT_APPEND_CASES])
def test_append_vrot_stagewise(name, shape):
    _say("append vrot", name)
    prob = synth.make_problem(shape, seed=33)
    rv, _ = synth.make_value_rotation(shape.hkv, seed=33)
    d = gu.upload(prob)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    plain = pa.Cache(prob.num_pages, shape.hkv)
    T = prob.k.shape[0]
    kdbg = torch.full((T, shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    vdbg = torch.full((T, shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    pa.dqk_quantize_append_vrot(cache, d["k"], d["v"], d["t_k"], gu.dev(rv), CLIP, d["cu"], d["page_table"],
                                kprime_dbg=kdbg, vprime_dbg=vdbg)
    pa.dqk_quantize_append(plain, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"])
    torch.cuda.synchronize()
    got = gu.cache_to_host(cache)
    kp_gpu, vp_gpu = gu.host(kdbg), gu.host(vdbg)
    # (1) v' from MFMA within the recursive-summation bound of the exact sum
    vp_ref = oracle.value_transform(prob.v, rv)
    v64 = np.abs(synth.bf16_bits_to_f32(prob.v).astype(np.float64))
    r64 = np.abs(synth.bf16_bits_to_f32(rv).astype(np.float64))
    absdot = np.einsum("tgi,gij->tgj", v64, r64)
    assert np.isfinite(vp_gpu).all() and np.isfinite(kp_gpu).all()
    err = np.abs(vp_gpu.astype(np.float64) - vp_ref.astype(np.float64))
    assert (err <= GAM * absdot + np.spacing(np.abs(vp_ref))).all()
    # (2) keys are those of the plain append; the whole pack is bit-exact given the GPU's own v'
    for nm in ("k_codes", "k_meta", "k_ch0"):
        np.testing.assert_array_equal(getattr(got, nm), getattr(gu.cache_to_host(plain), nm), err_msg=nm)
    want = oracle.pack_cache_vrot(kp_gpu, vp_gpu, CLIP, prob.cu_tokens, prob.page_table, prob.num_pages)
    for nm, a, b in zip(NAMES, got.arrays(), want.arrays()):
        np.testing.assert_array_equal(a, b, err_msg=nm)
    # (3) end to end against the oracle's own v': value codes differ only by one
    # level where v' sits within rounding of a threshold, metadata only where a
    # clipped extreme sits within rounding of a binary16 boundary
    kp_ref = oracle.key_transform(prob.k, prob.t_k)
    e2e = oracle.pack_cache_vrot(kp_ref, vp_ref, CLIP, prob.cu_tokens, prob.page_table, prob.num_pages)
    cg = cf.unpack_rows(got.v_codes).astype(int)
    ce = cf.unpack_rows(e2e.v_codes).astype(int)
    n_diff = int((cg != ce).sum())
    n_meta = int((got.v_meta != e2e.v_meta).sum())
    _say(f"  end-to-end value code mismatches: {n_diff} of {cg.size}; meta mismatches: {n_meta}")
    assert np.abs(cg - ce).max() <= 1
    assert n_diff <= max(8, 1e-4 * cg.size)
    assert n_meta <= max(8, 1e-3 * got.v_meta.size)


# ----------------------------------------------------------------- unrotation
@pytest.mark.parametrize("B,hq,hkv", [(4, 32, 8), (1, 8, 8), (3, 16, 2), (2, 64, 1), (2, 24, 2)])
def test_value_unrotate_within_the_summation_bound(B, hq, hkv):
    _say("unrotate", B, hq, hkv)
    rng = np.random.default_rng(B * hq + hkv)
    _, rinv = synth.make_value_rotation(hkv, seed=34)
    o = rng.standard_normal((B, hq, 128)).astype(np.float32)
    o[0, 0] *= 1e-3
    t = gu.dev(o)
    res = pa.dqk_value_unrotate(t, gu.dev(rinv), hkv)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.host(t), o)  # the input is left as it was
    got = gu.host(res).astype(np.float64)
    want = oracle.value_unrotate(o.astype(np.float64), rinv, hkv)
    grp = hq // hkv
    for h in range(hq):
        bound = GAM * (np.abs(o[:, h].astype(np.float64)) @ np.abs(rinv[h // grp].astype(np.float64)))
        assert (np.abs(got[:, h] - want[:, h]) <= bound + 1e-30).all(), h


# ----------------------------------------------------------------- end to end
E2E_CASES = [
    ("gqa-ragged", synth.Shape(2, 32, 8, [6000, 301], 77, shuffle_pages=True)),
    ("cfg0", synth.config_shape(0)),
    ("nk128", synth.Shape(1, 32, 8, [2500], 128)),
    ("g2-nk52", synth.Shape(2, 16, 8, [900, 1300], 52)),
]


@pytest.mark.parametrize("name,shape", E2E_CASES, ids=[c[0] for c in E2E_CASES])
def test_rotated_path_end_to_end(name, shape):
    """GPU: rotated append, base selection, decode, inverse rotation; oracle:
    the same steps on the GPU-built cache bytes (decode parity isolated from
    v' rounding)."""
    _say("vrot end to end", name)
    prob = synth.make_problem(shape, seed=35)
    rv, rinv = synth.make_value_rotation(shape.hkv, seed=35)
    w = synth.make_selection_scales(shape.hkv, seed=35)
    d = gu.upload(prob)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    pa.dqk_quantize_append_vrot(cache, d["k"], d["v"], d["t_k"], gu.dev(rv), CLIP, d["cu"], d["page_table"])
    qp, sel = pa.dqk_select_channels_base(d["q"], d["t_q"], gu.dev(w), shape.hkv, shape.n_keep)
    o_rot, lse = pa.dqk_decode_attn(cache, qp, sel, d["page_table"], d["seq_lens"], prob.sm_scale)
    out = pa.dqk_value_unrotate(o_rot, gu.dev(rinv), shape.hkv)
    torch.cuda.synchronize()
    host_cache = gu.cache_to_host(cache)
    qp_ref, sel_ref = oracle.select_channels_base(prob.q, prob.t_q, w, shape.hkv, shape.n_keep)
    np.testing.assert_array_equal(gu.host(sel), sel_ref)
    o_rot, _ = oracle.decode_attn(host_cache, qp_ref, sel_ref, prob.page_table, prob.seq_lens, prob.sm_scale)
    ref = oracle.value_unrotate(o_rot, rinv, shape.hkv)
    e = gu.row_rel_err(gu.host(out), ref)
    _say(f"  max row rel err {e.max():.3e}")
    assert e.max() <= gu.TOL


ONE_CALL_CASES = [
    ("g4-nk77", synth.Shape(2, 32, 8, [3000, 701], 77, shuffle_pages=True), 0),
    ("g4-nk128-3splits", synth.Shape(1, 32, 8, [2000], 128), 3),
    ("g4-nk9", synth.Shape(2, 32, 8, [900, 300], 9), 0),      # n_keep < 17: the selection is a launch of its own
    ("g2", synth.Shape(2, 16, 8, [1200, 600], 77), 0),       # group 2: the same
]


@pytest.mark.parametrize("name,shape,ns", ONE_CALL_CASES, ids=[c[0] for c in ONE_CALL_CASES])
def test_one_call_equals_three_calls(name, shape, ns):
    """dqk_select_decode_attn_vrot (the selection in the decode launch where
    possible, the inverse rotation in the merge) gives bit for bit the
    results of dqk_select_channels_base + dqk_decode_attn +
    dqk_value_unrotate, and stays within 2e-3 of the oracle."""
    _say("vrot one call", name)
    prob = synth.make_problem(shape, seed=36)
    rv, rinv = synth.make_value_rotation(shape.hkv, seed=36)
    w = synth.make_selection_scales(shape.hkv, seed=36)
    d = gu.upload(prob)
    w_d, rinv_d = gu.dev(w), gu.dev(rinv)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    pa.dqk_quantize_append_vrot(cache, d["k"], d["v"], d["t_k"], gu.dev(rv), CLIP, d["cu"], d["page_table"])
    out1, lse1, qp1, sel1 = pa.dqk_select_decode_attn_vrot(cache, d["q"], d["t_q"], w_d, rinv_d, shape.n_keep,
                                                           d["page_table"], d["seq_lens"], prob.sm_scale,
                                                           num_splits=ns)
    qp2, sel2 = pa.dqk_select_channels_base(d["q"], d["t_q"], w_d, shape.hkv, shape.n_keep)
    o_rot, lse2 = pa.dqk_decode_attn(cache, qp2, sel2, d["page_table"], d["seq_lens"], prob.sm_scale, num_splits=ns)
    out2 = pa.dqk_value_unrotate(o_rot, rinv_d, shape.hkv)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.host(qp1).view(np.uint32), gu.host(qp2).view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel1), gu.host(sel2))
    np.testing.assert_array_equal(gu.host(out1).view(np.uint32), gu.host(out2).view(np.uint32))
    np.testing.assert_array_equal(gu.host(lse1).view(np.uint32), gu.host(lse2).view(np.uint32))
    qp_ref, sel_ref = oracle.select_channels_base(prob.q, prob.t_q, w, shape.hkv, shape.n_keep)
    np.testing.assert_array_equal(gu.host(sel1), sel_ref)
    o_ref, _ = oracle.decode_attn(gu.cache_to_host(cache), qp_ref, sel_ref, prob.page_table, prob.seq_lens,
                                  prob.sm_scale)
    e = gu.row_rel_err(gu.host(out1), oracle.value_unrotate(o_ref, rinv, shape.hkv))
    _say(f"  max row rel err {e.max():.3e}")
    assert e.max() <= gu.TOL
