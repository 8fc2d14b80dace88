"""GPU parity: libdqk (through the C ABI) against the CPU oracle on the same
seeded inputs.  Bit-exact on q', selected indices and packed bytes; within
2e-3 max relative error per output row on attention."""
import numpy as np
import pytest
import torch

import oracle
import page_set_amd as pa
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------- select
@pytest.mark.parametrize("B,hq,hkv,nk", [(1, 8, 8, 77), (1, 32, 8, 77), (4, 32, 8, 1), (4, 32, 8, 52),
                                         (4, 32, 8, 103), (4, 32, 8, 128), (3, 16, 2, 64), (2, 64, 1, 77),
                                         (2, 8, 8, 128), (16, 32, 8, 77)])
def test_select_bit_exact(B, hq, hkv, nk):
    _say("select", B, hq, hkv, nk)
    shape = synth.Shape(B, hq, hkv, [128] * B, nk)
    prob = synth.make_problem(shape, seed=100 + hq + nk, materialize_kv=False)
    d = gu.upload(prob)
    qp, sel = pa.dqk_select_channels(d["q"], d["t_q"], hkv, nk)
    torch.cuda.synchronize()
    qp_ref, sel_ref = oracle.select_channels(prob.q, prob.t_q, hkv, nk)
    np.testing.assert_array_equal(gu.host(qp).view(np.uint32), qp_ref.view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel), sel_ref)


# ----------------------------------------------------------------- append
APPEND_CASES = [
    ("one-page-tail", synth.Shape(1, 8, 2, [5], 77)),
    ("ragged-shuffled", synth.Shape(4, 8, 2, [130, 128, 5, 257], 77, shuffle_pages=True)),
    ("cfg0-4k", synth.config_shape(0)),
    ("gqa-ragged", synth.Shape(2, 32, 8, [1000, 3000], 77, shuffle_pages=True)),
]


@pytest.mark.parametrize("name,shape", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_stagewise(name, shape):
    _say("append", name)
    prob = synth.make_problem(shape, seed=7)
    d = gu.upload(prob)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    kdbg = torch.full((prob.k.shape[0], shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    pa.dqk_quantize_append(cache, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"], kprime_dbg=kdbg)
    torch.cuda.synchronize()
    got = gu.cache_to_host(cache)
    kp_gpu = gu.host(kdbg)
    # (1) k' from MFMA within the recursive-summation bound of the exact sum
    kp_ref = oracle.key_transform(prob.k, prob.t_k)
    k64 = synth.bf16_bits_to_f32(prob.k).astype(np.float64)
    t64 = np.abs(synth.bf16_bits_to_f32(prob.t_k).astype(np.float64))
    absdot = np.einsum("tgi,gij->tgj", np.abs(k64), t64)
    gam = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)
    err = np.abs(kp_gpu.astype(np.float64) - kp_ref.astype(np.float64))
    assert np.isfinite(kp_gpu).all()
    assert (err <= gam * absdot + np.spacing(np.abs(kp_ref))).all()
    # (2) packing is bit-exact given the GPU's own k'
    want = oracle.pack_cache(kp_gpu, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    for nm, a, b in zip(["k_codes", "k_meta", "k_ch0", "v_codes", "v_meta"], got.arrays(), want.arrays()):
        np.testing.assert_array_equal(a, b, err_msg=nm)
    # (3) end to end against the oracle's own k': values are bit-exact (no
    # transform); key codes differ only where k' sits within rounding of a
    # threshold or a group extremum
    e2e = oracle.pack_cache(kp_ref, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    np.testing.assert_array_equal(got.v_codes, e2e.v_codes)
    np.testing.assert_array_equal(got.v_meta, e2e.v_meta)
    from tests import cachefmt as cf
    cg = cf.unpack_rows(got.k_codes).astype(int)
    ce = cf.unpack_rows(e2e.k_codes).astype(int)
    n_diff = int((cg != ce).sum())
    _say(f"  end-to-end key code mismatches: {n_diff} of {cg.size}; meta mismatches: "
         f"{int((got.k_meta != e2e.k_meta).sum())}")
    assert np.abs(cg - ce).max() <= 1
    assert n_diff <= max(4, 1e-4 * cg.size)


@pytest.mark.parametrize("shape", [synth.Shape(3, 8, 2, [1153, 128, 77], 77, shuffle_pages=True),
                                   synth.Shape(1, 32, 8, [4100], 77)], ids=["ragged-runs", "gqa-4100"])
def test_append_without_readback_writes_the_same_cache(shape):
    """The k' readback is a build option of the append kernel: without it the
    cache bytes are identical (that build is the one used in production)."""
    _say("append without readback", shape.seq_lens)
    prob = synth.make_problem(shape, seed=9)
    d = gu.upload(prob)
    c1 = pa.Cache(prob.num_pages, shape.hkv)
    c2 = pa.Cache(prob.num_pages, shape.hkv)
    kdbg = torch.empty((prob.k.shape[0], shape.hkv, 128), dtype=torch.float32, device="cuda")
    pa.dqk_quantize_append(c1, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"], kprime_dbg=kdbg)
    pa.dqk_quantize_append(c2, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"])
    torch.cuda.synchronize()
    for nm, a, b in zip(["k_codes", "k_meta", "k_ch0", "v_codes", "v_meta"], gu.cache_to_host(c1).arrays(),
                        gu.cache_to_host(c2).arrays()):
        np.testing.assert_array_equal(a, b, err_msg=nm)


# ----------------------------------------------------------------- decode
def _decode_case(shape, seed, num_splits=0, cache_fn=None):
    prob = synth.make_problem(shape, seed=seed)
    cache, _ = oracle.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    if cache_fn:
        cache = cache_fn(cache, prob)
    qp, sel = oracle.select_channels(prob.q, prob.t_q, shape.hkv, shape.n_keep)
    ref, ref_lse = oracle.decode_attn(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    gc = gu.cache_to_device(cache)
    out, lse = pa.dqk_decode_attn(gc, gu.dev(qp), gu.dev(sel), gu.dev(prob.page_table), gu.dev(prob.seq_lens),
                                  prob.sm_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return prob, cache, qp, sel, ref, ref_lse, gu.host(out), gu.host(lse)


DECODE_CASES = [
    ("cfg0", synth.config_shape(0)),
    ("ctx1", synth.Shape(1, 8, 2, [1], 77)),
    ("ctx128-129", synth.Shape(2, 32, 8, [128, 129], 77)),
    ("ragged", synth.Shape(3, 32, 8, [5000, 300, 77], 77, shuffle_pages=True)),
    ("nk128", synth.Shape(2, 32, 8, [2000, 700], 128)),
    ("nk103", synth.Shape(1, 32, 8, [3000], 103)),
    ("nk52", synth.Shape(1, 32, 8, [3000], 52)),
    ("nk1", synth.Shape(1, 32, 8, [1500], 1)),
    ("mha-nk2", synth.Shape(1, 4, 1, [129], 2)),
    ("g2", synth.Shape(2, 16, 8, [900, 1300], 77)),
    ("g8", synth.Shape(1, 16, 2, [2100], 77)),
    ("g16", synth.Shape(1, 16, 1, [700], 64)),
    ("g3", synth.Shape(1, 6, 2, [1500], 77)),
    ("g6-ragged", synth.Shape(2, 24, 4, [600, 1100], 77, shuffle_pages=True)),
]


@pytest.mark.parametrize("name,shape", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_parity(name, shape):
    _say("decode", name)
    prob, cache, qp, sel, ref, ref_lse, out, lse = _decode_case(shape, seed=3)
    rel = gu.row_rel_err(out, ref)
    _say(f"  max row rel err {rel.max():.3e}")
    assert (rel <= gu.TOL).all(), rel.max()
    gu.assert_lse(lse, ref_lse, gu.lse_bound(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale,
                                             ref_lse))


def test_decode_config1_full():
    _say("decode config 1")
    prob, cache, qp, sel, ref, ref_lse, out, lse = _decode_case(synth.config_shape(1), seed=1)
    rel = gu.row_rel_err(out, ref)
    _say(f"  max row rel err {rel.max():.3e}")
    assert (rel <= gu.TOL).all()


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 8), (48, 4)], ids=["g4", "g2", "g12"])
def test_decode_split_invariance_and_permutation(hq, hkv):
    """Split count changes only rounding.  The MFMA decode rounds the
    probabilities and P * scale to binary16 relative to each split's running
    maximum: two split counts agree within the bound derived from those
    roundings (gpu_util.split_bound), element by element, for every group
    size (a group of 2 is one padded set of four heads, 12 three sets)."""
    _say("decode splits/permutation", hq, hkv)
    shape = synth.Shape(2, hq, hkv, [4000, 2500], 77)
    outs = []
    for ns in (1, 2, 7, 0):
        prob, cache, qp, sel, ref, ref_lse, out, lse = _decode_case(shape, 9, num_splits=ns)
        outs.append(out)
        assert (gu.row_rel_err(out, ref) <= gu.TOL).all()
    bound = gu.split_bound(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    for o in outs[1:]:
        diff = np.abs(o.astype(np.float64) - outs[0])
        _say(f"  split difference / derived bound: max {(diff / bound).max():.3f}")
        assert (diff <= bound).all()

    def permute(cache, prob):
        perm = np.random.default_rng(4).permutation(prob.num_pages)
        c2 = oracle.Cache(prob.num_pages, cache.hkv)
        moved = []
        for a in cache.page_major():
            b = np.empty_like(a)
            b[perm] = a
            moved.append(b)
        c2.set_page_major(*moved)
        prob.page_table = np.where(prob.page_table >= 0, perm[np.maximum(prob.page_table, 0)], -1).astype(np.int32)
        return c2

    _, _, _, _, _, _, out_p, _ = _decode_case(shape, 9, num_splits=0, cache_fn=permute)
    np.testing.assert_array_equal(out_p, outs[-1])


def test_decode_ignores_garbage_past_sequence_end():
    _say("decode garbage")
    shape = synth.Shape(2, 32, 8, [300, 1000], 77)

    def garbage(cache, prob):
        rng = np.random.default_rng(8)
        for b in range(2):
            L = int(prob.seq_lens[b])
            p = int(prob.page_table[b, (L - 1) // 128])
            s = L % 128
            if s:
                cache.v_codes[p, :, s:] = rng.integers(0, 256, cache.v_codes[p, :, s:].shape, dtype=np.uint8)
                cache.v_meta[p, :, :, :, s:] = rng.integers(0, 0x3C00, cache.v_meta[p, :, :, :, s:].shape).astype(np.uint16)
                cache.k_ch0[p, :, s:] = rng.integers(0, 0x4000, cache.k_ch0[p, :, s:].shape).astype(np.uint16)
                cache.k_rows(p)[:, :, (s + 3) // 4:] = rng.integers(0, 256, cache.k_rows(p)[:, :, (s + 3) // 4:].shape,
                                                                    dtype=np.uint8)
        return cache

    _, _, _, _, ref, _, out, _ = _decode_case(shape, 5)
    _, _, _, _, ref_g, _, out_g, _ = _decode_case(shape, 5, cache_fn=garbage)
    np.testing.assert_array_equal(ref, ref_g)
    np.testing.assert_array_equal(out, out_g)


# ----------------------------------------------------------------- bf16 baseline
@pytest.mark.parametrize("shape", [synth.Shape(2, 32, 8, [1000, 129], 128, shuffle_pages=True),
                                   synth.Shape(1, 8, 8, [700], 128)])
def test_decode_bf16_parity(shape):
    _say("decode bf16", shape.seq_lens)
    prob = synth.make_problem(shape, seed=12)
    kb, vb = oracle.paged_bf16(prob.k, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    ref, ref_lse = oracle.decode_bf16(kb, vb, prob.q, prob.page_table, prob.seq_lens, prob.sm_scale)
    out, lse = pa.dqk_decode_attn_bf16(gu.dev(kb), gu.dev(vb), gu.dev(prob.q), gu.dev(prob.page_table),
                                       gu.dev(prob.seq_lens), prob.sm_scale)
    torch.cuda.synchronize()
    assert (gu.row_rel_err(gu.host(out), ref) <= gu.TOL).all()
    np.testing.assert_allclose(gu.host(lse), ref_lse, rtol=1e-5, atol=1e-5)


FUSED_CASES = [
    ("nk77-ragged", synth.Shape(3, 32, 8, [5000, 131, 2800], 77, shuffle_pages=True), 0),
    ("nk52-splits7", synth.Shape(2, 32, 8, [4000, 129], 52), 7),
    ("nk103", synth.Shape(1, 32, 8, [3000], 103), 0),
    ("nk20", synth.Shape(1, 32, 8, [1700], 20), 3),
    ("nk10-two-calls", synth.Shape(1, 32, 8, [1700], 10), 0),
    ("nk128", synth.Shape(1, 32, 8, [900], 128), 0),
    ("nk113-ragged", synth.Shape(2, 32, 8, [2100, 77], 113, shuffle_pages=True), 5),
    ("g2-two-calls", synth.Shape(2, 16, 8, [900, 300], 77), 0),
]


@pytest.mark.parametrize("name,shape,ns", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_select_decode_one_call_equals_two_calls(name, shape, ns):
    """dqk_select_decode_attn (selection inside the decode kernel where it
    can, two launches otherwise) returns exactly what dqk_select_channels then
    dqk_decode_attn return, and its selection matches the oracle."""
    _say("select+decode", name)
    prob = synth.make_problem(shape, seed=31)
    cache, _ = oracle.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    gc = gu.cache_to_device(cache)
    d = gu.upload(prob)
    qp1, sel1 = pa.dqk_select_channels(d["q"], d["t_q"], shape.hkv, shape.n_keep)
    out1, lse1 = pa.dqk_decode_attn(gc, qp1, sel1, d["page_table"], d["seq_lens"], prob.sm_scale, num_splits=ns)
    out2, lse2, qp2, sel2 = pa.dqk_select_decode_attn(gc, d["q"], d["t_q"], shape.n_keep, d["page_table"],
                                                      d["seq_lens"], prob.sm_scale, num_splits=ns)
    torch.cuda.synchronize()
    qp_ref, sel_ref = oracle.select_channels(prob.q, prob.t_q, shape.hkv, shape.n_keep)
    np.testing.assert_array_equal(gu.host(sel2), sel_ref)
    np.testing.assert_array_equal(gu.host(qp2).view(np.uint32), qp_ref.view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel2), gu.host(sel1))
    np.testing.assert_array_equal(gu.host(out2), gu.host(out1))
    np.testing.assert_array_equal(gu.host(lse2), gu.host(lse1))
