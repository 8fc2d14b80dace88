"""GPU parity of bucket-relative RoPE (Dual-QK paper, §3.4 and App. C.4: keys
stored in the frame of their 2048-token bucket's anchor, a turned query and a
mask per bucket, one softmax over all buckets): libdqk through the C ABI
against the CPU oracle on the same seeded inputs.  Selection bit-exact; the
turned keys bit-exact (T_K = I), packing bit-exact given the GPU's own k';
decode within 2e-3 per row on the same cache bytes with lse within its
derived bound; the one-call path bit for bit the two calls."""
import numpy as np
import pytest
import torch

import oracle
import page_set_amd as pa
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GAM = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)
NAMES = ["k_codes", "k_meta", "k_ch0", "v_codes", "v_meta"]


def _say(*a):
    print(*a, flush=True)


def _tables(shape, extra=0):
    nb = synth.rope_buckets(max(shape.seq_lens)) + extra
    cs, sn = synth.make_rope_tables(nb)
    return nb, cs, sn


def _virtual(page_table, seq_lens, nb):
    """Page table and lengths of the (sequence, bucket) rows: row (b, k) holds
    positions 2048 k .. of sequence b (pages 16 k .. 16 k + 15)."""
    B, mp = page_table.shape
    vpt = np.zeros((B * nb, 16), np.int32)
    vl = np.zeros(B * nb, np.int32)
    for b in range(B):
        for k in range(nb):
            n = max(0, min(16, mp - 16 * k))
            vpt[b * nb + k, :n] = np.maximum(page_table[b, 16 * k:16 * k + n], 0)
            vl[b * nb + k] = max(0, min(2048, int(seq_lens[b]) - 2048 * k))
    return vpt, vl


def _lse_bound(cache, qp, sel, page_table, seq_lens, sm_scale, lse_ref):
    """The decode's lse bound (largest logit error over every token, each
    scored by its bucket's query), taken over the bucket rows."""
    B, nb, hq = qp.shape[:3]
    vpt, vl = _virtual(page_table, seq_lens, nb)
    live = np.flatnonzero(vl > 0)          # bucket rows that hold tokens
    per_row = np.zeros((B * nb, hq))
    per_row[live] = gu.lse_bound(cache, qp.reshape(B * nb, hq, 128)[live],
                                 sel.reshape(B * nb, *sel.shape[2:])[live], vpt[live], vl[live], sm_scale,
                                 np.zeros((len(live), hq)))
    return per_row.reshape(B, nb, hq).max(1) + 2.0 ** -20 * np.abs(lse_ref)


# ----------------------------------------------------------------- select
@pytest.mark.parametrize("B,hq,hkv,nk,nb", [(2, 32, 8, 77, 3), (1, 8, 8, 128, 2), (3, 16, 2, 52, 5),
                                            (1, 12, 4, 77, 2), (2, 64, 1, 9, 2), (4, 32, 8, 1, 64)])
def test_select_rope_bit_exact(B, hq, hkv, nk, nb):
    _say("select rope", B, hq, hkv, nk, nb)
    shape = synth.Shape(B, hq, hkv, [128] * B, nk)
    prob = synth.make_problem(shape, seed=70 + hq + nk, materialize_kv=False)
    cs, sn = synth.make_rope_tables(nb)
    d = gu.upload(prob)
    qp, sel = pa.dqk_select_channels_rope(d["q"], d["t_q"], gu.dev(cs), gu.dev(sn), hkv, nk)
    torch.cuda.synchronize()
    qp_ref, sel_ref = oracle.select_channels_rope(prob.q, prob.t_q, cs, sn, hkv, nk)
    np.testing.assert_array_equal(gu.host(qp).view(np.uint32), qp_ref.view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel), sel_ref)


# ----------------------------------------------------------------- append
APPEND_CASES = [
    ("one-page", synth.Shape(1, 8, 2, [5], 77)),
    ("three-buckets-ragged", synth.Shape(2, 8, 2, [5000, 300], 77, shuffle_pages=True)),
    ("bucket-edges", synth.Shape(3, 8, 2, [2048, 2049, 4096], 77, shuffle_pages=True)),
    ("cfg0-4k", synth.config_shape(0)),
]


@pytest.mark.parametrize("name,shape", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_rope_stagewise(name, shape):
    _say("append rope", name)
    prob = synth.make_problem(shape, seed=71)
    nb, cs, sn = _tables(shape)
    d = gu.upload(prob)
    T = prob.k.shape[0]
    # (1) T_K = I: k' is the turned key rounded to bf16, bit for bit
    eye = np.broadcast_to(synth.f32_to_bf16_bits(np.eye(128, dtype=np.float32)), (shape.hkv, 128, 128)).copy()
    c0 = pa.Cache(prob.num_pages, shape.hkv)
    kd0 = torch.full((T, shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    pa.dqk_quantize_append_rope(c0, d["k"], d["v"], gu.dev(eye), gu.dev(cs), gu.dev(sn), d["cu"], d["page_table"],
                                kprime_dbg=kd0)
    torch.cuda.synchronize()
    turned = oracle.key_transform_rope(prob.k, eye, prob.cu_tokens, cs, sn)
    np.testing.assert_array_equal(gu.host(kd0).view(np.uint32), turned.view(np.uint32))
    # (2) real T_K: k' within the summation bound of the exact product of the turned keys
    cache = pa.Cache(prob.num_pages, shape.hkv)
    kdbg = torch.full((T, shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    pa.dqk_quantize_append_rope(cache, d["k"], d["v"], d["t_k"], gu.dev(cs), gu.dev(sn), d["cu"], d["page_table"],
                                kprime_dbg=kdbg)
    torch.cuda.synchronize()
    kp_gpu = gu.host(kdbg)
    kp_ref = oracle.key_transform_rope(prob.k, prob.t_k, prob.cu_tokens, cs, sn)
    t64 = np.abs(synth.bf16_bits_to_f32(prob.t_k).astype(np.float64))
    absdot = np.einsum("tgi,gij->tgj", np.abs(turned.astype(np.float64)), t64)
    assert np.isfinite(kp_gpu).all()
    err = np.abs(kp_gpu.astype(np.float64) - kp_ref.astype(np.float64))
    assert (err <= GAM * absdot + np.spacing(np.abs(kp_ref))).all()
    # (3) the pack of the GPU's own k', byte for byte
    got = gu.cache_to_host(cache)
    want = oracle.pack_cache(kp_gpu, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    for nm, a, b in zip(NAMES, got.arrays(), want.arrays()):
        np.testing.assert_array_equal(a, b, err_msg=nm)


def test_append_rope_zero_angles_is_the_plain_append():
    _say("append rope zero angles")
    shape = synth.Shape(2, 32, 8, [3000, 700], 77, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=72)
    d = gu.upload(prob)
    nb = 2
    a = pa.Cache(prob.num_pages, shape.hkv)
    b = pa.Cache(prob.num_pages, shape.hkv)
    pa.dqk_quantize_append_rope(a, d["k"], d["v"], d["t_k"], gu.dev(np.ones((nb, 64), np.float32)),
                                gu.dev(np.zeros((nb, 64), np.float32)), d["cu"], d["page_table"])
    pa.dqk_quantize_append(b, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"])
    torch.cuda.synchronize()
    for nm, x, y in zip(NAMES, a.arrays(), b.arrays()):
        assert torch.equal(x, y), nm


# ----------------------------------------------------------------- decode
def _decode_case(shape, seed, num_splits=0, extra=0):
    prob = synth.make_problem(shape, seed=seed)
    nb, cs, sn = _tables(shape, extra)
    cache, _ = oracle.quantize_append_rope(prob.k, prob.v, prob.t_k, cs, sn, prob.cu_tokens, prob.page_table,
                                           prob.num_pages)
    qp, sel = oracle.select_channels_rope(prob.q, prob.t_q, cs, sn, shape.hkv, shape.n_keep)
    ref, ref_lse = oracle.decode_attn_rope(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    gc = gu.cache_to_device(cache)
    out, lse = pa.dqk_decode_attn_rope(gc, gu.dev(qp), gu.dev(sel), gu.dev(prob.page_table), gu.dev(prob.seq_lens),
                                       prob.sm_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return prob, cache, qp, sel, ref, ref_lse, gu.host(out), gu.host(lse)


DECODE_CASES = [
    ("cfg0", synth.config_shape(0), 0),
    ("ctx1", synth.Shape(1, 8, 2, [1], 77), 0),
    ("edges", synth.Shape(3, 32, 8, [2048, 2049, 4095], 77, shuffle_pages=True), 0),
    ("ragged", synth.Shape(3, 32, 8, [6000, 300, 77], 77, shuffle_pages=True), 0),
    ("spare-buckets", synth.Shape(2, 32, 8, [2500, 100], 77), 2),
    ("nk128", synth.Shape(2, 32, 8, [4200, 700], 128), 0),
    ("nk52", synth.Shape(1, 32, 8, [5000], 52), 0),
    ("nk1", synth.Shape(1, 32, 8, [3000], 1), 0),
    ("g2", synth.Shape(2, 16, 8, [2900, 1300], 77), 0),
    ("g8", synth.Shape(1, 16, 2, [4100], 77), 0),
    ("g1", synth.Shape(1, 8, 8, [2100], 77), 0),
]


@pytest.mark.parametrize("name,shape,extra", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_rope_parity(name, shape, extra):
    _say("decode rope", name)
    prob, cache, qp, sel, ref, ref_lse, out, lse = _decode_case(shape, 73, extra=extra)
    rel = gu.row_rel_err(out, ref)
    _say(f"  max row rel err {rel.max():.3e}")
    assert (rel <= gu.TOL).all(), rel.max()
    gu.assert_lse(lse, ref_lse, _lse_bound(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale, ref_lse))


@pytest.mark.parametrize("lens,nk,ns", [([5000, 2100], 77, 1), ([5000, 2100], 77, 2), ([5000, 2100], 77, 16),
                                       ([20000], 77, 1), ([20000], 90, 1), ([20000], 128, 1), ([20000], 110, 3)],
                         ids=["short-1", "short-2", "short-16", "20k-1", "20k-nk90-1", "20k-nk128-1", "20k-nk110-3"])
def test_decode_rope_split_counts(lens, nk, ns):
    """Every split holds whole buckets; a requested count too small for the
    kernel's bucket area (more than 8 buckets, or 4 to 5 for the larger n_keep)
    is raised, and any count gives the oracle's result."""
    _say("decode rope splits", lens, nk, ns)
    shape = synth.Shape(len(lens), 32, 8, lens, nk)
    prob, cache, qp, sel, ref, ref_lse, out, lse = _decode_case(shape, 74, num_splits=ns)
    rel = gu.row_rel_err(out, ref)
    _say(f"  max row rel err {rel.max():.3e}")
    assert (rel <= gu.TOL).all(), rel.max()


@pytest.mark.parametrize("shape,ns", [(synth.Shape(2, 32, 8, [5000, 701], 77, shuffle_pages=True), 0),
                                      (synth.Shape(1, 32, 8, [4100], 128), 2),
                                      (synth.Shape(2, 32, 8, [2100, 300], 9), 0),
                                      (synth.Shape(2, 16, 8, [2200, 600], 77), 0)],
                         ids=["g4-nk77", "g4-nk128-2splits", "g4-nk9", "g2"])
def test_one_call_equals_two_calls(shape, ns):
    """dqk_select_decode_attn_rope (the per-bucket selection launch, then the
    decode reading it) gives bit for bit dqk_select_channels_rope +
    dqk_decode_attn_rope, and that selection is the oracle's."""
    _say("rope one call", shape.hq, shape.n_keep, ns)
    prob = synth.make_problem(shape, seed=75)
    nb, cs, sn = _tables(shape)
    d = gu.upload(prob)
    dcs, dsn = gu.dev(cs), gu.dev(sn)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    pa.dqk_quantize_append_rope(cache, d["k"], d["v"], d["t_k"], dcs, dsn, d["cu"], d["page_table"])
    out1, lse1, qp1, sel1 = pa.dqk_select_decode_attn_rope(cache, d["q"], d["t_q"], dcs, dsn, shape.n_keep,
                                                           d["page_table"], d["seq_lens"], prob.sm_scale,
                                                           num_splits=ns)
    qp2, sel2 = pa.dqk_select_channels_rope(d["q"], d["t_q"], dcs, dsn, shape.hkv, shape.n_keep)
    out2, lse2 = pa.dqk_decode_attn_rope(cache, qp2, sel2, d["page_table"], d["seq_lens"], prob.sm_scale,
                                         num_splits=ns)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.host(qp1).view(np.uint32), gu.host(qp2).view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel1), gu.host(sel2))
    np.testing.assert_array_equal(gu.host(out1).view(np.uint32), gu.host(out2).view(np.uint32))
    np.testing.assert_array_equal(gu.host(lse1).view(np.uint32), gu.host(lse2).view(np.uint32))
    qp_ref, sel_ref = oracle.select_channels_rope(prob.q, prob.t_q, cs, sn, shape.hkv, shape.n_keep)
    np.testing.assert_array_equal(gu.host(qp1).view(np.uint32), qp_ref.view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel1), sel_ref)


def test_gpu_built_rope_cache_end_to_end():
    """GPU append, per-bucket selection and decode in one call against the
    oracle's decode of the GPU-built cache bytes."""
    _say("rope end to end")
    shape = synth.Shape(2, 32, 8, [9000, 2049], 77, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=76)
    nb, cs, sn = _tables(shape)
    d = gu.upload(prob)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    pa.dqk_quantize_append_rope(cache, d["k"], d["v"], d["t_k"], gu.dev(cs), gu.dev(sn), d["cu"], d["page_table"])
    out, lse, qp, sel = pa.dqk_select_decode_attn_rope(cache, d["q"], d["t_q"], gu.dev(cs), gu.dev(sn),
                                                       shape.n_keep, d["page_table"], d["seq_lens"], prob.sm_scale)
    torch.cuda.synchronize()
    host_cache = gu.cache_to_host(cache)
    ref, ref_lse = oracle.decode_attn_rope(host_cache, gu.host(qp), gu.host(sel), prob.page_table, prob.seq_lens,
                                           prob.sm_scale)
    e = gu.row_rel_err(gu.host(out), ref)
    _say(f"  max row rel err {e.max():.3e}")
    assert e.max() <= gu.TOL
    gu.assert_lse(gu.host(lse), ref_lse, _lse_bound(host_cache, gu.host(qp), gu.host(sel), prob.page_table,
                                                    prob.seq_lens, prob.sm_scale, ref_lse))
