"""GPU parity of the per-token key grid layout (Dual-QK paper, §3.3: one
INT2 grid per token and KV head over channels 1..127, channel 0 in bf16
outside the range): libdqk through the C ABI against the CPU oracle on the
same seeded inputs.  Packing bit-exact given the GPU's own k'; decode within
2e-3 per row on the same cache bytes, lse within its derived bound, split
counts within the derived bound."""
import numpy as np
import pytest
import torch

import oracle
import page_set_amd as pa
import synth
from tests import cachefmt as cf
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GAM = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)
NAMES = ["k_codes", "k_meta", "k_ch0", "v_codes", "v_meta"]


def _say(*a):
    print(*a, flush=True)


APPEND_CASES = [
    ("one-page-tail", synth.Shape(1, 8, 2, [5], 77)),
    ("ragged-shuffled", synth.Shape(4, 8, 2, [130, 128, 5, 257], 77, shuffle_pages=True)),
    ("cfg0-4k", synth.config_shape(0)),
    ("gqa-ragged", synth.Shape(2, 32, 8, [1000, 3000], 77, shuffle_pages=True)),
]


@pytest.mark.parametrize("name,shape", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_tokgrid_stagewise(name, shape):
    _say("append tokgrid", name)
    prob = synth.make_problem(shape, seed=50)
    d = gu.upload(prob)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    plain = pa.Cache(prob.num_pages, shape.hkv)
    kdbg = torch.full((prob.k.shape[0], shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    pa.dqk_quantize_append_tokgrid(cache, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"], kprime_dbg=kdbg)
    pa.dqk_quantize_append(plain, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"])
    torch.cuda.synchronize()
    got = gu.cache_to_host(cache)
    kp_gpu = gu.host(kdbg)
    # (1) k' within the recursive-summation bound of the exact sum
    kp_ref = oracle.key_transform(prob.k, prob.t_k)
    k64 = np.abs(synth.bf16_bits_to_f32(prob.k).astype(np.float64))
    t64 = np.abs(synth.bf16_bits_to_f32(prob.t_k).astype(np.float64))
    assert np.isfinite(kp_gpu).all()
    err = np.abs(kp_gpu.astype(np.float64) - kp_ref.astype(np.float64))
    assert (err <= GAM * np.einsum("tgi,gij->tgj", k64, t64) + np.spacing(np.abs(kp_ref))).all()
    # (2) bit-exact against the oracle's pack of the GPU's own k'; values as the plain append
    want = oracle.pack_cache_tokgrid(kp_gpu, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    for nm, a, b in zip(NAMES, got.arrays(), want.arrays()):
        np.testing.assert_array_equal(a, b, err_msg=nm)
    pl = gu.cache_to_host(plain)
    np.testing.assert_array_equal(got.v_codes, pl.v_codes)
    np.testing.assert_array_equal(got.v_meta, pl.v_meta)
    np.testing.assert_array_equal(got.k_ch0, pl.k_ch0)
    # (3) end to end against the oracle's own k': codes differ by at most one level, rarely
    e2e = oracle.pack_cache_tokgrid(kp_ref, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    cg = cf.unpack_rows(got.k_codes).astype(int)
    ce = cf.unpack_rows(e2e.k_codes).astype(int)
    n_diff = int((cg != ce).sum())
    _say(f"  end-to-end key code mismatches: {n_diff} of {cg.size}; meta mismatches: "
         f"{int((got.k_meta != e2e.k_meta).sum())}")
    assert np.abs(cg - ce).max() <= 1
    assert n_diff <= max(8, 1e-4 * cg.size)


def _decode_case(shape, seed, num_splits=0):
    prob = synth.make_problem(shape, seed=seed)
    cache, _ = oracle.quantize_append_tokgrid(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table,
                                              prob.num_pages)
    qp, sel = oracle.select_channels(prob.q, prob.t_q, shape.hkv, shape.n_keep)
    ref, ref_lse = oracle.decode_attn_tokgrid(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    gc = gu.cache_to_device(cache)
    out, lse = pa.dqk_decode_attn(gc, gu.dev(qp), gu.dev(sel), gu.dev(prob.page_table), gu.dev(prob.seq_lens),
                                  prob.sm_scale, num_splits=num_splits, token_grid=True)
    torch.cuda.synchronize()
    return prob, cache, qp, sel, ref, ref_lse, gu.host(out), gu.host(lse)


DECODE_CASES = [
    ("cfg0", synth.config_shape(0)),
    ("ctx1", synth.Shape(1, 8, 2, [1], 77)),
    ("ctx128-129", synth.Shape(2, 32, 8, [128, 129], 77)),
    ("ragged", synth.Shape(3, 32, 8, [5000, 300, 77], 77, shuffle_pages=True)),
    ("nk128", synth.Shape(2, 32, 8, [2000, 700], 128)),
    ("nk52", synth.Shape(1, 32, 8, [3000], 52)),
    ("nk1", synth.Shape(1, 32, 8, [1500], 1)),
    ("g2", synth.Shape(2, 16, 8, [900, 1300], 77)),
    ("g8", synth.Shape(1, 16, 2, [2100], 77)),
]


@pytest.mark.parametrize("name,shape", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_tokgrid_parity(name, shape):
    _say("decode tokgrid", name)
    prob, cache, qp, sel, ref, ref_lse, out, lse = _decode_case(shape, seed=51)
    rel = gu.row_rel_err(out, ref)
    _say(f"  max row rel err {rel.max():.3e}")
    assert (rel <= gu.TOL).all(), rel.max()
    gu.assert_lse(lse, ref_lse, gu.lse_bound(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale, ref_lse,
                                             gather=cf.gather_seq_tokgrid))


def test_decode_tokgrid_split_invariance():
    _say("decode tokgrid splits")
    shape = synth.Shape(2, 32, 8, [4000, 2500], 77)
    outs = []
    for ns in (1, 3, 0):
        prob, cache, qp, sel, ref, ref_lse, out, lse = _decode_case(shape, 52, num_splits=ns)
        outs.append(out)
        assert (gu.row_rel_err(out, ref) <= gu.TOL).all()
    bound = gu.split_bound(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale,
                           gather=cf.gather_seq_tokgrid)
    for o in outs[1:]:
        diff = np.abs(o.astype(np.float64) - outs[0])
        _say(f"  split difference / derived bound: max {(diff / bound).max():.3f}")
        assert (diff <= bound).all()


def test_gpu_built_tokgrid_cache_end_to_end():
    """GPU append (per-token grids), selection and decode against the oracle
    on the GPU-built cache bytes."""
    _say("tokgrid end to end")
    shape = synth.Shape(2, 32, 8, [6000, 301], 77, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=53)
    d = gu.upload(prob)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    pa.dqk_quantize_append_tokgrid(cache, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"])
    qp, sel = pa.dqk_select_channels(d["q"], d["t_q"], shape.hkv, shape.n_keep)
    out, _ = pa.dqk_decode_attn(cache, qp, sel, d["page_table"], d["seq_lens"], prob.sm_scale, token_grid=True)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_attn_tokgrid(gu.cache_to_host(cache), gu.host(qp), gu.host(sel), prob.page_table,
                                        prob.seq_lens, prob.sm_scale)
    e = gu.row_rel_err(gu.host(out), ref)
    _say(f"  max row rel err {e.max():.3e}")
    assert e.max() <= gu.TOL


@pytest.mark.parametrize("shape,ns", [(synth.Shape(2, 32, 8, [3000, 701], 77, shuffle_pages=True), 0),
                                      (synth.Shape(1, 32, 8, [2000], 128), 3),
                                      (synth.Shape(2, 32, 8, [900, 300], 9), 0),
                                      (synth.Shape(2, 16, 8, [1200, 600], 77), 0)],
                         ids=["g4-nk77", "g4-nk128-3splits", "g4-nk9", "g2"])
def test_one_call_equals_two_calls(shape, ns):
    """dqk_select_decode_attn_tokgrid (the selection in the decode launch
    where possible) gives bit for bit dqk_select_channels +
    dqk_decode_attn_tokgrid."""
    _say("tokgrid one call", shape.hq, shape.n_keep, ns)
    prob = synth.make_problem(shape, seed=54)
    d = gu.upload(prob)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    pa.dqk_quantize_append_tokgrid(cache, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"])
    out1, lse1, qp1, sel1 = pa.dqk_select_decode_attn(cache, d["q"], d["t_q"], shape.n_keep, d["page_table"],
                                                      d["seq_lens"], prob.sm_scale, num_splits=ns, token_grid=True)
    qp2, sel2 = pa.dqk_select_channels(d["q"], d["t_q"], shape.hkv, shape.n_keep)
    out2, lse2 = pa.dqk_decode_attn(cache, qp2, sel2, d["page_table"], d["seq_lens"], prob.sm_scale, num_splits=ns,
                                    token_grid=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.host(qp1).view(np.uint32), gu.host(qp2).view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel1), gu.host(sel2))
    np.testing.assert_array_equal(gu.host(out1).view(np.uint32), gu.host(out2).view(np.uint32))
    np.testing.assert_array_equal(gu.host(lse1).view(np.uint32), gu.host(lse2).view(np.uint32))
