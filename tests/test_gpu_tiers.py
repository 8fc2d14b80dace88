"""GPU parity of the protected BF16 tiers (Dual-QK §3.3, §3.4) through the C
ABI: the tiered prefill writes the INT2 pages the plain append writes for the
same token range, bit for bit; per-token appends reproduce the prefill bit for
bit; tier keys are within one bf16 ulp of the oracle's; the tiered decode is
within 2e-3 per row of the oracle on the same cache and tier bytes."""
import numpy as np
import pytest
import torch

import oracle
import page_set_amd as pa
import synth
from tests import cachefmt as cf
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def tiers_to_host(t: pa.Tiers) -> oracle.Tiers:
    h = oracle.Tiers(t.batch, t.num_kv_heads)
    for src, dst in zip(t.arrays(), h.arrays()):
        dst[...] = gu.host(src, np.uint16)
    return h


def _live_tail_slots(L):
    P = oracle.tier_pages(L)
    return [(t - 64) % 384 for t in range(64 + 128 * P, L)] if L > 64 else []


def _prefill(prob, shape):
    d = gu.upload(prob)
    cache = pa.Cache(prob.num_pages, shape.hkv)
    tiers = pa.Tiers(shape.batch, shape.hkv)
    pa.dqk_prefill_tiered(cache, tiers, d["k"], d["v"], d["t_k"], d["cu"], d["page_table"])
    return d, cache, tiers


PREFILL_CASES = [
    ("short", synth.Shape(3, 8, 2, [5, 64, 300], 77)),
    ("boundaries", synth.Shape(4, 8, 2, [319, 320, 447, 448], 77, shuffle_pages=True)),
    ("gqa", synth.Shape(2, 32, 8, [2500, 1100], 77, shuffle_pages=True)),
]


@pytest.mark.parametrize("name,shape", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_tiered(name, shape):
    _say("tiered prefill", name)
    prob = synth.make_problem(shape, seed=61)
    d, cache, tiers = _prefill(prob, shape)
    # the plain append of the shifted token ranges (tokens 64 .. 64 + 128 P of each sequence)
    P = [oracle.tier_pages(L) for L in shape.seq_lens]
    segs_k = [prob.k[prob.cu_tokens[b] + 64:prob.cu_tokens[b] + 64 + 128 * P[b]] for b in range(shape.batch)]
    segs_v = [prob.v[prob.cu_tokens[b] + 64:prob.cu_tokens[b] + 64 + 128 * P[b]] for b in range(shape.batch)]
    cu2 = np.concatenate([[0], np.cumsum([128 * p for p in P])]).astype(np.int32)
    ref = pa.Cache(prob.num_pages, shape.hkv)
    if cu2[-1] > 0:
        pa.dqk_quantize_append(ref, gu.dev(np.concatenate(segs_k)), gu.dev(np.concatenate(segs_v)), d["t_k"],
                               gu.dev(cu2), d["page_table"])
    torch.cuda.synchronize()
    got_c, ref_c = gu.cache_to_host(cache), gu.cache_to_host(ref)
    for nm, a, w in zip(["k_codes", "k_meta", "k_ch0", "v_codes", "v_meta"], got_c.arrays(), ref_c.arrays()):
        np.testing.assert_array_equal(a, w, err_msg=nm)
    # tier bytes against the oracle's prefill: copies exact, k' within one bf16 ulp
    want_c, want_t = oracle.prefill_tiered(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table,
                                           prob.num_pages)
    got_t = tiers_to_host(tiers)
    t64 = np.abs(synth.bf16_bits_to_f32(prob.t_k).astype(np.float64))
    gam = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)
    n_off = 0
    for b, L in enumerate(shape.seq_lens):
        ns = min(L, 64)
        live = _live_tail_slots(L)
        np.testing.assert_array_equal(got_t.sink_v[b, :, :ns], want_t.sink_v[b, :, :ns])
        np.testing.assert_array_equal(got_t.tail_v[b][:, live], want_t.tail_v[b][:, live])
        np.testing.assert_array_equal(got_t.tail_kraw[b][:, live], want_t.tail_kraw[b][:, live])
        toks = list(range(ns)) + [t for t in range(64 + 128 * P[b], L)] if L > 64 else list(range(ns))
        k64 = np.abs(synth.bf16_bits_to_f32(prob.k[prob.cu_tokens[b] + np.array(toks, int)]).astype(np.float64))
        absdot = np.einsum("tgi,gij->gtj", k64, t64)                  # [Hkv][n][128]
        a = np.concatenate([got_t.sink_k[b, :, :ns], got_t.tail_k[b][:, live]], axis=1)
        w = np.concatenate([want_t.sink_k[b, :, :ns], want_t.tail_k[b][:, live]], axis=1)
        af, wf = cf.bf16(a).astype(np.float64), cf.bf16(w).astype(np.float64)
        # both sides round an fp32 k' to bf16: the fp32 values differ by at most
        # gamma_128 sum |k_i T_ij| (an fp32 chain against a rounded fp64 sum), and
        # rounding adds at most one bf16 ulp (2^-7 of the larger magnitude)
        tol = 2 * gam * absdot + np.maximum(np.abs(af), np.abs(wf)) * 2.0 ** -7
        assert (np.abs(af - wf) <= tol).all()
        n_off += int((a != w).sum())
    _say(f"  tier keys off the oracle's bf16: {n_off}")


@pytest.mark.parametrize("L0,L1", [(0, 80), (400, 600), (1000, 1200)])
def test_append_token_reproduces_prefill(L0, L1):
    """Token-by-token appends from a prefill of L0 tokens to L1 tokens write
    the same INT2 pages and live tier slots as a prefill of L1 tokens."""
    _say("append token", L0, L1)
    shape = synth.Shape(2, 32, 8, [L1, L1 - 3], 77, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=67)
    d_full, want_cache, want_tiers = _prefill(prob, shape)
    starts = [min(L0, L) for L in shape.seq_lens]
    cache = pa.Cache(prob.num_pages, shape.hkv)
    tiers = pa.Tiers(shape.batch, shape.hkv)
    if sum(starts):
        ks = np.concatenate([prob.k[prob.cu_tokens[b]:prob.cu_tokens[b] + starts[b]] for b in range(2)])
        vs = np.concatenate([prob.v[prob.cu_tokens[b]:prob.cu_tokens[b] + starts[b]] for b in range(2)])
        cu = np.concatenate([[0], np.cumsum(starts)]).astype(np.int32)
        pa.dqk_prefill_tiered(cache, tiers, gu.dev(ks), gu.dev(vs), d_full["t_k"], gu.dev(cu),
                              d_full["page_table"])
    lens = np.array(starts, np.int32)
    final = np.array(shape.seq_lens, np.int32)
    kt, vt = gu.dev(prob.k), gu.dev(prob.v)
    cu_full = prob.cu_tokens
    while (lens < final).any():
        # a finished sequence rewrites its last token at its last position (same bytes, no new page)
        pos = np.where(lens < final, lens, lens - 1).astype(np.int32)
        idx = torch.from_numpy((cu_full[:2] + pos).astype(np.int64)).to("cuda")
        pa.dqk_append_token(cache, tiers, kt[idx].contiguous(), vt[idx].contiguous(), d_full["t_k"],
                            gu.dev(pos), d_full["page_table"])
        lens = np.minimum(lens + 1, final)
    torch.cuda.synchronize()
    for nm, a, w in zip(["k_codes", "k_meta", "k_ch0", "v_codes", "v_meta"], gu.cache_to_host(cache).arrays(),
                        gu.cache_to_host(want_cache).arrays()):
        np.testing.assert_array_equal(a, w, err_msg=nm)
    got_t, want_t = tiers_to_host(tiers), tiers_to_host(want_tiers)
    for b, L in enumerate(shape.seq_lens):
        ns = min(L, 64)
        live = _live_tail_slots(L)
        np.testing.assert_array_equal(got_t.sink_k[b, :, :ns], want_t.sink_k[b, :, :ns])
        np.testing.assert_array_equal(got_t.sink_v[b, :, :ns], want_t.sink_v[b, :, :ns])
        for a, w in zip((got_t.tail_k, got_t.tail_v, got_t.tail_kraw), (want_t.tail_k, want_t.tail_v,
                                                                         want_t.tail_kraw)):
            np.testing.assert_array_equal(a[b][:, live], w[b][:, live])


def _tier_lse_bound(cache, tiers, qp, sel, page_table, seq_lens, sm_scale, lse_ref):
    """Allowed |lse_gpu - lse_oracle|: every logit (INT2 tokens: >= 21-bit
    query-side operands; BF16 tokens: an fp32 fma chain over 128 channels) is
    within 2^-16 of the sum of the absolute values of its terms; the lse is a
    weighted mean of logits plus the fp32 exp/log and merge roundings."""
    B, hq = qp.shape[0], qp.shape[1]
    hkv = sel.shape[1]
    grp = hq // hkv
    out = np.zeros((B, hq))
    for b in range(B):
        L = int(seq_lens[b])
        P = oracle.tier_pages(L)
        for g in range(hkv):
            rows = [cf.bf16(tiers.sink_k[b, g, t]) for t in range(min(L, 64))]
            rows += [cf.bf16(tiers.tail_k[b, g, (t - 64) % 384]) for t in range(64 + 128 * P, L)] if L > 64 else []
            k = np.array(rows, np.float64)
            if P:
                ki, _ = cf.gather_seq(cache, page_table, b, 128 * P, g)
                k = np.concatenate([k, ki.astype(np.float64)])
            mask = np.zeros(128)
            mask[sel[b, g]] = 1.0
            qa = np.abs(qp[b, g * grp:(g + 1) * grp].astype(np.float64)) * mask
            out[b, g * grp:(g + 1) * grp] = (np.abs(k) @ qa.T).max(0) * sm_scale
    return 2.0 ** -16 * out + 2.0 ** -20 * np.abs(lse_ref)


DECODE_CASES = [
    ("all-bf16", synth.Shape(3, 32, 8, [1, 63, 300], 77)),
    ("page-edges", synth.Shape(4, 32, 8, [320, 447, 448, 449], 77, shuffle_pages=True)),
    ("long-g4", synth.Shape(2, 32, 8, [5000, 1300], 77, shuffle_pages=True)),
    ("nk128", synth.Shape(1, 32, 8, [3000], 128)),
    ("g2", synth.Shape(2, 16, 8, [2000, 700], 77)),
    ("mha", synth.Shape(1, 4, 4, [900], 52)),
]


@pytest.mark.parametrize("name,shape", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_tiered_parity(name, shape):
    _say("tiered decode", name)
    prob = synth.make_problem(shape, seed=71)
    d, cache, tiers = _prefill(prob, shape)
    qp, sel = pa.dqk_select_channels(d["q"], d["t_q"], shape.hkv, shape.n_keep)
    out, lse = pa.dqk_decode_attn_tiered(cache, tiers, qp, sel, d["page_table"], d["seq_lens"], prob.sm_scale)
    torch.cuda.synchronize()
    hc, ht = gu.cache_to_host(cache), tiers_to_host(tiers)
    qh, sh = gu.host(qp), gu.host(sel)
    ref, ref_lse = oracle.decode_tiered(hc, ht, qh, sh, prob.page_table, prob.seq_lens, prob.sm_scale)
    rel = gu.row_rel_err(gu.host(out), ref)
    _say(f"  max row rel err {rel.max():.3e}")
    assert (rel <= gu.TOL).all()
    bound = _tier_lse_bound(hc, ht, qh, sh, prob.page_table, prob.seq_lens, prob.sm_scale, ref_lse)
    gu.assert_lse(gu.host(lse), ref_lse, bound)


def test_decode_tiered_sink_regime():
    """A sink token about 12 nats above a flat background (the regime the
    protected tier exists for) at token 2, in the BF16 sink tier, at 32K
    tokens: most of the softmax mass sits in one BF16 token, the rest is
    spread over INT2 pages and the BF16 tail."""
    from tests.test_gpu_regimes import _sink
    _say("tiered decode, sink")
    shape = synth.Shape(1, 32, 8, [32768], 77)
    prob = synth.make_problem(shape, seed=73)
    gaps = _sink(prob, [2], 12.0)
    _say(f"  sink gaps (nats): {np.round(np.asarray(gaps, float).ravel(), 1).tolist()}")
    d, cache, tiers = _prefill(prob, shape)
    qp, sel = pa.dqk_select_channels(d["q"], d["t_q"], shape.hkv, shape.n_keep)
    out, lse = pa.dqk_decode_attn_tiered(cache, tiers, qp, sel, d["page_table"], d["seq_lens"], prob.sm_scale)
    torch.cuda.synchronize()
    hc, ht = gu.cache_to_host(cache), tiers_to_host(tiers)
    ref, ref_lse = oracle.decode_tiered(hc, ht, gu.host(qp), gu.host(sel), prob.page_table, prob.seq_lens,
                                        prob.sm_scale)
    rel = gu.row_rel_err(gu.host(out), ref)
    _say(f"  max row rel err {rel.max():.3e}")
    assert (rel <= gu.TOL).all()


ONE_CALL_CASES = [
    ("all-bf16", synth.Shape(3, 32, 8, [1, 63, 300], 77), 0),
    ("page-edges", synth.Shape(4, 32, 8, [320, 447, 448, 449], 77, shuffle_pages=True), 0),
    ("long-g4", synth.Shape(2, 32, 8, [5000, 1300], 77, shuffle_pages=True), 0),
    ("long-g4-3splits", synth.Shape(2, 32, 8, [5000, 1300], 77, shuffle_pages=True), 3),
    ("nk128", synth.Shape(1, 32, 8, [3000], 128), 0),
    ("nk9", synth.Shape(1, 32, 8, [3000], 9), 0),
    ("g2", synth.Shape(2, 16, 8, [2000, 700], 77), 0),
]


@pytest.mark.parametrize("name,shape,ns", ONE_CALL_CASES, ids=[c[0] for c in ONE_CALL_CASES])
def test_one_call_tiered_equals_two_calls(name, shape, ns):
    """dqk_select_decode_attn_tiered gives bit for bit dqk_select_channels +
    dqk_decode_attn_tiered, and that selection is the oracle's."""
    _say("tiered one call", name)
    prob = synth.make_problem(shape, seed=74)
    d, cache, tiers = _prefill(prob, shape)
    out1, lse1, qp1, sel1 = pa.dqk_select_decode_attn_tiered(cache, tiers, d["q"], d["t_q"], shape.n_keep,
                                                             d["page_table"], d["seq_lens"], prob.sm_scale,
                                                             num_splits=ns)
    qp2, sel2 = pa.dqk_select_channels(d["q"], d["t_q"], shape.hkv, shape.n_keep)
    out2, lse2 = pa.dqk_decode_attn_tiered(cache, tiers, qp2, sel2, d["page_table"], d["seq_lens"], prob.sm_scale,
                                           num_splits=ns)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.host(qp1).view(np.uint32), gu.host(qp2).view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel1), gu.host(sel2))
    np.testing.assert_array_equal(gu.host(out1).view(np.uint32), gu.host(out2).view(np.uint32))
    np.testing.assert_array_equal(gu.host(lse1).view(np.uint32), gu.host(lse2).view(np.uint32))
    qp_ref, sel_ref = oracle.select_channels(prob.q, prob.t_q, shape.hkv, shape.n_keep)
    np.testing.assert_array_equal(gu.host(qp1).view(np.uint32), qp_ref.view(np.uint32))
    np.testing.assert_array_equal(gu.host(sel1), sel_ref)
