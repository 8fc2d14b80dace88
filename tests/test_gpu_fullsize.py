"""Parity at the benchmark's full sizes.

The GPU builds the INT2 cache (dqk_quantize_append, sequence by sequence),
selects and decodes the whole batch in the launch configuration bench.py
times (automatic split count).  Then EVERY (sequence, KV head) unit is
recomputed by the oracle from the same cache bytes (the unit's pages,
downloaded), the units spread over host threads: selected channels
bit-exact, output rows within 2e-3, log-sum-exp within the bound derived from
the kernels' arithmetic.  The key transform and packing are checked stage by
stage on sampled pages of a 131072-token x 8-head prefill, and the BF16
baseline at 32768 tokens.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle
import page_set_amd as pa
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))


def _say(*a):
    print(*a, flush=True)


def _build_cache(shape, prob, d, kprime_seq0=None):
    cache = pa.Cache(prob.num_pages, shape.hkv)
    for b in range(shape.batch):
        kb, vb = synth.make_kv_seq(shape, prob.seed, b, prob.outliers)
        L = kb.shape[0]
        cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        pa.dqk_quantize_append(cache, gu.dev(kb), gu.dev(vb), d["t_k"], cu, d["page_table"][b:b + 1].clone(),
                               kprime_dbg=kprime_seq0 if b == 0 else None)
        torch.cuda.synchronize()
    return cache


def _unit_cache(pm, pages, g):
    """The pages of one sequence for KV head g, as a one-head oracle cache
    (pm: the GPU cache's page-major copies)."""
    idx = torch.from_numpy(np.ascontiguousarray(pages, dtype=np.int64)).to("cuda")
    sub = oracle.Cache(len(pages), 1)
    dst = [np.zeros((sub.num_pages, 1) + tuple(a.shape[2:]), dtype=b)
           for a, b in zip(pm, (np.uint8, np.uint16, np.uint16, np.uint8, np.uint16))]
    for src, d in zip(pm, dst):
        d[:len(pages), 0] = gu.host(src.index_select(0, idx)[:, g].contiguous(), d.dtype)
    sub.set_page_major(*dst)
    return sub


def _meta_lse_bound(sub, qp, sel, sm_scale, lse_ref):
    """The derived lse bound of gpu_util.lse_bound with max_t |k_tj| replaced by
    its per-channel upper bound from the page metadata (max over pages of
    |zero| and |zero + 3 scale|, channel 0 from its bf16 values)."""
    km = sub.page_major()[1]
    s = km[:, 0, :, 0].view(np.float16).astype(np.float64)
    z = km[:, 0, :, 1].view(np.float16).astype(np.float64)
    kmax = np.maximum(np.abs(z), np.abs(z + 3 * s)).max(0)
    kmax[0] = np.abs(synth.bf16_bits_to_f32(sub.k_ch0[:, 0]).astype(np.float64)).max()
    mask = np.zeros(128)
    mask[sel[0, 0]] = 1
    a = (np.abs(qp[0].astype(np.float64)) * mask) @ kmax * sm_scale
    return 2.0 ** -16 * a + 2.0 ** -20 * np.abs(lse_ref[0])


@pytest.mark.parametrize("cfg", [3, 4, 2], ids=["b4-128k", "ragged-b32", "b16-32k"])
def test_full_size_every_unit(cfg):
    shape = synth.config_shape(cfg)
    _say("full size", shape.name, "lengths", min(shape.seq_lens), "..", max(shape.seq_lens))
    prob = synth.make_problem(shape, seed=0, materialize_kv=False)
    d = gu.upload(prob)
    cache = _build_cache(shape, prob, d)
    qp, sel = pa.dqk_select_channels(d["q"], d["t_q"], shape.hkv, shape.n_keep)
    out, lse = pa.dqk_decode_attn(cache, qp, sel, d["page_table"], d["seq_lens"], prob.sm_scale)
    torch.cuda.synchronize()
    out_h, lse_h, sel_h = gu.host(out), gu.host(lse), gu.host(sel)
    grp = shape.hq // shape.hkv
    qp_ref, sel_ref = oracle.select_channels(prob.q, prob.t_q, shape.hkv, shape.n_keep)
    np.testing.assert_array_equal(sel_h, sel_ref)
    np.testing.assert_array_equal(gu.host(qp).view(np.uint32), qp_ref.view(np.uint32))

    units = [(b, g) for b in range(shape.batch) for g in range(shape.hkv)]

    def check(unit, sub):
        b, g = unit
        L = int(prob.seq_lens[b])
        npg = (L + 127) // 128
        heads = slice(g * grp, (g + 1) * grp)
        q1 = np.ascontiguousarray(qp_ref[b:b + 1, heads])
        s1 = np.ascontiguousarray(sel_ref[b:b + 1, g:g + 1])
        ref, ref_lse = oracle.decode_attn(sub, q1, s1, np.arange(npg, dtype=np.int32)[None],
                                          np.array([L], np.int32), prob.sm_scale)
        rel = gu.row_rel_err(out_h[b, heads], ref[0])
        err = np.abs(lse_h[b, heads] - ref_lse[0])
        bound = _meta_lse_bound(sub, q1, s1, prob.sm_scale, ref_lse)
        return float(rel.max()), bool((err <= bound).all()), float((err / bound).max())

    worst, lse_ok, futs = 0.0, True, []
    pm = cache.page_major()
    with cf.ThreadPoolExecutor(max_workers=THREADS) as ex:
        for b, g in units:
            L = int(prob.seq_lens[b])
            sub = _unit_cache(pm, prob.page_table[b, :(L + 127) // 128], g)
            futs.append(ex.submit(check, (b, g), sub))
        for (b, g), f in zip(units, futs):
            rel, ok, ratio = f.result()
            worst = max(worst, rel)
            lse_ok &= ok
            assert rel <= gu.TOL, (b, g, rel)
            assert ok, (b, g, ratio)
    _say(f"  {len(units)} units: worst row rel err {worst:.3e}; lse within the derived bound: {lse_ok}")


def test_append_stagewise_at_prefill_size():
    """131072 tokens x 8 KV heads through dqk_quantize_append with the k'
    readback: on 24 sampled pages, k' is within the recursive-summation bound
    of the exact sum and the packed bytes equal the oracle's pack of the
    GPU's own k'."""
    shape = synth.config_shape(3)
    shape = synth.Shape(1, shape.hq, shape.hkv, [shape.seq_lens[0]], shape.n_keep, name="prefill-128k")
    prob = synth.make_problem(shape, seed=5, materialize_kv=False)
    d = gu.upload(prob)
    L = shape.seq_lens[0]
    kdbg = torch.full((L, shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    cache = _build_cache(shape, prob, d, kprime_seq0=kdbg)
    kb, vb = synth.make_kv_seq(shape, prob.seed, 0, prob.outliers)
    pages = np.random.default_rng(11).choice(L // 128, size=24, replace=False)
    pm = cache.page_major()
    gam = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)
    t64 = np.abs(synth.bf16_bits_to_f32(prob.t_k).astype(np.float64))
    for pi in pages:
        p = int(prob.page_table[0, pi])
        t0 = int(pi) * 128
        kseg = np.ascontiguousarray(kb[t0:t0 + 128])
        vseg = np.ascontiguousarray(vb[t0:t0 + 128])
        kp_gpu = gu.host(kdbg[t0:t0 + 128])
        kp_ref = oracle.key_transform(kseg, prob.t_k)
        absdot = np.einsum("tgi,gij->tgj", np.abs(synth.bf16_bits_to_f32(kseg).astype(np.float64)), t64)
        err = np.abs(kp_gpu.astype(np.float64) - kp_ref.astype(np.float64))
        assert (err <= gam * absdot + np.spacing(np.abs(kp_ref))).all(), pi
        want = oracle.pack_cache(kp_gpu, vseg, np.array([0, 128], np.int32), np.zeros((1, 1), np.int32), 1)
        want_pm = want.page_major()
        for g in range(shape.hkv):
            got = _unit_cache(pm, [p], g).page_major()
            for nm, a, w in zip(["k_codes", "k_meta", "k_ch0", "v_codes", "v_meta"], got, want_pm):
                np.testing.assert_array_equal(a[0, 0], w[0, g], err_msg=f"{nm} page {pi} head {g}")
    _say(f"  {len(pages)} sampled pages x {shape.hkv} heads: stagewise parity holds")


def test_bf16_baseline_32k():
    shape = synth.Shape(1, 32, 8, [32768], 128, shuffle_pages=True)
    prob = synth.make_problem(shape, seed=13)
    kb, vb = oracle.paged_bf16(prob.k, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    ref, ref_lse = oracle.decode_bf16(kb, vb, prob.q, prob.page_table, prob.seq_lens, prob.sm_scale)
    out, lse = pa.dqk_decode_attn_bf16(gu.dev(kb), gu.dev(vb), gu.dev(prob.q), gu.dev(prob.page_table),
                                       gu.dev(prob.seq_lens), prob.sm_scale)
    torch.cuda.synchronize()
    rel = gu.row_rel_err(gu.host(out), ref)
    _say(f"  bf16 32k: max row rel err {rel.max():.3e}")
    assert (rel <= gu.TOL).all()
    np.testing.assert_allclose(gu.host(lse), ref_lse, rtol=1e-5, atol=1e-5)


def test_rotated_values_at_full_size():
    """The rotated-value path at the benchmark's shape (batch 4 x 131072
    tokens, GQA 32/8, n_keep 77, clip 0.92), in the launch configuration
    bench.py times: the cache built by dqk_quantize_append_vrot sequence by
    sequence (v' read back for sequence 0), then base selection, decode and
    the inverse rotation.  Stage by stage on 16 sampled pages of sequence 0
    (v' within the recursive-summation bound, value bytes equal the oracle's
    pack of the GPU's own v'); selection bit-exact; 8 sampled (sequence, KV
    head) units recomputed by the oracle from the same cache bytes, rows
    within 2e-3."""
    clip = 0.92
    shape = synth.config_shape(3)
    _say("rotated values at full size", shape.name)
    prob = synth.make_problem(shape, seed=0, materialize_kv=False)
    rv, rinv = synth.make_value_rotation(shape.hkv, 0)
    w = synth.make_selection_scales(shape.hkv, 0)
    d = gu.upload(prob)
    L0 = shape.seq_lens[0]
    vdbg = torch.full((L0, shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    cache = pa.Cache(prob.num_pages, shape.hkv)
    rv_d = gu.dev(rv)
    for b in range(shape.batch):
        kb, vb = synth.make_kv_seq(shape, prob.seed, b, prob.outliers)
        cu = torch.tensor([0, kb.shape[0]], dtype=torch.int32, device="cuda")
        pa.dqk_quantize_append_vrot(cache, gu.dev(kb), gu.dev(vb), d["t_k"], rv_d, clip, cu,
                                    d["page_table"][b:b + 1].clone(), vprime_dbg=vdbg if b == 0 else None)
        torch.cuda.synchronize()
    qp, sel = pa.dqk_select_channels_base(d["q"], d["t_q"], gu.dev(w), shape.hkv, shape.n_keep)
    o_rot, _ = pa.dqk_decode_attn(cache, qp, sel, d["page_table"], d["seq_lens"], prob.sm_scale)
    out = pa.dqk_value_unrotate(o_rot, gu.dev(rinv), shape.hkv)
    torch.cuda.synchronize()
    qp_ref, sel_ref = oracle.select_channels_base(prob.q, prob.t_q, w, shape.hkv, shape.n_keep)
    np.testing.assert_array_equal(gu.host(sel), sel_ref)
    np.testing.assert_array_equal(gu.host(qp).view(np.uint32), qp_ref.view(np.uint32))
    pm = cache.page_major()
    # stage by stage on sampled pages of sequence 0
    kb, vb = synth.make_kv_seq(shape, prob.seed, 0, prob.outliers)
    gam = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)
    r64 = np.abs(synth.bf16_bits_to_f32(rv).astype(np.float64))
    for pi in np.random.default_rng(12).choice(L0 // 128, size=16, replace=False):
        p = int(prob.page_table[0, pi])
        t0 = int(pi) * 128
        vseg = np.ascontiguousarray(vb[t0:t0 + 128])
        vp_gpu = gu.host(vdbg[t0:t0 + 128])
        vp_ref = oracle.value_transform(vseg, rv)
        absdot = np.einsum("tgi,gij->tgj", np.abs(synth.bf16_bits_to_f32(vseg).astype(np.float64)), r64)
        err = np.abs(vp_gpu.astype(np.float64) - vp_ref.astype(np.float64))
        assert (err <= gam * absdot + np.spacing(np.abs(vp_ref))).all(), pi
        kp = oracle.key_transform(np.ascontiguousarray(kb[t0:t0 + 128]), prob.t_k)
        want = oracle.pack_cache_vrot(kp, vp_gpu, clip, np.array([0, 128], np.int32), np.zeros((1, 1), np.int32), 1)
        want_pm = want.page_major()
        for g in range(shape.hkv):
            got = _unit_cache(pm, [p], g).page_major()
            for nm, i in (("v_codes", 3), ("v_meta", 4)):
                np.testing.assert_array_equal(got[i][0, 0], want_pm[i][0, g], err_msg=f"{nm} page {pi} head {g}")
    # sampled units end to end
    grp = shape.hq // shape.hkv
    out_h = gu.host(out)
    rng = np.random.default_rng(13)
    units = [(int(b), int(g)) for b, g in zip(rng.integers(0, shape.batch, 8), rng.integers(0, shape.hkv, 8))]

    def check(unit):
        b, g = unit
        L = int(prob.seq_lens[b])
        npg = (L + 127) // 128
        sub = _unit_cache(pm, prob.page_table[b, :npg], g)
        heads = slice(g * grp, (g + 1) * grp)
        o_ref, _ = oracle.decode_attn(sub, np.ascontiguousarray(qp_ref[b:b + 1, heads]),
                                      np.ascontiguousarray(sel_ref[b:b + 1, g:g + 1]),
                                      np.arange(npg, dtype=np.int32)[None], np.array([L], np.int32), prob.sm_scale)
        ref = oracle.value_unrotate(o_ref, np.ascontiguousarray(rinv[g:g + 1]), 1)
        return float(gu.row_rel_err(out_h[b, heads], ref[0]).max())

    with cf.ThreadPoolExecutor(max_workers=THREADS) as ex:
        errs = list(ex.map(check, units))
    _say(f"  16 sampled pages stagewise; {len(units)} sampled units: worst row rel err {max(errs):.3e}")
    assert max(errs) <= gu.TOL


def test_token_grid_at_full_size():
    """The per-token key grid layout at the benchmark's shape (batch 4 x
    131072 tokens, GQA 32/8, n_keep 77) in the launch configuration bench.py
    times: the cache built by dqk_quantize_append_tokgrid sequence by
    sequence (k' read back for sequence 0), selection and
    dqk_decode_attn_tokgrid.  Stage by stage on 16 sampled pages of sequence
    0 (every byte equals the oracle's pack of the GPU's own k'); 8 sampled
    units recomputed by the oracle from the same cache bytes, rows within
    2e-3."""
    shape = synth.config_shape(3)
    _say("per-token key grids at full size", shape.name)
    prob = synth.make_problem(shape, seed=0, materialize_kv=False)
    d = gu.upload(prob)
    L0 = shape.seq_lens[0]
    kdbg = torch.full((L0, shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    cache = pa.Cache(prob.num_pages, shape.hkv)
    for b in range(shape.batch):
        kb, vb = synth.make_kv_seq(shape, prob.seed, b, prob.outliers)
        cu = torch.tensor([0, kb.shape[0]], dtype=torch.int32, device="cuda")
        pa.dqk_quantize_append_tokgrid(cache, gu.dev(kb), gu.dev(vb), d["t_k"], cu, d["page_table"][b:b + 1].clone(),
                                       kprime_dbg=kdbg if b == 0 else None)
        torch.cuda.synchronize()
    qp, sel = pa.dqk_select_channels(d["q"], d["t_q"], shape.hkv, shape.n_keep)
    out, _ = pa.dqk_decode_attn(cache, qp, sel, d["page_table"], d["seq_lens"], prob.sm_scale, token_grid=True)
    torch.cuda.synchronize()
    pm = cache.page_major()
    # the key metadata token-major per block: [P/8][Hkv][8 slot][128 tok][2]
    km_tok = gu.host(cache.k_meta, np.uint16).reshape(prob.num_pages // 8, shape.hkv, 8, 128, 2)
    kb, vb = synth.make_kv_seq(shape, prob.seed, 0, prob.outliers)
    for pi in np.random.default_rng(14).choice(L0 // 128, size=16, replace=False):
        p = int(prob.page_table[0, pi])
        t0 = int(pi) * 128
        kp_gpu = gu.host(kdbg[t0:t0 + 128])
        want = oracle.pack_cache_tokgrid(kp_gpu, np.ascontiguousarray(vb[t0:t0 + 128]), np.array([0, 128], np.int32),
                                         np.zeros((1, 1), np.int32), 8)
        want_pm = want.page_major()
        want_tok = want.k_meta.reshape(1, shape.hkv, 8, 128, 2)
        for g in range(shape.hkv):
            for nm, i in (("k_codes", 0), ("k_ch0", 2), ("v_codes", 3), ("v_meta", 4)):
                got_i = gu.host(pm[i][p:p + 1, g].contiguous(), want_pm[i].dtype)
                np.testing.assert_array_equal(got_i[0], want_pm[i][0, g], err_msg=f"{nm} page {pi} head {g}")
            np.testing.assert_array_equal(km_tok[p // 8, g, p % 8], want_tok[0, g, 0], err_msg=f"k_meta page {pi}")
    grp = shape.hq // shape.hkv
    out_h, qp_h, sel_h = gu.host(out), gu.host(qp), gu.host(sel)
    rng = np.random.default_rng(15)
    units = [(int(b), int(g)) for b, g in zip(rng.integers(0, shape.batch, 8), rng.integers(0, shape.hkv, 8))]

    def check(unit):
        b, g = unit
        L = int(prob.seq_lens[b])
        npg = (L + 127) // 128
        pages = prob.page_table[b, :npg]
        sub = _unit_cache(pm, pages, g)
        sub_tok = sub.k_meta.reshape(sub.num_pages // 8, 1, 8, 128, 2)  # a view: the token layout of the unit
        for i, p in enumerate(pages):
            sub_tok[i // 8, 0, i % 8] = km_tok[p // 8, g, p % 8]
        heads = slice(g * grp, (g + 1) * grp)
        ref, _ = oracle.decode_attn_tokgrid(sub, np.ascontiguousarray(qp_h[b:b + 1, heads]),
                                            np.ascontiguousarray(sel_h[b:b + 1, g:g + 1]),
                                            np.arange(npg, dtype=np.int32)[None], np.array([L], np.int32),
                                            prob.sm_scale)
        return float(gu.row_rel_err(out_h[b, heads], ref[0]).max())

    with cf.ThreadPoolExecutor(max_workers=THREADS) as ex:
        errs = list(ex.map(check, units))
    _say(f"  16 sampled pages stagewise; {len(units)} sampled units: worst row rel err {max(errs):.3e}")
    assert max(errs) <= gu.TOL


def test_rope_at_full_size():
    """Bucket-relative RoPE at the benchmark's shape (batch 4 x 131072 tokens,
    64 buckets of 2048, GQA 32/8, n_keep 77) in the launch configuration
    bench.py times: the cache built by dqk_quantize_append_rope sequence by
    sequence (k' read back for sequence 0), then one dqk_select_decode_attn_rope
    call.  Stage by stage on 16 sampled pages of sequence 0 (k' within the
    summation bound of the oracle's turned-key product, every byte equal to
    the oracle's pack of the GPU's own k'); the per-bucket selection bit-exact
    for the whole batch; 8 sampled units recomputed by the oracle from the
    same cache bytes, rows within 2e-3."""
    shape = synth.config_shape(3)
    _say("bucket-relative RoPE at full size", shape.name)
    prob = synth.make_problem(shape, seed=0, materialize_kv=False)
    d = gu.upload(prob)
    nb = synth.rope_buckets(max(shape.seq_lens))
    cs, sn = synth.make_rope_tables(nb)
    dcs, dsn = gu.dev(cs), gu.dev(sn)
    L0 = shape.seq_lens[0]
    kdbg = torch.full((L0, shape.hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    cache = pa.Cache(prob.num_pages, shape.hkv)
    for b in range(shape.batch):
        kb, vb = synth.make_kv_seq(shape, prob.seed, b, prob.outliers)
        cu = torch.tensor([0, kb.shape[0]], dtype=torch.int32, device="cuda")
        pa.dqk_quantize_append_rope(cache, gu.dev(kb), gu.dev(vb), d["t_k"], dcs, dsn, cu,
                                    d["page_table"][b:b + 1].clone(), kprime_dbg=kdbg if b == 0 else None)
        torch.cuda.synchronize()
    out, _, qp, sel = pa.dqk_select_decode_attn_rope(cache, d["q"], d["t_q"], dcs, dsn, shape.n_keep,
                                                     d["page_table"], d["seq_lens"], prob.sm_scale)
    torch.cuda.synchronize()
    qp_h, sel_h, out_h = gu.host(qp), gu.host(sel), gu.host(out)
    qp_ref, sel_ref = oracle.select_channels_rope(prob.q, prob.t_q, cs, sn, shape.hkv, shape.n_keep)
    np.testing.assert_array_equal(qp_h.view(np.uint32), qp_ref.view(np.uint32))
    np.testing.assert_array_equal(sel_h, sel_ref)
    pm = cache.page_major()
    kb, vb = synth.make_kv_seq(shape, prob.seed, 0, prob.outliers)
    eye = np.broadcast_to(synth.f32_to_bf16_bits(np.eye(128, dtype=np.float32)), (shape.hkv, 128, 128)).copy()
    t64 = np.abs(synth.bf16_bits_to_f32(prob.t_k).astype(np.float64))
    one = np.array([0, 128], np.int32)
    gam = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)
    for pi in np.random.default_rng(16).choice(L0 // 128, size=16, replace=False):
        p, t0, bk = int(prob.page_table[0, pi]), int(pi) * 128, int(pi) // 16
        kpage = np.ascontiguousarray(kb[t0:t0 + 128])
        tabs = (np.ascontiguousarray(cs[bk:bk + 1]), np.ascontiguousarray(sn[bk:bk + 1]))
        turned = oracle.key_transform_rope(kpage, eye, one, *tabs).astype(np.float64)
        kp_ref = oracle.key_transform_rope(kpage, prob.t_k, one, *tabs).astype(np.float64)
        kp_gpu = gu.host(kdbg[t0:t0 + 128])
        bound = gam * np.einsum("tgi,gij->tgj", np.abs(turned), t64) + np.spacing(np.abs(kp_ref))
        assert (np.abs(kp_gpu.astype(np.float64) - kp_ref) <= bound).all(), f"k' page {pi}"
        want_pm = oracle.pack_cache(kp_gpu, np.ascontiguousarray(vb[t0:t0 + 128]), one, np.zeros((1, 1), np.int32),
                                    1).page_major()
        for g in range(shape.hkv):
            got = _unit_cache(pm, [p], g).page_major()
            for nm, x, w in zip(["k_codes", "k_meta", "k_ch0", "v_codes", "v_meta"], got, want_pm):
                np.testing.assert_array_equal(x[0, 0], w[0, g], err_msg=f"{nm} page {pi} head {g}")
    grp = shape.hq // shape.hkv
    rng = np.random.default_rng(17)
    units = [(int(b), int(g)) for b, g in zip(rng.integers(0, shape.batch, 8), rng.integers(0, shape.hkv, 8))]

    def check(unit):
        b, g = unit
        L = int(prob.seq_lens[b])
        npg = (L + 127) // 128
        sub = _unit_cache(pm, prob.page_table[b, :npg], g)
        heads = slice(g * grp, (g + 1) * grp)
        ref, _ = oracle.decode_attn_rope(sub, np.ascontiguousarray(qp_h[b:b + 1, :, heads]),
                                         np.ascontiguousarray(sel_h[b:b + 1, :, g:g + 1]),
                                         np.arange(npg, dtype=np.int32)[None], np.array([L], np.int32),
                                         prob.sm_scale)
        return float(gu.row_rel_err(out_h[b, heads], ref[0]).max())

    with cf.ThreadPoolExecutor(max_workers=THREADS) as ex:
        errs = list(ex.map(check, units))
    _say(f"  16 sampled pages stagewise; {len(units)} sampled units: worst row rel err {max(errs):.3e}")
    assert max(errs) <= gu.TOL
