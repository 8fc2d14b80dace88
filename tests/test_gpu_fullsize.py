"""Parity at the benchmark's full sizes.

The GPU builds the INT2 cache (dqk_quantize_append, sequence by sequence),
selects and decodes the whole batch in the launch configuration bench.py
times (automatic split count).  Two (sequence, KV head) units per workload,
drawn with a fixed seed, are then recomputed by the oracle from the same
cache bytes (the unit's pages, downloaded) and compared: selected channels
bit-exact, output rows within 2e-3, log-sum-exp within 2e-5.
"""
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


def _build_cache(shape, prob, d):
    cache = pa.Cache(prob.num_pages, shape.hkv)
    for b in range(shape.batch):
        kb, vb = synth.make_kv_seq(shape, prob.seed, b, prob.outliers)
        L = kb.shape[0]
        cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        pa.dqk_quantize_append(cache, gu.dev(kb), gu.dev(vb), d["t_k"], cu, d["page_table"][b:b + 1].clone())
        torch.cuda.synchronize()
    return cache


def _unit_cache(cache, pages, g):
    """The pages of one sequence for KV head g, as a one-head oracle cache."""
    idx = torch.from_numpy(np.ascontiguousarray(pages, dtype=np.int64)).to("cuda")
    sub = oracle.Cache(len(pages), 1)
    for src, dst in zip(cache.arrays(), sub.arrays()):
        dst[:, 0] = gu.host(src.index_select(0, idx)[:, g].contiguous(), dst.dtype)
    return sub


@pytest.mark.parametrize("cfg", [3, 4, 2], ids=["b4-128k", "ragged-b32", "b16-32k"])
def test_full_size_sampled_units(cfg):
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
    units = np.random.default_rng(123 + cfg).choice(shape.batch * shape.hkv, size=2, replace=False)
    for u in units:
        b, g = divmod(int(u), shape.hkv)
        L = int(prob.seq_lens[b])
        npg = (L + 127) // 128
        heads = slice(g * grp, (g + 1) * grp)
        q = np.ascontiguousarray(prob.q[b:b + 1, heads])
        qp_ref, sel_ref = oracle.select_channels(q, prob.t_q[g:g + 1], 1, shape.n_keep)
        np.testing.assert_array_equal(sel_h[b, g], sel_ref[0, 0])
        sub = _unit_cache(cache, prob.page_table[b, :npg], g)
        ref, ref_lse = oracle.decode_attn(sub, qp_ref, sel_ref, np.arange(npg, dtype=np.int32)[None],
                                          np.array([L], np.int32), prob.sm_scale)
        rel = gu.row_rel_err(out_h[b, heads], ref[0])
        _say(f"  unit b={b} g={g} L={L}: max row rel err {rel.max():.3e}")
        assert (rel <= gu.TOL).all(), rel.max()
        np.testing.assert_allclose(lse_h[b, heads], ref_lse[0], rtol=2e-5, atol=2e-5)
