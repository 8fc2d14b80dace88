"""GPU decode against the oracle in numerical regimes the Gaussian workloads
do not reach: an attention sink far above a long flat background, a sharp
softmax, keys and values scaled by 1e-3 and 1e3, values with a large mean,
and constant quantization groups (scale 0).

The dual-transform cache keeps the sink and recent tokens in BF16 because
attention mass concentrates there (Dual-QK §3.3); whatever tier a token sits
in, the decode has to keep the one softmax over the context accurate (§3.4),
including the long tail of tokens whose weight is 1e-4 .. 1e-7 of the sink's.

Each case perturbs the seeded raw q/k/v (bf16), lets the oracle build the
cache, select and decode, uploads the oracle's cache bytes, q' and selection,
and decodes on the GPU at several split counts.  Bar: max row relative error
2e-3 against the oracle.
"""
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


def _f(bits):
    return synth.bf16_bits_to_f32(bits)


def _b(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _sink_keys(prob, positions, reach_by_g):
    sh = prob.shape
    grp = sh.hq // sh.hkv
    k = _f(prob.k0).copy()
    q = _f(prob.q).astype(np.float64)
    for b in range(sh.batch):
        s = int(prob.cu_tokens[b])
        for g in range(sh.hkv):
            u = q[b, g * grp:(g + 1) * grp].sum(0)
            u /= np.linalg.norm(u)
            for t in positions:
                k[s + t, g] = reach_by_g[b][g] * u
    prob.k = _b(k)


def _gaps(prob, positions):
    """Realised logit of the first sink token above the background mean (nats),
    averaged over the query heads of each KV head, through the oracle's
    transform, selection and quantization."""
    sh = prob.shape
    grp = sh.hq // sh.hkv
    cache, _ = oracle.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = oracle.select_channels(prob.q, prob.t_q, sh.hkv, sh.n_keep)
    out = []
    for b in range(sh.batch):
        L = int(prob.seq_lens[b])
        row = []
        for g in range(sh.hkv):
            kh, _ = cf.gather_seq(cache, prob.page_table, b, L, g)
            mask = np.zeros(128)
            mask[sel[b, g]] = 1
            qm = qp[b, g * grp:(g + 1) * grp].astype(np.float64) * mask
            x = (kh.astype(np.float64) @ qm.T) * prob.sm_scale          # [L][grp]
            bg = np.delete(x, positions, axis=0)
            row.append(float((x[positions[0]] - bg.mean(0)).mean()))
        out.append(row)
    return out


def _sink(prob, positions, nats):
    """Keys at `positions` of every sequence point along the summed query of
    their KV head's group, with a length calibrated (two passes through the
    oracle, the logit being linear in the key) so that the realised sink logit
    sits `nats` above the background mean."""
    prob.k0 = prob.k.copy()
    sh = prob.shape
    reach = [[4.0 * nats] * sh.hkv for _ in range(sh.batch)]
    _sink_keys(prob, positions, reach)
    gaps = _gaps(prob, positions)
    reach = [[reach[b][g] * nats / max(gaps[b][g], 0.5) for g in range(sh.hkv)] for b in range(sh.batch)]
    _sink_keys(prob, positions, reach)
    return _gaps(prob, positions)


def _check(prob, splits=(0, 1, 7), label="", kprime_fn=None):
    sh = prob.shape
    kp = oracle.key_transform(prob.k, prob.t_k)
    if kprime_fn is not None:
        kp = kprime_fn(kp)
    cache = oracle.pack_cache(kp, prob.v, prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = oracle.select_channels(prob.q, prob.t_q, sh.hkv, sh.n_keep)
    ref, ref_lse = oracle.decode_attn(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale)
    bound = gu.lse_bound(cache, qp, sel, prob.page_table, prob.seq_lens, prob.sm_scale, ref_lse)
    gc = gu.cache_to_device(cache)
    outs = []
    for ns in splits:
        out, lse = pa.dqk_decode_attn(gc, gu.dev(qp), gu.dev(sel), gu.dev(prob.page_table), gu.dev(prob.seq_lens),
                                      prob.sm_scale, num_splits=ns)
        torch.cuda.synchronize()
        o = gu.host(out)
        rel = gu.row_rel_err(o, ref)
        _say(f"  {label} splits={ns}: max row rel err {rel.max():.3e}")
        assert np.isfinite(o).all()
        assert (rel <= gu.TOL).all(), (ns, rel.max())
        gu.assert_lse(gu.host(lse), ref_lse, bound)
        outs.append(o)
    return cache, qp, sel, ref, outs


LONG = synth.Shape(1, 8, 2, [32768], 77)          # group of 4: MFMA path
LONG_G2 = synth.Shape(1, 4, 2, [32768], 77)       # group of 2: one padded set of four heads


@pytest.mark.parametrize("shape", [LONG, LONG_G2], ids=["g4", "g2"])
@pytest.mark.parametrize("nats", [8.0, 12.0, 14.0])
def test_sink_over_long_flat_background(shape, nats):
    _say("sink", shape.hq, shape.hkv, nats)
    prob = synth.make_problem(shape, seed=201)
    gaps = _sink(prob, [0, 1, 2, 3], nats)
    _say(f"  realised sink gaps over the background mean: {np.round(gaps, 2).tolist()} nats")
    assert np.abs(np.asarray(gaps) - nats).max() <= 1.5
    _check(prob, label=f"sink{nats:g}")


@pytest.mark.parametrize("vscale,voff", [(1e-3, 0.0), (1.0, 1000.0)], ids=["small-values", "offset-values"])
def test_sink_with_value_extremes(vscale, voff):
    _say("sink + values", vscale, voff)
    prob = synth.make_problem(LONG, seed=202)
    _sink(prob, [0, 1, 2, 3], 12.0)
    prob.v = _b(_f(prob.v) * np.float32(vscale) + np.float32(voff))
    _check(prob, label="sink+v")


def test_sink_with_small_patterned_values():
    """Small values whose 2-bit codes carry a fixed pattern across the
    channels of each group: the background tokens' code terms no longer
    average out, so losing them (an underflowing probability x scale product)
    shows up in the output."""
    _say("sink + small patterned values")
    prob = synth.make_problem(LONG, seed=208)
    _sink(prob, [0, 1, 2, 3], 12.0)
    pattern = np.where(np.arange(128) % 2 == 0, 3.0, -3.0).astype(np.float32)
    prob.v = _b((_f(prob.v) * np.float32(0.5) + pattern) * np.float32(1e-3))
    _check(prob, label="sink+pattern")


def test_late_sharp_token():
    """The largest logit arrives late in the context, after many pages have
    been accumulated against a smaller running maximum."""
    _say("late sharp token")
    prob = synth.make_problem(LONG, seed=203)
    _sink(prob, [20000, 31000], 14.0)
    _check(prob, label="late")


def test_sharp_token_in_a_short_last_page():
    """The largest logit sits in a last page holding fewer than 65 tokens, so
    the running maximum rises on a page whose second token half is empty:
    everything accumulated for that half so far must still be rescaled."""
    _say("sharp token in a short last page")
    shape = synth.Shape(1, 8, 2, [32768 + 40], 77)
    prob = synth.make_problem(shape, seed=209)
    _sink(prob, [32768 + 30], 10.0)
    _check(prob, label="short-last-page")


@pytest.mark.parametrize("qscale", [8.0])
def test_sharp_softmax_scaled_queries(qscale):
    _say("q x", qscale)
    prob = synth.make_problem(synth.Shape(2, 32, 8, [6000, 1300], 77), seed=204)
    prob.q = _b(_f(prob.q) * np.float32(qscale))
    _check(prob, label=f"q*{qscale:g}")


@pytest.mark.parametrize("kscale", [1e-3, 1e3])
def test_key_scales(kscale):
    _say("k x", kscale)
    prob = synth.make_problem(synth.Shape(2, 32, 8, [5000, 900], 77), seed=205)
    prob.k = _b(_f(prob.k) * np.float32(kscale))
    _check(prob, label=f"k*{kscale:g}")


@pytest.mark.parametrize("vscale,voff", [(1e-3, 0.0), (1e3, 0.0), (1.0, 1000.0)],
                         ids=["v-small", "v-large", "v-offset"])
def test_value_scales(vscale, voff):
    _say("v", vscale, voff)
    prob = synth.make_problem(synth.Shape(2, 32, 8, [5000, 900], 77), seed=206)
    prob.v = _b(_f(prob.v) * np.float32(vscale) + np.float32(voff))
    _check(prob, label="v")


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 8)], ids=["g4", "g2"])
def test_constant_groups(hq, hkv):
    """A page whose transformed keys are one binary16-exact row packs every
    key channel with scale 0 (all codes 3); value groups set to one constant
    pack with scale 0 too."""
    _say("constant groups", hq, hkv)
    prob = synth.make_problem(synth.Shape(2, hq, hkv, [1000, 700], 77), seed=207)
    v = _f(prob.v).copy()
    for b in range(2):
        s = int(prob.cu_tokens[b])
        v[s:s + int(prob.seq_lens[b]):3, :, 0:32] = 0.75
    prob.v = _b(v)

    def const_page(kp):
        kp = kp.copy()
        for b in range(2):
            s = int(prob.cu_tokens[b])
            row = kp[s + 128].astype(np.float16).astype(np.float32)
            kp[s + 128:s + 256] = row
        return kp

    cache, *_ = _check(prob, label="const", kprime_fn=const_page)
    p = int(prob.page_table[0, 1])
    assert (cache.k_meta_page(p)[:, 1:, 0] == 0).all()          # every key channel of the page has scale 0
    assert (cache.v_meta[int(prob.page_table[0, 0]), :, 0, 0, 0] == 0).all()
