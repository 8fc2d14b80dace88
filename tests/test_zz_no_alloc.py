"""The decode entry point that allocates nothing (its split partials live in
the library's own device array) against the workspace entry point it wraps:
same kernels, same split count, so the outputs must be identical.  Two calls
in a row, the second smaller, and a request too large for the array."""
import numpy as np
import pytest
import torch

import oracle
import page_set_amd as pa
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(shape, seed):
    prob = synth.make_problem(shape, seed=seed)
    cache, _ = oracle.quantize_append(prob.k, prob.v, prob.t_k, prob.cu_tokens, prob.page_table, prob.num_pages)
    qp, sel = oracle.select_channels(prob.q, prob.t_q, shape.hkv, shape.n_keep)
    return prob, gu.cache_to_device(cache), gu.dev(qp), gu.dev(sel), gu.dev(prob.page_table), gu.dev(prob.seq_lens)


def test_noalloc_equals_workspace_entry_twice():
    cases = [(synth.Shape(4, 32, 8, [20000, 5000, 131, 9000], 77), 1, 0),
             (synth.Shape(2, 32, 8, [3000, 700], 52), 2, 3),        # smaller, explicit split count
             (synth.Shape(3, 24, 4, [1500, 40, 900], 30), 3, 0)]    # group 6: two head sets (4 + 2)
    for shape, seed, ns in cases:
        print("noalloc", shape.batch, shape.hq, shape.hkv, shape.seq_lens, "splits", ns, flush=True)
        prob, gc, qp, sel, pt, sl = _case(shape, seed)
        out1, lse1 = pa.dqk_decode_attn(gc, qp, sel, pt, sl, prob.sm_scale, num_splits=ns)
        out2, lse2 = pa.dqk_decode_attn_noalloc(gc, qp, sel, pt, sl, prob.sm_scale, num_splits=ns)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gu.host(out2), gu.host(out1))
        np.testing.assert_array_equal(gu.host(lse2), gu.host(lse1))


def test_noalloc_rejects_partials_beyond_its_array():
    cap = pa.lib().dqk_decode_noalloc_max_bytes()
    assert cap == 16 << 20
    shape = synth.Shape(4, 32, 8, [32768] * 4, 77)
    prob, gc, qp, sel, pt, sl = _case(shape, 4)
    splits = 256                                  # 4 * 32 * 256 * 528 bytes > 16 MiB
    assert 4 * 32 * splits * 528 > cap
    with pytest.raises(RuntimeError, match="dqk_decode_attn_noalloc"):
        pa.dqk_decode_attn_noalloc(gc, qp, sel, pt, sl, prob.sm_scale, num_splits=splits)
