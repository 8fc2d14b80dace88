"""Pins of the oracle's query transform and dynamic channel selection (§3.2 Eq. 4)."""
import numpy as np
import pytest

import synth

U = 2.0 ** -24


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (4, 1)])
def test_query_transform_within_fma_chain_bound(orc, hq, hkv):
    shape = synth.Shape(3, hq, hkv, [128] * 3, 77)
    prob = synth.make_problem(shape, seed=11, materialize_kv=False)
    qp, _ = orc.select_channels(prob.q, prob.t_q, hkv, 77)
    q64 = synth.bf16_bits_to_f32(prob.q).astype(np.float64)
    grp = hq // hkv
    for b in range(shape.batch):
        for h in range(hq):
            tq = prob.t_q[h // grp].astype(np.float64)
            ref = q64[b, h] @ tq
            bound = (128 * U / (1 - 128 * U)) * (np.abs(q64[b, h]) @ np.abs(tq))
            assert (np.abs(qp[b, h] - ref) <= bound).all()


def _pooled_fp64(qp, grp):
    B, hq, d = qp.shape
    return (qp.astype(np.float64) ** 2).reshape(B, hq // grp, grp, d).sum(axis=2)


@pytest.mark.parametrize("hq,hkv,n_keep", [(8, 8, 77), (32, 8, 77), (32, 8, 1), (32, 8, 128), (16, 2, 52)])
def test_selection_is_top_k_of_pooled_energy(orc, hq, hkv, n_keep):
    """Brute force: a full sort of the pooled energy (fp64) picks the same set,
    except where two channels' energies are within fp32 rounding."""
    shape = synth.Shape(4, hq, hkv, [128] * 4, n_keep)
    prob = synth.make_problem(shape, seed=12, materialize_kv=False)
    qp, sel = orc.select_channels(prob.q, prob.t_q, hkv, n_keep)
    S = _pooled_fp64(qp, hq // hkv)
    for b in range(shape.batch):
        for g in range(hkv):
            idx = sel[b, g]
            assert (np.diff(idx) > 0).all() and idx.min() >= 0 and idx.max() < 128
            order = sorted(range(128), key=lambda j: (-S[b, g, j], j))
            want = set(order[:n_keep])
            got = set(idx.tolist())
            if got != want:
                # the boundary pair must be a near-tie
                thr = S[b, g, order[n_keep - 1]]
                for j in got ^ want:
                    assert abs(S[b, g, j] - thr) <= 8 * U * thr * (hq // hkv)


def test_selection_is_nested_in_k(orc):
    shape = synth.Shape(2, 32, 8, [128] * 2, 1)
    prob = synth.make_problem(shape, seed=13, materialize_kv=False)
    prev = None
    for k in range(1, 129):
        _, sel = orc.select_channels(prob.q, prob.t_q, 8, k)
        sets = [[set(sel[b, g].tolist()) for g in range(8)] for b in range(2)]
        if prev is not None:
            for b in range(2):
                for g in range(8):
                    assert prev[b][g] <= sets[b][g]
        prev = sets
    assert all(s == set(range(128)) for row in prev for s in row)


def test_single_head_groups_reduce_to_top_k_magnitude(orc):
    """With one query head per KV head the pooled energy is |q'_j|^2, so the
    mask is the top-k of |q'| (ties are measure-zero for Gaussian q)."""
    shape = synth.Shape(2, 8, 8, [128] * 2, 77)
    prob = synth.make_problem(shape, seed=14, materialize_kv=False)
    qp, sel = orc.select_channels(prob.q, prob.t_q, 8, 77)
    for b in range(2):
        for h in range(8):
            want = np.sort(np.argsort(-np.abs(qp[b, h]), kind="stable")[:77])
            np.testing.assert_array_equal(sel[b, h], want)


def test_select_rejects_bad_shapes(orc):
    q = np.zeros((1, 6, 128), np.uint16)
    tq = np.zeros((4, 128, 128), np.float32)
    with pytest.raises(ValueError):
        orc.select_channels(q, tq, 4, 77)      # 6 % 4 != 0
    with pytest.raises(ValueError):
        orc.select_channels(q[:, :4], tq, 4, 0)


def test_exact_ties_go_to_the_lower_channel(orc):
    """Hand-built ties: T_Q = I, so q' = q and the pooled energy is sum_h q_h^2.
    Equal energies are ranked by channel index (lower first)."""
    tq = np.eye(128, dtype=np.float32)[None]
    q = np.full((1, 1, 128), 0.5, np.float32)
    q[0, 0, 100] = 2.0
    q[0, 0, 7] = -2.0                         # same energy as channel 100
    qb = synth.f32_to_bf16_bits(q)
    _, sel = orc.select_channels(qb, tq, 1, 4)
    assert sel[0, 0].tolist() == [0, 1, 7, 100]
    _, sel = orc.select_channels(qb, tq, 1, 1)
    assert sel[0, 0].tolist() == [7]
    # two heads pooled: (1, 1) and (sqrt2-ish, 0) do not tie; (1,1) vs (-1,1) do
    q2 = np.zeros((1, 2, 128), np.float32)
    q2[0, :, 5] = [1.0, 1.0]
    q2[0, :, 3] = [-1.0, 1.0]
    q2[0, :, 9] = [1.0, -1.0]
    _, sel = orc.select_channels(synth.f32_to_bf16_bits(q2), tq, 1, 2)
    assert sel[0, 0].tolist() == [3, 5]
