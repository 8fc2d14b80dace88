"""Pins of the oracle's number-format helpers against library-enumerated grids."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore")


def _f16_grid():
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    ok = np.isfinite(vals)
    vals, bits = vals[ok], bits[ok]
    order = np.argsort(vals, kind="stable")
    return vals[order], bits[order]


def test_f16_value_matches_numpy(orc):
    for b in list(range(0, 0x10000, 97)) + [0x0001, 0x03FF, 0x0400, 0x7BFF, 0x8001, 0xFBFF]:
        want = np.array([b], dtype=np.uint16).view(np.float16).astype(np.float64)[0]
        got = orc.f16_value(b)
        assert (np.isnan(got) and np.isnan(want)) or got == want


def test_f16_directed_rounding_against_enumerated_grid(orc):
    vals, _ = _f16_grid()
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 5, 3000),
        vals[rng.integers(0, len(vals), 500)],            # exactly representable
        np.array([0.0, 65504.0, -65504.0, 6.1e-5, -5.96e-8, 1e-9]),
    ]).astype(np.float32)
    for x in xs:
        xd = float(x)
        lo = vals[np.searchsorted(vals, xd, side="right") - 1] if xd >= vals[0] else -np.inf
        hi_i = np.searchsorted(vals, xd, side="left")
        hi = vals[hi_i] if hi_i < len(vals) else np.inf
        rd = orc.f16_value(orc.f16_round_down(x))
        ru = orc.f16_value(orc.f16_round_up(x))
        if abs(xd) <= 65504:
            assert rd == lo, (x, rd, lo)
            assert ru == hi, (x, ru, hi)
        assert rd <= xd <= ru


def test_f16_rounding_beyond_range(orc):
    assert orc.f16_value(orc.f16_round_up(70000.0)) == np.inf
    assert orc.f16_value(orc.f16_round_down(70000.0)) == 65504.0
    assert orc.f16_value(orc.f16_round_down(-70000.0)) == -np.inf
    assert orc.f16_value(orc.f16_round_up(-70000.0)) == -65504.0


def test_bf16_nearest_even_matches_torch(orc):
    rng = np.random.default_rng(2)
    xs = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 4000).astype(np.float32),
        # exact ties: bf16 value + half a bf16 step
        (np.array([1.0, 1.0078125, -3.0, 257.0], dtype=np.float32)
         + np.array([2 ** -8, 2 ** -8, -2 ** -7, 1.0], dtype=np.float32)),
        np.array([1e-39, -1e-40, 3.3e38], dtype=np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_round_nearest(x) for x in xs], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)
