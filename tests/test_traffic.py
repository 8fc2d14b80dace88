"""The storage/read-volume accounting reproduces the bits-per-element figures
the Dual-QK paper prints (Table 1, §4.2; abstract ratios) and gives the byte
mix of this library's page format."""
import json
import os

import numpy as np
import pytest

from page_set_amd import traffic

GOLD = os.path.join(os.path.dirname(__file__), "golden", "bpe_table1.json")


def test_table1_bits_per_element():
    g = json.load(open(GOLD))
    for fmt, (cap, bw) in g["table1"].items():
        c, b = traffic.bits_per_element(fmt, g["n_tokens"], g["n_keep"])
        # the table prints two decimals (3.125 appears as 3.13: half rounds up)
        assert abs(c - cap) <= 0.005 + 1e-12, fmt
        assert abs(b - bw) <= 0.005 + 1e-12, fmt
    c, b = traffic.bits_per_element("dual-qk")
    assert round(16 / c, 1) == g["abstract_ratios"]["compression"]
    assert round(16 / b, 1) == g["abstract_ratios"]["read_reduction"]


@pytest.mark.parametrize("n_keep,with0,without0", [(128, 85.71875, 84.0), (103, 78.6875, 76.96875),
                                                   (77, 71.375, 69.65625), (52, 64.34375, 62.625)])
def test_bytes_per_token_head(n_keep, with0, without0):
    assert traffic.bytes_per_token_head(n_keep, True) == with0
    assert traffic.bytes_per_token_head(n_keep, False) == without0


def test_decode_cache_bytes_counts_the_actual_mask():
    lens = np.array([256, 130], np.int32)
    sel = np.zeros((2, 2, 77), np.int32)
    sel[0, 0] = np.arange(77)          # channel 0 kept
    sel[0, 1] = np.arange(1, 78)       # channel 0 pruned
    sel[1, 0] = np.arange(77)
    sel[1, 1] = np.arange(77)
    got = traffic.decode_cache_bytes(lens, sel)
    want = (2 * 76 * 36 + 256 * 50) + (2 * 77 * 36 + 256 * 48) + 2 * (2 * 76 * 36 + 130 * 50)
    assert got == want


def test_tiered_bytes_by_enumeration():
    """decode_tiered_bytes against a token-by-token count: every token is in
    the sink, an INT2 page or the tail, and reads what its tier stores."""
    from page_set_amd import traffic as tr
    rng = np.random.default_rng(3)
    for L in (1, 64, 65, 319, 320, 447, 448, 5000, 131072):
        sel = np.sort(rng.choice(128, size=(1, 2, 77), replace=True), axis=-1).astype(np.int32)
        sel[0, 0, 0] = 0  # head 0 keeps channel 0, head 1 may not
        want = 0
        for g in range(2):
            s = sel[0, g]
            has0 = bool((s == 0).any())
            r = len(s) - (1 if has0 else 0)
            P = tr.tier_pages(L)
            n_int2 = 0
            for t in range(L):
                if t < 64 or t >= 64 + 128 * P:
                    want += 77 * 2 + 128 * 2
                else:
                    n_int2 += 1
                    want += (2 if has0 else 0) + 48
            assert n_int2 == 128 * P
            want += P * r * 36
        assert tr.decode_tiered_bytes([L], sel) == want


def test_tokgrid_bytes_by_enumeration():
    """decode_cache_bytes_tokgrid against a count page by page and token by
    token: a selected INT2 row is 32 bytes of a page, every valid token reads
    its 4-byte key grid, channel 0 (2 bytes) when selected, 48 value bytes."""
    rng = np.random.default_rng(5)
    lens = np.array([1, 128, 129, 3000], np.int32)
    sel = np.sort(rng.choice(128, size=(4, 2, 77), replace=True), axis=-1).astype(np.int32)
    sel[:, 0, 0] = 0
    sel[:, 1] = np.arange(1, 78)
    want = 0
    for b, L in enumerate(lens):
        for g in range(2):
            s = sel[b, g]
            has0 = bool((s == 0).any())
            for p in range((int(L) + 127) // 128):
                want += (len(s) - has0) * 32
            for t in range(int(L)):
                want += 4 + 2 * has0 + 32 + 16
    assert traffic.decode_cache_bytes_tokgrid(lens, sel) == want
