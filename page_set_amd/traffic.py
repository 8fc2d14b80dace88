"""Storage and read-volume accounting for 2-bit KV cache formats (host-side arithmetic only).

Used by the tests (to pin the accounting
against the figures the paper prints) and by the benchmark (to turn a
measured time into algorithmic bytes per second).

Closed form of the effective bits per KV element that "Dual-QK: Sharp Queries
and Flat Keys for Prunable 2-bit KV Caches" reports in Table 1 and Table 9.
Per §4.1 the paper gives two figures: a capacity figure for what the cache
stores, and a bandwidth figure for what one decode step reads once channels
are pruned; both include the quantization metadata and the BF16-kept tokens
(the sink and the recent window):

    bits/element = [(N - n_prot) * b_tok + n_prot * b_prot] / (N * 2 d)

with b_tok the bits one quantized token stores (capacity) or reads (bandwidth)
for its key and value, and b_prot the same for a BF16-protected token.  The
paper's metadata width is not stated; 16-bit scale + 16-bit zero per group is
the reading under which all four printed formats reproduce.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

D = 128


@dataclasses.dataclass(frozen=True)
class Format:
    name: str
    k_cap: float      # bits per token for keys (capacity)
    v_cap: float
    k_bw: float       # bits per token for keys actually read at the given n_keep
    v_bw: float
    n_prot: int       # BF16-protected tokens (sink + recent / residual)
    prot_k_bw: float  # key bits read for a protected token


def _formats(n_keep: int = 77) -> Dict[str, Format]:
    r = n_keep - 1  # INT2 channels read when channel 0 is among the kept channels
    bf = 16
    return {
        # ch0 in bf16 + 127 INT2 channels + one (scale, zero) per token; values
        # per-token INT2 + (scale, zero); 64 sink + 256 recent BF16 tokens.
        "dual-qk": Format("dual-qk", 127 * 2 + bf + 32, D * 2 + 32, r * 2 + bf + 32, D * 2 + 32, 64 + 256,
                          n_keep * bf),
        # same without channel-0 protection (all 128 channels INT2)
        "oscar": Format("oscar", D * 2 + 32, D * 2 + 32, n_keep * 2 + 32, D * 2 + 32, 64 + 256, n_keep * bf),
        # groups of 32 (keys per channel over tokens, values per token over
        # channels) with 32-bit metadata; 128 residual BF16 tokens
        "kivi": Format("kivi", D * 3, D * 3, n_keep * 3, D * 3, 128, n_keep * bf),
        # 3 bits per coordinate plus one 16-bit norm per vector, nothing protected
        "turboquant": Format("turboquant", D * 3 + bf, D * 3 + bf, n_keep * 3 + bf, D * 3 + bf, 0, n_keep * bf),
    }


def bits_per_element(fmt: str, n_tokens: int = 131072, n_keep: int = 77) -> Tuple[float, float]:
    """(capacity, bandwidth) effective bits per KV element."""
    f = _formats(n_keep)[fmt]
    denom = n_tokens * 2 * D
    prot_cap = 2 * D * 16
    prot_bw = f.prot_k_bw + D * 16
    q = n_tokens - f.n_prot
    cap = (q * (f.k_cap + f.v_cap) + f.n_prot * prot_cap) / denom
    bw = (q * (f.k_bw + f.v_bw) + f.n_prot * prot_bw) / denom
    return cap, bw


# ----------------------------------------------------------------------------
# This library's cache format (per page p, KV head g): k_codes 32 B per
# channel row, k_meta 4 B per channel, k_ch0 2 B per token, v_codes 32 B per
# token, v_meta 16 B per token (4 groups x fp16 scale + fp16 zero).

K_ROW_BYTES = 32
K_META_BYTES = 4
CH0_BYTES = 2
V_TOKEN_BYTES = 32 + 16
PAGE = 128


def bytes_per_token_head(n_keep: int, ch0_selected: bool = True) -> float:
    """Algorithmic cache bytes one decode step reads per (token, KV head)."""
    r = n_keep - (1 if ch0_selected else 0)
    return r * (K_ROW_BYTES + K_META_BYTES) / PAGE + (CH0_BYTES if ch0_selected else 0) + V_TOKEN_BYTES


def decode_cache_bytes(seq_lens, sel_idx) -> int:
    """Cache bytes a decode step must read, counting each KV head's actual
    selected set: per page the selected INT2 rows and their metadata, per
    valid token channel 0 (when selected) and the value codes and metadata."""
    total = 0
    B, hkv, _ = sel_idx.shape
    for b in range(B):
        L = int(seq_lens[b])
        pages = (L + PAGE - 1) // PAGE
        for g in range(hkv):
            sel = sel_idx[b, g]
            has0 = bool((sel == 0).any())
            r = len(sel) - (1 if has0 else 0)
            total += pages * r * (K_ROW_BYTES + K_META_BYTES) + L * ((CH0_BYTES if has0 else 0) + V_TOKEN_BYTES)
    return total


def decode_cache_bytes_tokgrid(seq_lens, sel_idx) -> int:
    """decode_cache_bytes for the per-token key grid layout: per page the
    selected INT2 rows (32 B each), per valid token its key (scale, zero)
    (4 B, read whatever the mask), channel 0 when selected, and the values."""
    total = 0
    B, hkv, _ = sel_idx.shape
    for b in range(B):
        L = int(seq_lens[b])
        pages = (L + PAGE - 1) // PAGE
        for g in range(hkv):
            sel = sel_idx[b, g]
            has0 = bool((sel == 0).any())
            r = len(sel) - (1 if has0 else 0)
            total += pages * r * K_ROW_BYTES + L * (K_META_BYTES + (CH0_BYTES if has0 else 0) + V_TOKEN_BYTES)
    return total


TIER_SINK, TIER_RECENT = 64, 256


def decode_rope_bytes(seq_lens, sel_idx) -> int:
    """decode_cache_bytes with bucket-relative RoPE: sel_idx [B][n_buckets]
    [Hkv][n_keep]; bucket k of sequence b (at most 2048 tokens, 16 pages) is
    read with its own selected set."""
    B, nb = sel_idx.shape[0], sel_idx.shape[1]
    lens = [max(0, min(2048, int(seq_lens[b]) - 2048 * k)) for b in range(B) for k in range(nb)]
    return decode_cache_bytes(lens, sel_idx.reshape(B * nb, *sel_idx.shape[2:]))


def tier_pages(L: int) -> int:
    """INT2 pages of a sequence of L tokens in the tiered layout: pages of
    tokens 64 + 128 i .., all older than the 256 most recent tokens."""
    return (L - TIER_SINK - TIER_RECENT) // PAGE if L >= TIER_SINK + TIER_RECENT else 0


def decode_tiered_bytes(seq_lens, sel_idx) -> int:
    """Cache bytes a tiered decode step reads: the INT2 pages as
    decode_cache_bytes, and per BF16 token (sink and tail) the selected
    channels of its bf16 k' plus its 128 bf16 values."""
    B, hkv, n_keep = sel_idx.shape
    int2 = decode_cache_bytes([PAGE * tier_pages(int(L)) for L in seq_lens], sel_idx)
    tier_tokens = sum(int(L) - PAGE * tier_pages(int(L)) for L in seq_lens)
    return int2 + tier_tokens * hkv * (n_keep * 2 + D * 2)


def decode_fixed_bytes(batch: int, hq: int, hkv: int, n_keep: int, max_pages: int) -> Dict[str, int]:
    """Per-step bytes outside the cache: the select step reads q (bf16) and
    T_Q (fp32) and writes q' and the selected indices; decode reads q', the
    indices and the page table and writes the fp32 output."""
    return {
        "select": batch * hq * D * 2 + hkv * D * D * 4 + batch * hq * D * 4 + batch * hkv * n_keep * 4,
        "decode": batch * hq * D * 4 + batch * hkv * n_keep * 4 + batch * max_pages * 4 + batch * hq * D * 4,
    }


def bf16_cache_bytes(seq_lens, hkv: int) -> int:
    return int(sum(int(L) for L in seq_lens)) * hkv * 2 * D * 2
