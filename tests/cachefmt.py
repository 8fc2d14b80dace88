"""Independent numpy reader of the paged INT2 cache format (test helper).

Layout (key rows and key metadata in aligned blocks of eight pages; page p
is slot p & 7 of block p >> 3):
  k_codes u8 [P/8][Hkv][128 ch][8][32]  token t at byte t>>2, bits 2*(t&3)
  k_meta f16 [P/8][Hkv][128 ch][8][2]   (scale, zero)
  k_ch0 bf16 [P][Hkv][128 tok]
  v_codes u8 [P][Hkv][128 tok][32]  channel c at byte c>>2, bits 2*(c&3)
  v_meta f16 [P][Hkv][2][4][128]    [0]=scale, [1]=zero per (group, token)
Dequantized value = code * scale + zero; code*scale is exact in fp32 (binary16
scale times an integer below 4), so fp32 multiply-then-add equals fmaf.
"""
import numpy as np


def f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def bf16(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def unpack_rows(rows: np.ndarray) -> np.ndarray:
    """[..., 32] bytes -> [..., 128] 2-bit fields, little-endian within bytes."""
    r = rows.astype(np.uint8)
    fields = np.stack([(r >> (2 * i)) & 3 for i in range(4)], axis=-1)  # [...,32,4]
    return fields.reshape(*rows.shape[:-1], 128)


def k_codes(cache, p, g):
    """codes [128 ch][128 tok]"""
    return unpack_rows(cache.k_codes[p >> 3, g, :, p & 7])


def v_codes(cache, p, g):
    """codes [128 tok][128 ch]"""
    return unpack_rows(cache.v_codes[p, g])


def decode_k(cache, p, g):
    """Dequantized k' of a page: [128 tok][128 ch] fp32 (channel 0 from bf16)."""
    c = k_codes(cache, p, g).astype(np.float32)            # [ch][tok]
    s = f16(cache.k_meta[p >> 3, g, :, p & 7, 0])[:, None]
    z = f16(cache.k_meta[p >> 3, g, :, p & 7, 1])[:, None]
    k = (c * s + z).T.copy()
    k[:, 0] = bf16(cache.k_ch0[p, g])
    return k


def decode_v(cache, p, g):
    c = v_codes(cache, p, g).astype(np.float32)            # [tok][ch]
    s = f16(cache.v_meta[p, g, 0])                           # [4][tok]
    z = f16(cache.v_meta[p, g, 1])
    grp = np.arange(128) // 32
    return c * s[grp].T + z[grp].T


def gather_seq(cache, page_table, b, L, g):
    """Dequantized (k', v) of sequence b, KV head g: [L][128] each."""
    ks, vs = [], []
    for pi in range((L + 127) // 128):
        p = int(page_table[b, pi])
        ks.append(decode_k(cache, p, g))
        vs.append(decode_v(cache, p, g))
    return np.concatenate(ks)[:L], np.concatenate(vs)[:L]


def gather_vparts(cache, page_table, b, L, g):
    """Value codes [L][128], scales and zero points [L][128] (each channel's
    group metadata) of sequence b, KV head g."""
    cs, ss, zs = [], [], []
    grp = np.arange(128) // 32
    for pi in range((L + 127) // 128):
        p = int(page_table[b, pi])
        cs.append(v_codes(cache, p, g))
        ss.append(f16(cache.v_meta[p, g, 0])[grp].T)
        zs.append(f16(cache.v_meta[p, g, 1])[grp].T)
    return np.concatenate(cs)[:L], np.concatenate(ss)[:L], np.concatenate(zs)[:L]


def k_token_meta(cache, p, g):
    """Per-token key (scale, zero) of page p, KV head g in the per-token grid
    layout k_meta [P/8][Hkv][8 slot][128 tok][2] (the block's metadata bytes
    read token-major): fp32 arrays [128] each."""
    flat = cache.k_meta.reshape(cache.k_meta.shape[0], cache.k_meta.shape[1], -1)   # [P/8][Hkv][2048]
    m = flat[p >> 3, g].reshape(8, 128, 2)[p & 7]
    return f16(m[:, 0]), f16(m[:, 1])


def decode_k_tokgrid(cache, p, g):
    """Dequantized k' of a page with per-token grids: [128 tok][128 ch] fp32."""
    c = k_codes(cache, p, g).astype(np.float32).T             # [tok][ch]
    s, z = k_token_meta(cache, p, g)
    k = c * s[:, None] + z[:, None]
    k[:, 0] = bf16(cache.k_ch0[p, g])
    return k


def gather_seq_tokgrid(cache, page_table, b, L, g):
    ks, vs = [], []
    for pi in range((L + 127) // 128):
        p = int(page_table[b, pi])
        ks.append(decode_k_tokgrid(cache, p, g))
        vs.append(decode_v(cache, p, g))
    return np.concatenate(ks)[:L], np.concatenate(vs)[:L]
