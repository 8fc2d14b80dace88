"""The C-ABI library loads, exports every entry point include/dqk.h declares,
and rejects bad arguments on the host before enqueueing anything (no GPU)."""
import ctypes
import os
import re

import pytest

import page_set_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dqk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dqk_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point():
    L = pa.lib()
    names = _declared()
    assert {"dqk_quantize_append", "dqk_select_channels", "dqk_decode_attn", "dqk_decode_workspace_size",
            "dqk_decode_attn_bf16", "dqk_status_string", "dqk_last_hip_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for st in (pa.DQK_OK, pa.DQK_ERR_NULL, pa.DQK_ERR_SHAPE, pa.DQK_ERR_ALIGN, pa.DQK_ERR_UNSUPPORTED,
               pa.DQK_ERR_WORKSPACE, pa.DQK_ERR_HIP):
        assert pa.lib().dqk_status_string(st)
    assert pa.lib().dqk_status_string(12345) == b"unknown status"


A = ctypes.c_void_p(4096)        # aligned, never dereferenced (validation fails first)
MIS = ctypes.c_void_p(4096 + 8)  # misaligned


def _sel(**kw):
    a = dict(q=A, tq=A, B=1, hq=32, hkv=8, nk=77, qp=A, sel=A)
    a.update(kw)
    return pa.lib().dqk_select_channels(a["q"], a["tq"], a["B"], a["hq"], a["hkv"], a["nk"], a["qp"], a["sel"], None)


def test_select_validation():
    assert _sel(q=None) == pa.DQK_ERR_NULL
    assert _sel(sel=None) == pa.DQK_ERR_NULL
    assert _sel(hq=30) == pa.DQK_ERR_SHAPE
    assert _sel(nk=0) == pa.DQK_ERR_SHAPE
    assert _sel(nk=129) == pa.DQK_ERR_SHAPE
    assert _sel(B=0) == pa.DQK_ERR_SHAPE
    assert _sel(hq=256, hkv=1) == pa.DQK_ERR_UNSUPPORTED
    assert _sel(tq=MIS) == pa.DQK_ERR_ALIGN


def _cache(**kw):
    c = pa.dqk_cache(8, 64, 4096, 4096, 4096, 4096, 4096)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _dec(c=None, **kw):
    c = c or _cache()
    a = dict(qp=A, sel=A, nk=77, B=4, hq=32, pt=A, mp=16, sl=A, sm=0.088, ns=0, ws=A, wsb=1 << 30, out=A, lse=None)
    a.update(kw)
    return pa.lib().dqk_decode_attn(ctypes.byref(c), a["qp"], a["sel"], a["nk"], a["B"], a["hq"], a["pt"], a["mp"],
                                    a["sl"], a["sm"], a["ns"], a["ws"], a["wsb"], a["out"], a["lse"], None)


def test_decode_validation():
    assert _dec(c=_cache(k_codes=None)) == pa.DQK_ERR_NULL
    assert _dec(qp=None) == pa.DQK_ERR_NULL
    assert _dec(ws=None) == pa.DQK_ERR_NULL
    assert _dec(hq=30) == pa.DQK_ERR_SHAPE
    assert _dec(nk=0) == pa.DQK_ERR_SHAPE
    assert _dec(ns=17) == pa.DQK_ERR_SHAPE
    assert _dec(c=_cache(num_kv_heads=0)) == pa.DQK_ERR_SHAPE
    assert _dec(c=_cache(num_pages=60)) == pa.DQK_ERR_SHAPE        # the pool is whole 8-page blocks
    assert _dec(hq=8 * 32) == pa.DQK_ERR_UNSUPPORTED          # group of 32 query heads
    assert _dec(c=_cache(v_meta=4096 + 2)) == pa.DQK_ERR_ALIGN
    assert _dec(lse=MIS) == pa.DQK_ERR_ALIGN
    need = pa.dqk_decode_workspace_size(4, 32, 8, 16, 4)
    assert need == 4 * 32 * 4 * 132 * 4
    assert _dec(ns=4, wsb=need - 4) == pa.DQK_ERR_WORKSPACE


def test_workspace_size():
    assert pa.dqk_decode_workspace_size(0, 32, 8, 16, 0) == 0
    assert pa.dqk_decode_workspace_size(2, 8, 8, 16, 3) == 2 * 8 * 3 * 132 * 4
    assert pa.dqk_decode_workspace_size(4, 32, 8, 1024, 0) >= 4 * 32 * 132 * 4


def test_append_validation():
    L = pa.lib()
    c = _cache()

    def app(c=c, **kw):
        a = dict(k=A, v=A, tk=A, n=2, cu=A, tot=300, pt=A, mp=4, dbg=None)
        a.update(kw)
        return L.dqk_quantize_append(ctypes.byref(c), a["k"], a["v"], a["tk"], a["n"], a["cu"], a["tot"], a["pt"],
                                     a["mp"], a["dbg"], None)

    assert app(k=None) == pa.DQK_ERR_NULL
    assert app(c=_cache(k_ch0=None)) == pa.DQK_ERR_NULL
    assert app(n=0) == pa.DQK_ERR_SHAPE
    assert app(tot=0) == pa.DQK_ERR_SHAPE
    assert app(dbg=MIS) == pa.DQK_ERR_ALIGN


def test_bf16_validation():
    L = pa.lib()

    def dec(**kw):
        a = dict(k=A, v=A, hkv=8, np_=64, q=A, B=2, hq=32, pt=A, mp=16, sl=A, ns=0, ws=A, wsb=1 << 30, out=A)
        a.update(kw)
        return L.dqk_decode_attn_bf16(a["k"], a["v"], a["hkv"], a["np_"], a["q"], a["B"], a["hq"], a["pt"], a["mp"],
                                      a["sl"], 0.088, a["ns"], a["ws"], a["wsb"], a["out"], None, None)

    assert dec(k=None) == pa.DQK_ERR_NULL
    assert dec(hq=31) == pa.DQK_ERR_SHAPE
    assert dec(wsb=64) == pa.DQK_ERR_WORKSPACE
    assert dec(q=MIS) == pa.DQK_ERR_ALIGN


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(pa, "_lib", None)
    monkeypatch.setattr(pa, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError):
        pa.lib()


def test_stream_read_validation():
    L = pa.lib()
    assert L.dqk_stream_read(None, 16384, A, None) == pa.DQK_ERR_NULL
    assert L.dqk_stream_read(A, 0, A, None) == pa.DQK_ERR_SHAPE
    assert L.dqk_stream_read(A, 16384 + 16, A, None) == pa.DQK_ERR_SHAPE
    assert L.dqk_stream_read(MIS, 16384, A, None) == pa.DQK_ERR_ALIGN


def _noalloc(c=None, **kw):
    c = c or _cache()
    a = dict(qp=A, sel=A, nk=77, B=4, hq=32, pt=A, mp=16, sl=A, sm=0.088, ns=0, out=A, lse=None)
    a.update(kw)
    return pa.lib().dqk_decode_attn_noalloc(ctypes.byref(c), a["qp"], a["sel"], a["nk"], a["B"], a["hq"], a["pt"],
                                            a["mp"], a["sl"], a["sm"], a["ns"], a["out"], a["lse"], None)


def test_noalloc_validation_before_any_device_call():
    """Shape errors and partials beyond the library's 16 MiB array are
    reported on the host, before the array's address is looked up."""
    assert pa.lib().dqk_decode_noalloc_max_bytes() == 16 << 20
    assert _noalloc(c=_cache(k_codes=None)) == pa.DQK_ERR_NULL
    assert _noalloc(hq=30) == pa.DQK_ERR_SHAPE
    assert _noalloc(ns=17) == pa.DQK_ERR_SHAPE
    # 64 sequences x 64 heads x 16 splits x 528 bytes = 33 MiB of partials
    assert _noalloc(c=pa.dqk_cache(16, 64, 4096, 4096, 4096, 4096, 4096), B=64, hq=64, ns=16) == pa.DQK_ERR_WORKSPACE


def _tiers(**kw):
    t = pa.dqk_tiers(4, 8, 4096, 4096, 4096, 4096, 4096)
    for k, v in kw.items():
        setattr(t, k, v)
    return t


def test_tiered_validation():
    """Every tier entry point rejects bad arguments on the host (nothing is
    enqueued, so no device is touched)."""
    L = pa.lib()
    c = _cache()

    def pre(t=None, **kw):
        a = dict(k=A, v=A, tk=A, n=2, cu=A, tot=300, pt=A, mp=4)
        a.update(kw)
        return L.dqk_prefill_tiered(ctypes.byref(c), ctypes.byref(t or _tiers()), a["k"], a["v"], a["tk"], a["n"],
                                    a["cu"], a["tot"], a["pt"], a["mp"], None)

    assert pre(t=_tiers(tail_kraw=None)) == pa.DQK_ERR_NULL
    assert pre(k=None) == pa.DQK_ERR_NULL
    assert pre(n=5) == pa.DQK_ERR_SHAPE                     # more sequences than the tiers hold
    assert pre(t=_tiers(num_kv_heads=4)) == pa.DQK_ERR_SHAPE  # head count differs from the cache's
    assert pre(t=_tiers(sink_v=4096 + 2)) == pa.DQK_ERR_ALIGN

    def app(t=None, **kw):
        a = dict(k=A, v=A, tk=A, B=4, lb=A, pt=A, mp=4)
        a.update(kw)
        return L.dqk_append_token(ctypes.byref(c), ctypes.byref(t or _tiers()), a["k"], a["v"], a["tk"], a["B"],
                                  a["lb"], a["pt"], a["mp"], None)

    assert app(lb=None) == pa.DQK_ERR_NULL
    assert app(B=0) == pa.DQK_ERR_SHAPE
    assert app(B=5) == pa.DQK_ERR_SHAPE
    assert app(pt=MIS) == pa.DQK_ERR_ALIGN

    def dec(t=None, **kw):
        a = dict(qp=A, sel=A, nk=77, B=4, hq=32, pt=A, mp=16, sl=A, ns=0, ws=A, wsb=1 << 30, out=A)
        a.update(kw)
        return L.dqk_decode_attn_tiered(ctypes.byref(c), ctypes.byref(t or _tiers()), a["qp"], a["sel"], a["nk"],
                                        a["B"], a["hq"], a["pt"], a["mp"], a["sl"], 0.088, a["ns"], a["ws"], a["wsb"],
                                        a["out"], None, None)

    assert dec(t=_tiers(sink_k=None)) == pa.DQK_ERR_NULL
    assert dec(hq=30) == pa.DQK_ERR_SHAPE
    assert dec(B=5) == pa.DQK_ERR_SHAPE
    need = pa.dqk_decode_tiered_workspace_size(4, 32, 8, 16, 4)
    assert need == 4 * 32 * 4 * 132 * 4 + 4 * 32 * 7 * 132 * 4 + 16   # 7 partials of 64 BF16 tokens
    assert dec(ns=4, wsb=need - 4) == pa.DQK_ERR_WORKSPACE
    assert dec(out=MIS) == pa.DQK_ERR_ALIGN


def test_vrot_validation():
    L = pa.lib()
    c = _cache()

    def app(c=c, **kw):
        a = dict(k=A, v=A, tk=A, rv=A, clip=0.92, n=2, cu=A, tot=300, pt=A, mp=4, kd=None, vd=None)
        a.update(kw)
        return L.dqk_quantize_append_vrot(ctypes.byref(c), a["k"], a["v"], a["tk"], a["rv"], a["clip"], a["n"],
                                          a["cu"], a["tot"], a["pt"], a["mp"], a["kd"], a["vd"], None)

    assert app(rv=None) == pa.DQK_ERR_NULL
    assert app(c=_cache(v_codes=None)) == pa.DQK_ERR_NULL
    for bad in (0.0, -0.5, 1.5, float("nan"), float("inf")):
        assert app(clip=bad) == pa.DQK_ERR_SHAPE, bad
    assert app(n=0) == pa.DQK_ERR_SHAPE
    assert app(rv=MIS) == pa.DQK_ERR_ALIGN
    assert app(vd=MIS) == pa.DQK_ERR_ALIGN

    def sel(**kw):
        a = dict(q=A, tq=A, sc=A, B=1, hq=32, hkv=8, nk=77, qp=A, si=A)
        a.update(kw)
        return L.dqk_select_channels_base(a["q"], a["tq"], a["sc"], a["B"], a["hq"], a["hkv"], a["nk"], a["qp"],
                                          a["si"], None)

    assert sel(sc=None) == pa.DQK_ERR_NULL
    assert sel(hq=30) == pa.DQK_ERR_SHAPE
    assert sel(nk=129) == pa.DQK_ERR_SHAPE
    assert sel(hq=256, hkv=1) == pa.DQK_ERR_UNSUPPORTED
    assert sel(sc=MIS) == pa.DQK_ERR_ALIGN

    def unrot(**kw):
        a = dict(o=A, r=A, B=4, hq=32, hkv=8, out=ctypes.c_void_p(1 << 20))
        a.update(kw)
        return L.dqk_value_unrotate(a["o"], a["r"], a["B"], a["hq"], a["hkv"], a["out"], None)

    assert unrot(r=None) == pa.DQK_ERR_NULL
    assert unrot(out=None) == pa.DQK_ERR_NULL
    assert unrot(out=A) == pa.DQK_ERR_UNSUPPORTED                             # in place
    assert unrot(out=ctypes.c_void_p(4096 + 4 * 32 * 512 - 16)) == pa.DQK_ERR_UNSUPPORTED  # overlapping
    assert unrot(hq=30) == pa.DQK_ERR_SHAPE
    assert unrot(B=0) == pa.DQK_ERR_SHAPE
    assert unrot(hq=65 * 2, hkv=2) == pa.DQK_ERR_UNSUPPORTED
    assert unrot(out=ctypes.c_void_p((1 << 20) + 8)) == pa.DQK_ERR_ALIGN


def test_one_call_vrot_validation():
    L = pa.lib()

    def call(c=None, **kw):
        c = c or _cache()
        a = dict(q=A, tq=A, sc=A, ri=A, nk=77, B=4, hq=32, pt=A, mp=16, sl=A, sm=0.088, ns=0, ws=A, wsb=1 << 30,
                 out=A, lse=None, qp=A, si=A)
        a.update(kw)
        return L.dqk_select_decode_attn_vrot(ctypes.byref(c), a["q"], a["tq"], a["sc"], a["ri"], a["nk"], a["B"],
                                             a["hq"], a["pt"], a["mp"], a["sl"], a["sm"], a["ns"], a["ws"], a["wsb"],
                                             a["out"], a["lse"], a["qp"], a["si"], None)

    assert call(sc=None) == pa.DQK_ERR_NULL
    assert call(ri=None) == pa.DQK_ERR_NULL
    assert call(q=None) == pa.DQK_ERR_NULL
    assert call(ri=MIS) == pa.DQK_ERR_ALIGN
    assert call(hq=30) == pa.DQK_ERR_SHAPE
    assert call(nk=0) == pa.DQK_ERR_SHAPE
    assert call(hq=8 * 32) == pa.DQK_ERR_UNSUPPORTED
    need = pa.dqk_decode_workspace_size(4, 32, 8, 16, 4)
    assert call(ns=4, wsb=need - 4) == pa.DQK_ERR_WORKSPACE


def test_rope_validation():
    L = pa.lib()
    c = _cache()

    def app(c=c, **kw):
        a = dict(k=A, v=A, tk=A, cs=A, sn=A, nb=1, n=2, cu=A, tot=300, pt=A, mp=4, kd=None)
        a.update(kw)
        return L.dqk_quantize_append_rope(ctypes.byref(c), a["k"], a["v"], a["tk"], a["cs"], a["sn"], a["nb"],
                                          a["n"], a["cu"], a["tot"], a["pt"], a["mp"], a["kd"], None)

    assert app(cs=None) == pa.DQK_ERR_NULL
    assert app(sn=None) == pa.DQK_ERR_NULL
    assert app(nb=0) == pa.DQK_ERR_SHAPE
    assert app(nb=1, mp=17) == pa.DQK_ERR_SHAPE          # pages 16.. have no table
    assert app(n=0) == pa.DQK_ERR_SHAPE
    assert app(sn=MIS) == pa.DQK_ERR_ALIGN

    def sel(**kw):
        a = dict(q=A, tq=A, cs=A, sn=A, nb=4, B=2, hq=32, hkv=8, nk=77, qp=A, si=A)
        a.update(kw)
        return L.dqk_select_channels_rope(a["q"], a["tq"], a["cs"], a["sn"], a["nb"], a["B"], a["hq"], a["hkv"],
                                          a["nk"], a["qp"], a["si"], None)

    assert sel(cs=None) == pa.DQK_ERR_NULL
    assert sel(nb=0) == pa.DQK_ERR_SHAPE
    assert sel(hq=30) == pa.DQK_ERR_SHAPE
    assert sel(nk=129) == pa.DQK_ERR_SHAPE
    assert sel(B=1024, nb=64) == pa.DQK_ERR_UNSUPPORTED   # 65536 (sequence, bucket) rows
    assert sel(cs=MIS) == pa.DQK_ERR_ALIGN

    def dec(c=None, one=False, **kw):
        c = c or _cache()
        a = dict(q=A, tq=A, cs=A, sn=A, qp=A, si=A, nk=77, nb=4, B=2, hq=32, pt=A, mp=64, sl=A, sm=0.088, ns=0,
                 ws=A, wsb=1 << 30, out=A, lse=None)
        a.update(kw)
        if one:
            return L.dqk_select_decode_attn_rope(ctypes.byref(c), a["q"], a["tq"], a["cs"], a["sn"], a["nk"],
                                                 a["nb"], a["B"], a["hq"], a["pt"], a["mp"], a["sl"], a["sm"],
                                                 a["ns"], a["ws"], a["wsb"], a["out"], a["lse"], a["qp"], a["si"],
                                                 None)
        return L.dqk_decode_attn_rope(ctypes.byref(c), a["qp"], a["si"], a["nk"], a["nb"], a["B"], a["hq"],
                                      a["pt"], a["mp"], a["sl"], a["sm"], a["ns"], a["ws"], a["wsb"], a["out"],
                                      a["lse"], None)

    for one in (False, True):
        assert dec(one=one, sl=None) == pa.DQK_ERR_NULL
        assert dec(one=one, nb=3) == pa.DQK_ERR_SHAPE          # 48 pages < max_pages 64
        assert dec(one=one, nb=0) == pa.DQK_ERR_SHAPE
        assert dec(one=one, ns=65) == pa.DQK_ERR_SHAPE          # more splits than pages
        assert dec(one=one, hq=30) == pa.DQK_ERR_SHAPE
        assert dec(one=one, hq=8 * 32) == pa.DQK_ERR_UNSUPPORTED
        assert dec(one=one, B=2048, nb=64, mp=1024) == pa.DQK_ERR_UNSUPPORTED
        assert dec(one=one, out=MIS) == pa.DQK_ERR_ALIGN
        need = pa.dqk_decode_rope_workspace_size(2, 32, 8, 4, 2)
        assert need == 2 * 32 * 2 * 132 * 4                     # partials per sequence and split
        assert dec(one=one, ns=2, wsb=need - 4) == pa.DQK_ERR_WORKSPACE
    assert dec(one=True, q=None) == pa.DQK_ERR_NULL
    assert dec(one=True, cs=None) == pa.DQK_ERR_NULL
    assert dec(one=True, qp=None) == pa.DQK_ERR_NULL
    assert dec(one=True, sn=MIS) == pa.DQK_ERR_ALIGN
    assert dec(one=False, si=None) == pa.DQK_ERR_NULL
    assert dec(one=False, qp=MIS) == pa.DQK_ERR_ALIGN
    assert pa.dqk_decode_rope_workspace_size(2, 32, 8, 0, 0) == 0


def test_one_call_tiered_validation():
    """dqk_select_decode_attn_tiered rejects bad arguments on the host before
    anything is enqueued (no device is touched)."""
    L = pa.lib()
    c = _cache()

    def one(t=None, **kw):
        a = dict(q=A, tq=A, nk=77, B=4, hq=32, pt=A, mp=16, sl=A, ns=0, ws=A, wsb=1 << 30, out=A, qp=A, sel=A)
        a.update(kw)
        return L.dqk_select_decode_attn_tiered(ctypes.byref(c), ctypes.byref(t or _tiers()), a["q"], a["tq"],
                                               a["nk"], a["B"], a["hq"], a["pt"], a["mp"], a["sl"], 0.088, a["ns"],
                                               a["ws"], a["wsb"], a["out"], None, a["qp"], a["sel"], None)

    assert one(t=_tiers(sink_k=None)) == pa.DQK_ERR_NULL
    assert one(q=None) == pa.DQK_ERR_NULL
    assert one(sel=None) == pa.DQK_ERR_NULL
    assert one(hq=30) == pa.DQK_ERR_SHAPE
    assert one(B=5) == pa.DQK_ERR_SHAPE                      # more sequences than the tiers hold
    assert one(nk=0) == pa.DQK_ERR_SHAPE
    assert one(hq=8 * 17) == pa.DQK_ERR_UNSUPPORTED          # more query heads per KV head than the decode serves
    need = pa.dqk_decode_tiered_workspace_size(4, 32, 8, 16, 4)
    assert one(ns=4, wsb=need - 4) == pa.DQK_ERR_WORKSPACE
    assert one(qp=MIS) == pa.DQK_ERR_ALIGN
    assert one(tq=MIS) == pa.DQK_ERR_ALIGN
