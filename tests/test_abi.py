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
    assert _dec(hq=8 * 32) == pa.DQK_ERR_UNSUPPORTED          # group of 32 query heads
    assert _dec(c=_cache(v_meta=4096 + 2)) == pa.DQK_ERR_ALIGN
    assert _dec(lse=MIS) == pa.DQK_ERR_ALIGN
    need = pa.dqk_decode_workspace_size(4, 32, 8, 16, 4)
    assert need == 4 * 32 * 4 * 130 * 4
    assert _dec(ns=4, wsb=need - 4) == pa.DQK_ERR_WORKSPACE


def test_workspace_size():
    assert pa.dqk_decode_workspace_size(0, 32, 8, 16, 0) == 0
    assert pa.dqk_decode_workspace_size(2, 8, 8, 16, 3) == 2 * 8 * 3 * 130 * 4
    assert pa.dqk_decode_workspace_size(4, 32, 8, 1024, 0) >= 4 * 32 * 130 * 4


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
