#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Workload (default): batch 4, GQA 32 query / 8 KV heads, head_dim 128, 131072
tokens of context per sequence, INT2 keys/values with channel 0 in bf16, 40%
query-channel sparsity (77 of 128 channels kept).  One step = one decode step
of one attention layer: dqk_select_channels (q' = q T_Q, pooled-energy top-k)
followed by dqk_decode_attn (split-K decode + log-sum-exp merge) over the
whole batch.  Inputs are seeded synthetic data (see synth/), already resident
in HBM; the INT2 cache is built once on the GPU by dqk_quantize_append.  Each
step reads a different one of several identical cache copies so that no step
finds its cache in the 256 MB Infinity Cache.

Prints one JSON line (metric, value = decode-attention tokens/s, roofline of
the decode kernel, CPU-oracle baseline on a bounded sample).
"""
import argparse
import concurrent.futures as cf
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "decode-attn tokens/s @128K, INT2 KV, 40% q-prune; achieved HBM GB/s %"
PEAK_HBM_GBS = 8000.0
DECODE_SOURCES = ["page_set_amd/csrc/dqk_decode_blk.hip", "page_set_amd/csrc/dqk_decode.hip",
                  "page_set_amd/csrc/dqk_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash():
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel_hash):
    """HBM traffic per decode launch from committed rocprofv3 PMC runs, if the
    decode kernel has not changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_hash") != kernel_hash:
        return None
    return rec


def _counter_means(path, counter):
    """Per-dispatch mean of one counter for every kernel name in a rocprofv3 counter CSV."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic(fetch_csv, write_csv, out_json):
    """HBM bytes per decode launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the 1 GiB copy of --calib-copy
    (1 GiB read, 1 GiB written)."""
    fetch, write = _counter_means(fetch_csv, "FETCH_SIZE"), _counter_means(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "elementwise" in k and "Mul" in k]
    if not copy:
        copy = [k for k in fetch if "elementwise" in k]
    copy_f = max(fetch[k] for k in copy)
    copy_w = max(write.get(k, 0.0) for k in copy)
    gib_kib = float(1 << 20)
    ff, fw = gib_kib / copy_f, gib_kib / copy_w
    rec = {"kernel_hash": source_hash(), "fetch_scale": round(ff, 4), "write_scale": round(fw, 4),
           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w, "kernels": {}}
    total = 0.0
    for k in fetch:  # the one-call entry's kernels: the decode with the selection inside, then the merge
        if ("decode_blk_kernel" in k and "true>" in k) or "merge_kernel" in k:
            b = fetch[k] * 1024 * ff + write.get(k, 0.0) * 1024 * fw
            rec["kernels"][k[:60]] = {"fetch_kib": fetch[k], "write_kib": write.get(k, 0.0), "hbm_bytes": b}
            total += b
    rec["hbm_bytes_per_launch"] = total
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def build_cache(prob, shape, d, pa, torch, one_call=False):
    """Pack the whole batch into the INT2 cache on the GPU (dqk_quantize_append,
    inputs resident in HBM); each append call is timed with HIP events on its
    stream.  Sequence by sequence by default; `one_call` appends the whole
    ragged batch in a single call (cu_tokens over all sequences)."""
    cache = pa.Cache(prob.num_pages, shape.hkv)
    times, tokens = [], 0
    stream = torch.cuda.current_stream()

    def timed(k_d, v_d, cu, pt, warm):
        if warm:  # untimed first call (loads the code object); rewrites the same pages
            pa.dqk_quantize_append(cache, k_d, v_d, d["t_k"], cu, pt, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pa.dqk_quantize_append(cache, k_d, v_d, d["t_k"], cu, pt, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        futs = [ex.submit(synth.make_kv_seq, shape, prob.seed, b, prob.outliers) for b in range(shape.batch)]
        if one_call:
            kk, vv = zip(*[f.result() for f in futs])
            k_d = torch.from_numpy(np.concatenate(kk).view(np.int16)).to("cuda")
            v_d = torch.from_numpy(np.concatenate(vv).view(np.int16)).to("cuda")
            del kk, vv
            timed(k_d, v_d, d["cu"], d["page_table"], True)
            tokens = int(k_d.shape[0])
            del k_d, v_d
            return cache, sum(times), tokens
        for b, f in enumerate(futs):
            kb, vb = f.result()
            L = kb.shape[0]
            k_d = torch.from_numpy(kb.view(np.int16)).to("cuda")
            v_d = torch.from_numpy(vb.view(np.int16)).to("cuda")
            cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
            timed(k_d, v_d, cu, d["page_table"][b:b + 1].clone(), b == 0)
            tokens += L
            del k_d, v_d
    return cache, sum(times), tokens


def build_bf16_pages(prob, shape, torch):
    """The unpruned BF16 cache of the baseline: raw keys and values laid out in
    128-token pages [page][Hkv][128 tok][128 ch] on the GPU (page table as in
    the INT2 cache)."""
    kp = torch.zeros((prob.num_pages, shape.hkv, 128, 128), dtype=torch.int16, device="cuda")
    vp = torch.zeros_like(kp)
    for b in range(shape.batch):
        kb, vb = synth.make_kv_seq(shape, prob.seed, b, prob.outliers)
        L = kb.shape[0]
        npg = (L + 127) // 128
        pages = torch.from_numpy(prob.page_table[b, :npg].astype(np.int64)).to("cuda")
        for src, dst in ((kb, kp), (vb, vp)):
            x = torch.zeros((npg * 128, shape.hkv, 128), dtype=torch.int16, device="cuda")
            x[:L] = torch.from_numpy(src.view(np.int16)).to("cuda")
            dst[pages] = x.view(npg, 128, shape.hkv, 128).permute(0, 2, 1, 3)
            del x
    return kp, vp


def append_roofline(seconds, tokens, pages, hkv):
    """Quantize-append: bf16 K and V read, INT2 pages written; K x T_K on MFMA."""
    rd = tokens * hkv * 128 * 2 * 2 + hkv * 128 * 128 * 2
    wr = pages * hkv * (128 * 32 + 128 * 4 + 128 * 2 + 128 * 32 + 2048)
    flops = 2.0 * tokens * hkv * 128 * 128
    gbs = (rd + wr) / seconds / 1e9
    tfs = flops / seconds / 1e12
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": int(rd + wr), "seconds": round(seconds, 6),
            "mfma_tflops": round(tfs, 2), "mfma_peak_tflops": 2500.0, "mfma_frac": round(tfs / 2500.0, 4),
            "tokens": int(tokens)}


def stream_read_gbs(torch, pa, nbytes):
    """Read bandwidth of dqk_stream_read (a plain streaming read through LDS) over a
    buffer of the same size as the decode call's algorithmic bytes: the box's
    practical ceiling for this traffic, for context."""
    blk = 16384 * 4096  # 4096 single-wave workgroups of whole 16 KiB units
    n = max(blk, nbytes // blk * blk)
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pa.dqk_stream_read(x, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        pa.dqk_stream_read(x, sink)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 10
    del x, sink
    return n / t / 1e9


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, seed, n_keep, max_workers=16):
    """The CPU oracle (as written: single-threaded C, fp64) on the same workload,
    on a bounded sample of its (sequence, KV head) units.  Each unit's cache is
    built by the oracle from the same seeded inputs; then `w` units are decoded
    at once on `w` host threads (ctypes releases the GIL, so the oracle calls
    run in parallel), and one unit is decoded alone for the single-core figure.
    Step time = units per step x the per-unit time / threads."""
    import oracle
    prob = synth.make_problem(shape, seed, materialize_kv=False)
    grp = shape.hq // shape.hkv
    units_all = shape.batch * shape.hkv
    w = max(1, min(max_workers, os.cpu_count() or 1, units_all))
    units = [(u // shape.hkv, u % shape.hkv) for u in range(w)]

    kv = {}
    for b in sorted({b for b, _ in units}):
        kb, vb = synth.make_kv_seq(shape, seed, b, prob.outliers)
        for bb, g in units:
            if bb == b:
                kv[(b, g)] = (np.ascontiguousarray(kb[:, g:g + 1]), np.ascontiguousarray(vb[:, g:g + 1]))
        del kb, vb

    def build(unit):
        b, g = unit
        kk, vv = kv[unit]
        L = kk.shape[0]
        npg = (L + 127) // 128
        pt = np.arange(npg, dtype=np.int32)[None]
        cache, _ = oracle.quantize_append(kk, vv, prob.t_k[g:g + 1], np.array([0, L], np.int32), pt, npg)
        q = np.ascontiguousarray(prob.q[b:b + 1, g * grp:(g + 1) * grp])
        return cache, q, pt, np.array([L], np.int32), prob.t_q[g:g + 1]

    def run(args):
        cache, q, pt, lens, tq = args
        t0 = time.perf_counter()
        qp, sel = oracle.select_channels(q, tq, 1, n_keep)
        oracle.decode_attn(cache, qp, sel, pt, lens, prob.sm_scale)
        return time.perf_counter() - t0

    with cf.ThreadPoolExecutor(max_workers=w) as ex:
        built = list(ex.map(build, units))
        kv.clear()
        t0 = time.perf_counter()
        per_unit = list(ex.map(run, built))
        wall = time.perf_counter() - t0
    single = min(run(built[0]) for _ in range(2))
    t_step_all = units_all * wall / w
    t_step_one = units_all * single
    L = shape.seq_lens[0]
    return {"value": round(shape.batch / t_step_all, 4), "unit": "tokens/s", "cores": w, "kind": "oracle",
            "single_core_value": round(shape.batch / t_step_one, 4), "nproc": os.cpu_count(),
            "cpu_model": _cpu_model(),
            "sample": f"{w} of the {units_all} (sequence, KV head) units of the workload ({grp} query heads x "
                      f"{L} tokens each), select + decode by the oracle: {w} units at once on {w} threads took "
                      f"{wall:.2f} s (per unit {min(per_unit):.2f}-{max(per_unit):.2f} s), one unit alone "
                      f"{single:.2f} s; step time = {units_all} units x unit time / threads"}


def _copies_for(nbytes, target=1 << 30, cap=48):
    """Cache copies rotated across steps so that one pass over all of them
    exceeds the 256 MB Infinity Cache several times over."""
    return int(max(2, min(cap, -(-target // max(1, nbytes)))))


class Int2Workload:
    """One INT2 decode workload resident on the GPU: inputs, cache copies and
    output buffers of a config."""

    def __init__(self, shape, seed, pa, torch, one_call=False):
        self.shape, self.pa, self.torch = shape, pa, torch
        self.prob = synth.make_problem(shape, seed, materialize_kv=False)
        p = self.prob
        self.d = {"q": torch.from_numpy(p.q.view(np.int16)).to("cuda"),
                  "t_q": torch.from_numpy(p.t_q).to("cuda"),
                  "t_k": torch.from_numpy(p.t_k.view(np.int16)).to("cuda"),
                  "page_table": torch.from_numpy(p.page_table).to("cuda"),
                  "seq_lens": torch.from_numpy(p.seq_lens).to("cuda"),
                  "cu": torch.from_numpy(p.cu_tokens).to("cuda")}
        cache, self.append_s, self.append_tokens = build_cache(p, shape, self.d, pa, torch, one_call=one_call)
        self.caches = [cache]
        for _ in range(_copies_for(cache.nbytes()) - 1):
            c2 = pa.Cache(cache.num_pages, cache.num_kv_heads)
            for a, b in zip(cache.arrays(), c2.arrays()):
                b.copy_(a)
            self.caches.append(c2)
        torch.cuda.synchronize()
        self.max_pages = int(p.page_table.shape[1])

    def time_steps(self, n_keep, steps, warmup, num_splits=0, fused=False):
        """Wall time per step over `steps` steps (synchronised on both sides),
        plus HIP-event averages of the select and decode calls on their stream
        (fused: the one-call select + decode; its time is reported as the
        decode call's and the select time is 0)."""
        torch, pa, sh = self.torch, self.pa, self.shape
        B, hq, hkv = sh.batch, sh.hq, sh.hkv
        q_prime = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
        sel = torch.empty((B, hkv, n_keep), dtype=torch.int32, device="cuda")
        out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
        ws_bytes = pa.dqk_decode_workspace_size(B, hq, hkv, self.max_pages, num_splits)
        ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
        ws_bytes = ws.numel() * 4
        stream = torch.cuda.current_stream()
        d = self.d

        nc = len(self.caches)
        mp = self.max_pages
        if fused:  # selection inside the decode launch (one call)
            calls = [[pa.prepared("dqk_select_decode_attn", c, d["q"], d["t_q"], n_keep, B, hq, d["page_table"], mp,
                                  d["seq_lens"], float(self.prob.sm_scale), int(num_splits), ws, ws_bytes, out,
                                  None, q_prime, sel, stream)] for c in self.caches]
        else:
            calls = [[pa.prepared("dqk_select_channels", d["q"], d["t_q"], B, hq, hkv, n_keep, q_prime, sel, stream),
                      pa.prepared("dqk_decode_attn", c, q_prime, sel, n_keep, B, hq, d["page_table"], mp,
                                  d["seq_lens"], float(self.prob.sm_scale), int(num_splits), ws, ws_bytes, out,
                                  None, stream)] for c in self.caches]

        def step(i, ev=None):
            fs = calls[i % nc]
            if ev is not None:
                ev[0].record(stream)
            if len(fs) == 2:
                fs[0]()
            if ev is not None:
                ev[1].record(stream)
            fs[-1]()
            if ev is not None:
                ev[2].record(stream)

        for i in range(warmup):
            step(i)
        # wall clock over exactly `steps` steps, nothing but the launches in the loop
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        # per-call GPU times from HIP events on the stream (a separate pass)
        ne = min(steps, 30)
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(ne)]
        for i in range(ne):
            step(i, evs[i])
        torch.cuda.synchronize()
        sel_us = [a.elapsed_time(b) * 1e3 for a, b, _ in evs]
        dec_us = [b.elapsed_time(c) * 1e3 for _, b, c in evs]
        sel_h = sel.cpu().numpy()
        from page_set_amd import traffic
        cache_bytes = traffic.decode_cache_bytes(self.prob.seq_lens, sel_h)
        fixed = traffic.decode_fixed_bytes(B, hq, hkv, n_keep, self.max_pages)
        return {"t_step_us": wall * 1e6, "select_us": float(np.mean(sel_us)), "decode_us": float(np.mean(dec_us)),
                "decode_p10_us": float(np.percentile(dec_us, 10)), "decode_p90_us": float(np.percentile(dec_us, 90)),
                "cache_bytes": cache_bytes, "decode_bytes": cache_bytes + fixed["decode"],
                "step_bytes": cache_bytes + fixed["decode"] + fixed["select"],
                "bytes_per_token_head": cache_bytes / (hkv * float(np.sum(self.prob.seq_lens)))}


def tiered_record(shape, seed, pa, torch, steps):
    """The headline workload in the protected-tier layout: one prefill call
    into the BF16 sink/tail tiers and the INT2 pages; a step is one
    dqk_select_decode_attn_tiered call (wall clock per step over cache copies
    rotated as for the headline, the two-call form beside it); then one
    appended token per sequence per call on the first copy, each timed with
    HIP events on the stream."""
    from page_set_amd import traffic
    prob = synth.make_problem(shape, seed, materialize_kv=False)
    B, hq, hkv, n_keep = shape.batch, shape.hq, shape.hkv, shape.n_keep
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    q, t_q, t_k = dev(prob.q.view(np.int16)), dev(prob.t_q), dev(prob.t_k.view(np.int16))
    pt, cu = dev(prob.page_table), dev(prob.cu_tokens)
    kv = [synth.make_kv_seq(shape, seed, b, prob.outliers) for b in range(B)]
    k_d = dev(np.concatenate([x[0] for x in kv]).view(np.int16))
    v_d = dev(np.concatenate([x[1] for x in kv]).view(np.int16))
    extra = [kv[b][0][-1:].copy() for b in range(B)]  # the token appended each step (its position grows)
    del kv
    cache = pa.Cache(prob.num_pages, hkv)
    tiers = pa.Tiers(B, hkv)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pa.dqk_prefill_tiered(cache, tiers, k_d, v_d, t_k, cu, pt)  # warm
    torch.cuda.synchronize()
    e0.record(stream)
    pa.dqk_prefill_tiered(cache, tiers, k_d, v_d, t_k, cu, pt)
    e1.record(stream)
    torch.cuda.synchronize()
    prefill_us = e0.elapsed_time(e1) * 1e3
    del k_d, v_d
    lens = dev(prob.seq_lens)
    qp = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, hkv, n_keep), dtype=torch.int32, device="cuda")
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    mp = int(prob.page_table.shape[1])
    ws_n = pa.dqk_decode_tiered_workspace_size(B, hq, hkv, mp, 0)
    ws = torch.empty(ws_n // 4 + 4, dtype=torch.float32, device="cuda")
    kn = dev(np.concatenate(extra).reshape(B, hkv, 128).view(np.int16))
    vn = torch.zeros_like(kn)
    # copies of the cache and tiers, rotated across steps as for the headline,
    # so that a step does not find its cache in the Infinity Cache
    n_cp = _copies_for(cache.nbytes())
    copies = [(cache, tiers)]
    for _ in range(n_cp - 1):
        c2, t2 = pa.Cache(cache.num_pages, hkv), pa.Tiers(B, hkv)
        for a, b in list(zip(cache.arrays(), c2.arrays())) + list(zip(tiers.arrays(), t2.arrays())):
            b.copy_(a)
        copies.append((c2, t2))
    torch.cuda.synchronize()
    sel_call = pa.prepared("dqk_select_channels", q, t_q, B, hq, hkv, n_keep, qp, sel, stream)
    dec_calls = [pa.prepared("dqk_decode_attn_tiered", c, t, qp, sel, n_keep, B, hq, pt, mp, lens,
                             float(prob.sm_scale), 0, ws, ws.numel() * 4, out, None, stream) for c, t in copies]
    one_calls = [pa.prepared("dqk_select_decode_attn_tiered", c, t, q, t_q, n_keep, B, hq, pt, mp, lens,
                             float(prob.sm_scale), 0, ws, ws.numel() * 4, out, None, qp, sel, stream)
                 for c, t in copies]

    def wall(fn, n):
        for i in range(100):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    def two(i):
        sel_call()
        dec_calls[i % n_cp]()

    # the step: one dqk_select_decode_attn_tiered call; it and the two-call
    # form are timed alternately, twice each, and the better of each is kept
    t_step, t_two = float("inf"), float("inf")
    for _ in range(2):
        t_step = min(t_step, wall(lambda i: one_calls[i % n_cp](), steps))
        t_two = min(t_two, wall(two, steps))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        dec_calls[i % n_cp]()
        b.record(stream)
    torch.cuda.synchronize()
    dec_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evs]))
    del copies[1:], dec_calls, one_calls
    # appends: one token per sequence per call, 128 calls, so that each sequence
    # packs one page from its tail on the way (the page table has room for it)
    n_app = 128
    assert int(max(traffic.tier_pages(int(L) + n_app) for L in prob.seq_lens)) < mp
    app_evs = []
    for _ in range(n_app):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        pa.dqk_append_token(cache, tiers, kn, vn, t_k, lens, pt, stream=stream)
        b.record(stream)
        app_evs.append((a, b))
        lens += 1
    torch.cuda.synchronize()
    app_us = [a.elapsed_time(b) * 1e3 for a, b in app_evs]
    sel_h = sel.cpu().numpy()
    cache_bytes = traffic.decode_tiered_bytes(prob.seq_lens, sel_h)
    fixed = traffic.decode_fixed_bytes(B, hq, hkv, n_keep, mp)
    step_bytes = cache_bytes + fixed["decode"] + fixed["select"]
    return {"workload": shape.name + "-tiered",
            "entry": "dqk_select_decode_attn_tiered (selection, BF16 tokens, INT2 decode, merge)",
            "t_step_us": round(t_step * 1e6, 2), "tokens_per_s": round(B / t_step, 1),
            "two_calls": {"entries": "dqk_select_channels + dqk_decode_attn_tiered", "t_step_us": round(t_two * 1e6, 2),
                          "decode_call_us": round(dec_us, 2)},
            "algorithmic_bytes_per_step": int(step_bytes),
            "frac_step": round(step_bytes / t_step / 1e9 / PEAK_HBM_GBS, 4), "cache_copies": n_cp,
            "prefill_us": round(prefill_us, 1), "append_token_us": round(float(np.median(app_us)), 2),
            "append_token_max_us": round(float(np.max(app_us)), 2),
            "append_note": "median and max over 128 calls, one token per sequence each; the max includes "
                           "packing a page from the tail"}


def vrot_record(shape, seed, pa, torch, steps, clip=0.92):
    """The headline workload with rotated, clipped values and selection in base
    coordinates: the cache is built sequence by sequence with
    dqk_quantize_append_vrot (HIP events), then a step is one
    dqk_select_decode_attn_vrot call (base selection in the decode launch, the
    inverse rotation in the merge) over cache copies rotated as in the
    headline; the same step as three calls (dqk_select_channels_base +
    dqk_decode_attn + dqk_value_unrotate) is reported beside it."""
    from page_set_amd import traffic
    prob = synth.make_problem(shape, seed, materialize_kv=False)
    B, hq, hkv, n_keep = shape.batch, shape.hq, shape.hkv, shape.n_keep
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    rv, rinv = synth.make_value_rotation(hkv, seed)
    wsel = synth.make_selection_scales(hkv, seed)
    q, t_q, t_k = dev(prob.q.view(np.int16)), dev(prob.t_q), dev(prob.t_k.view(np.int16))
    rv_d, rinv_d, w_d = dev(rv.view(np.int16)), dev(rinv), dev(wsel)
    pt, lens = dev(prob.page_table), dev(prob.seq_lens)
    mp = int(prob.page_table.shape[1])
    stream = torch.cuda.current_stream()
    cache = pa.Cache(prob.num_pages, hkv)
    app_s, tokens = 0.0, 0
    for b in range(B):
        kb, vb = synth.make_kv_seq(shape, seed, b, prob.outliers)
        L = kb.shape[0]
        k_d, v_d = dev(kb.view(np.int16)), dev(vb.view(np.int16))
        cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        ptb = pt[b:b + 1].clone()
        if b == 0:  # untimed first call
            pa.dqk_quantize_append_vrot(cache, k_d, v_d, t_k, rv_d, clip, cu, ptb, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pa.dqk_quantize_append_vrot(cache, k_d, v_d, t_k, rv_d, clip, cu, ptb, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        app_s += e0.elapsed_time(e1) * 1e-3
        tokens += L
        del k_d, v_d
    caches = [cache]
    for _ in range(_copies_for(cache.nbytes()) - 1):
        c2 = pa.Cache(cache.num_pages, hkv)
        for a, b2 in zip(cache.arrays(), c2.arrays()):
            b2.copy_(a)
        caches.append(c2)
    qp = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, hkv, n_keep), dtype=torch.int32, device="cuda")
    o_rot = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.dqk_decode_workspace_size(B, hq, hkv, mp, 0) // 4 + 4, dtype=torch.float32, device="cuda")
    calls = [[pa.prepared("dqk_select_channels_base", q, t_q, w_d, B, hq, hkv, n_keep, qp, sel, stream),
              pa.prepared("dqk_decode_attn", c, qp, sel, n_keep, B, hq, pt, mp, lens, float(prob.sm_scale), 0, ws,
                          ws.numel() * 4, o_rot, None, stream),
              pa.prepared("dqk_value_unrotate", o_rot, rinv_d, B, hq, hkv, out, stream)] for c in caches]
    one = [pa.prepared("dqk_select_decode_attn_vrot", c, q, t_q, w_d, rinv_d, n_keep, B, hq, pt, mp, lens,
                       float(prob.sm_scale), 0, ws, ws.numel() * 4, out, None, qp, sel, stream) for c in caches]
    nc = len(caches)

    def wall(fn_of_step, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fn_of_step(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    def three(i):
        for f in calls[i % nc]:
            f()

    def single(i):
        one[i % nc]()

    for i in range(100):
        single(i)
        three(i)
    t_one = wall(single, steps)
    t_step = wall(three, steps)
    ne = min(steps, 30)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(ne)]
    for i in range(ne):
        evs[i][0].record(stream)
        for j, f in enumerate(calls[i % nc]):
            f()
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    us = [float(np.mean([e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs])) for j in range(3)]
    e1 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ne)]
    for i in range(ne):
        e1[i][0].record(stream)
        single(i)
        e1[i][1].record(stream)
    torch.cuda.synchronize()
    one_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in e1]))
    sel_h = sel.cpu().numpy()
    cache_bytes = traffic.decode_cache_bytes(prob.seq_lens, sel_h)
    fixed = traffic.decode_fixed_bytes(B, hq, hkv, n_keep, mp)
    unrot_bytes = 2 * B * hq * 128 * 4 + hkv * 128 * 128 * 4
    step_bytes = cache_bytes + fixed["decode"] + fixed["select"] + hkv * 128 * 4 + unrot_bytes
    app = append_roofline(app_s, tokens, prob.num_pages, hkv)
    app_flops = 4.0 * tokens * hkv * 128 * 128  # k T_K and v R_V
    app["mfma_tflops"] = round(app_flops / app_s / 1e12, 2)
    app["mfma_frac"] = round(app["mfma_tflops"] / 2500.0, 4)
    app["workload"] = f"rotated-value prefill of {shape.seq_lens[0]} tokens x {hkv} KV heads per call, {B} calls"
    return {"workload": shape.name + "-vrot", "clip": clip,
            "entry": "dqk_select_decode_attn_vrot (base selection in the decode launch, merge with the inverse "
                     "rotation)",
            "t_step_us": round(t_one * 1e6, 2), "tokens_per_s": round(B / t_one, 1), "call_us": round(one_us, 2),
            "algorithmic_bytes_per_step": int(step_bytes),
            "frac_step": round(step_bytes / t_one / 1e9 / PEAK_HBM_GBS, 4), "cache_copies": nc,
            "three_calls": {"entries": "dqk_select_channels_base + dqk_decode_attn + dqk_value_unrotate",
                            "t_step_us": round(t_step * 1e6, 2), "select_us": round(us[0], 2),
                            "decode_call_us": round(us[1], 2), "unrotate_us": round(us[2], 2)},
            "append": app}


def tokgrid_record(shape, seed, pa, torch, steps):
    """The headline workload with one key grid per token (the paper's key
    format): the cache is built sequence by sequence with
    dqk_quantize_append_tokgrid (HIP events), then a step is one
    dqk_select_decode_attn_tokgrid call over cache copies rotated as in the
    headline; the same step as two calls (dqk_select_channels +
    dqk_decode_attn_tokgrid) is reported beside it."""
    from page_set_amd import traffic
    prob = synth.make_problem(shape, seed, materialize_kv=False)
    B, hq, hkv, n_keep = shape.batch, shape.hq, shape.hkv, shape.n_keep
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    q, t_q, t_k = dev(prob.q.view(np.int16)), dev(prob.t_q), dev(prob.t_k.view(np.int16))
    pt, lens = dev(prob.page_table), dev(prob.seq_lens)
    mp = int(prob.page_table.shape[1])
    stream = torch.cuda.current_stream()
    cache = pa.Cache(prob.num_pages, hkv)
    app_s, tokens = 0.0, 0
    for b in range(B):
        kb, vb = synth.make_kv_seq(shape, seed, b, prob.outliers)
        L = kb.shape[0]
        k_d, v_d = dev(kb.view(np.int16)), dev(vb.view(np.int16))
        cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        ptb = pt[b:b + 1].clone()
        if b == 0:  # untimed first call
            pa.dqk_quantize_append_tokgrid(cache, k_d, v_d, t_k, cu, ptb, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pa.dqk_quantize_append_tokgrid(cache, k_d, v_d, t_k, cu, ptb, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        app_s += e0.elapsed_time(e1) * 1e-3
        tokens += L
        del k_d, v_d
    caches = [cache]
    for _ in range(_copies_for(cache.nbytes()) - 1):
        c2 = pa.Cache(cache.num_pages, hkv)
        for a, b2 in zip(cache.arrays(), c2.arrays()):
            b2.copy_(a)
        caches.append(c2)
    qp = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, hkv, n_keep), dtype=torch.int32, device="cuda")
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.dqk_decode_workspace_size(B, hq, hkv, mp, 0) // 4 + 4, dtype=torch.float32, device="cuda")
    sel_call = pa.prepared("dqk_select_channels", q, t_q, B, hq, hkv, n_keep, qp, sel, stream)
    dec = [pa.prepared("dqk_decode_attn_tokgrid", c, qp, sel, n_keep, B, hq, pt, mp, lens, float(prob.sm_scale), 0,
                       ws, ws.numel() * 4, out, None, stream) for c in caches]
    one = [pa.prepared("dqk_select_decode_attn_tokgrid", c, q, t_q, n_keep, B, hq, pt, mp, lens,
                       float(prob.sm_scale), 0, ws, ws.numel() * 4, out, None, qp, sel, stream) for c in caches]
    nc = len(caches)
    for i in range(100):
        one[i % nc]()
        sel_call()
        dec[i % nc]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one[i % nc]()
    torch.cuda.synchronize()
    t_one = (time.perf_counter() - t0) / steps
    t0 = time.perf_counter()
    for i in range(steps):
        sel_call()
        dec[i % nc]()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / steps
    ne = min(steps, 30)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ne)]
    for i in range(ne):
        sel_call()
        evs[i][0].record(stream)
        dec[i % nc]()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    dec_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evs]))
    sel_h = sel.cpu().numpy()
    cache_bytes = traffic.decode_cache_bytes_tokgrid(prob.seq_lens, sel_h)
    fixed = traffic.decode_fixed_bytes(B, hq, hkv, n_keep, mp)
    step_bytes = cache_bytes + fixed["decode"] + fixed["select"]
    app = append_roofline(app_s, tokens, prob.num_pages, hkv)
    app["workload"] = f"per-token key grid prefill of {shape.seq_lens[0]} tokens x {hkv} KV heads per call, {B} calls"
    return {"workload": shape.name + "-tokgrid",
            "entry": "dqk_select_decode_attn_tokgrid (the selection in the decode launch, then merge)",
            "t_step_us": round(t_one * 1e6, 2), "tokens_per_s": round(B / t_one, 1),
            "two_calls": {"entries": "dqk_select_channels + dqk_decode_attn_tokgrid",
                          "t_step_us": round(t_step * 1e6, 2), "decode_call_us": round(dec_us, 2)},
            "algorithmic_bytes_per_step": int(step_bytes),
            "bytes_per_token_head": round(cache_bytes / (hkv * float(np.sum(prob.seq_lens))), 3),
            "frac_step": round(step_bytes / t_one / 1e9 / PEAK_HBM_GBS, 4),
            "frac_call": round((cache_bytes + fixed["decode"]) / (dec_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "cache_copies": nc, "append": app}


def rope_record(shape, seed, pa, torch, steps):
    """The headline workload with bucket-relative RoPE (2048-token buckets,
    64 at 128K): the cache is built sequence by sequence with
    dqk_quantize_append_rope (HIP events), then a step is one
    dqk_select_decode_attn_rope call (per-bucket turned queries and masks,
    bucket merge) over cache copies rotated as in the headline; the same step
    as two calls (dqk_select_channels_rope + dqk_decode_attn_rope) is
    reported beside it."""
    from page_set_amd import traffic
    prob = synth.make_problem(shape, seed, materialize_kv=False)
    B, hq, hkv, n_keep = shape.batch, shape.hq, shape.hkv, shape.n_keep
    nb = synth.rope_buckets(max(shape.seq_lens))
    cs_h, sn_h = synth.make_rope_tables(nb)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    q, t_q, t_k = dev(prob.q.view(np.int16)), dev(prob.t_q), dev(prob.t_k.view(np.int16))
    cs, sn = dev(cs_h), dev(sn_h)
    pt, lens = dev(prob.page_table), dev(prob.seq_lens)
    mp = int(prob.page_table.shape[1])
    stream = torch.cuda.current_stream()
    cache = pa.Cache(prob.num_pages, hkv)
    app_s, tokens = 0.0, 0
    for b in range(B):
        kb, vb = synth.make_kv_seq(shape, seed, b, prob.outliers)
        L = kb.shape[0]
        k_d, v_d = dev(kb.view(np.int16)), dev(vb.view(np.int16))
        cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        ptb = pt[b:b + 1].clone()
        if b == 0:  # untimed first call
            pa.dqk_quantize_append_rope(cache, k_d, v_d, t_k, cs, sn, cu, ptb, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pa.dqk_quantize_append_rope(cache, k_d, v_d, t_k, cs, sn, cu, ptb, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        app_s += e0.elapsed_time(e1) * 1e-3
        tokens += L
        del k_d, v_d
    caches = [cache]
    for _ in range(_copies_for(cache.nbytes()) - 1):
        c2 = pa.Cache(cache.num_pages, hkv)
        for a, b2 in zip(cache.arrays(), c2.arrays()):
            b2.copy_(a)
        caches.append(c2)
    qp = torch.empty((B, nb, hq, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, nb, hkv, n_keep), dtype=torch.int32, device="cuda")
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.dqk_decode_rope_workspace_size(B, hq, hkv, nb, 0) // 4 + 4, dtype=torch.float32,
                     device="cuda")
    sel_call = pa.prepared("dqk_select_channels_rope", q, t_q, cs, sn, nb, B, hq, hkv, n_keep, qp, sel, stream)
    dec = [pa.prepared("dqk_decode_attn_rope", c, qp, sel, n_keep, nb, B, hq, pt, mp, lens, float(prob.sm_scale), 0,
                       ws, ws.numel() * 4, out, None, stream) for c in caches]
    one = [pa.prepared("dqk_select_decode_attn_rope", c, q, t_q, cs, sn, n_keep, nb, B, hq, pt, mp, lens,
                       float(prob.sm_scale), 0, ws, ws.numel() * 4, out, None, qp, sel, stream) for c in caches]
    nc = len(caches)
    for i in range(100):
        one[i % nc]()
        sel_call()
        dec[i % nc]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one[i % nc]()
    torch.cuda.synchronize()
    t_one = (time.perf_counter() - t0) / steps
    t0 = time.perf_counter()
    for i in range(steps):
        sel_call()
        dec[i % nc]()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / steps
    ne = min(steps, 30)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ne)]
    sevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ne)]
    for i in range(ne):
        sevs[i][0].record(stream)
        sel_call()
        sevs[i][1].record(stream)
        evs[i][0].record(stream)
        dec[i % nc]()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    dec_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evs]))
    sel_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in sevs]))
    sel_h = sel.cpu().numpy()
    cache_bytes = traffic.decode_rope_bytes(prob.seq_lens, sel_h)
    fixed = traffic.decode_fixed_bytes(B * nb, hq, hkv, n_keep, 16)
    step_bytes = cache_bytes + fixed["decode"] + fixed["select"] + 2 * nb * 64 * 4
    app = append_roofline(app_s, tokens, prob.num_pages, hkv)
    app["workload"] = f"bucket-frame prefill of {shape.seq_lens[0]} tokens x {hkv} KV heads per call, {B} calls"
    return {"workload": shape.name + "-rope", "n_buckets": nb,
            "entry": "dqk_select_decode_attn_rope (per-bucket selection, decode switching buckets per split, merge)",
            "t_step_us": round(t_one * 1e6, 2), "tokens_per_s": round(B / t_one, 1),
            "two_calls": {"entries": "dqk_select_channels_rope + dqk_decode_attn_rope",
                          "t_step_us": round(t_step * 1e6, 2), "select_call_us": round(sel_us, 2),
                          "decode_call_us": round(dec_us, 2)},
            "algorithmic_bytes_per_step": int(step_bytes),
            "bytes_per_token_head": round(cache_bytes / (hkv * float(np.sum(prob.seq_lens))), 3),
            "frac_step": round(step_bytes / t_one / 1e9 / PEAK_HBM_GBS, 4),
            "frac_call": round((cache_bytes + fixed["decode"]) / (dec_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "cache_copies": nc, "append": app}


def _summary(name, w, r, n_keep):
    B = w.shape.batch
    rec = {"workload": name, "batch": B, "context": (max(w.shape.seq_lens) if len(set(w.shape.seq_lens)) == 1
                                                     else "ragged"),
           "n_keep": n_keep, "t_step_us": round(r["t_step_us"], 2), "tokens_per_s": round(B / (r["t_step_us"] * 1e-6), 1),
           "entry": "dqk_select_decode_attn", "call_us": round(r["decode_us"], 2),
           "algorithmic_bytes_per_step": int(r["step_bytes"]),
           "bytes_per_token_head": round(r["bytes_per_token_head"], 3),
           "achieved_step_gbs": round(r["step_bytes"] / (r["t_step_us"] * 1e-6) / 1e9, 1),
           "frac_step": round(r["step_bytes"] / (r["t_step_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
           "achieved_call_gbs": round(r["step_bytes"] / (r["decode_us"] * 1e-6) / 1e9, 1),
           "frac_call": round(r["step_bytes"] / (r["decode_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
           "cache_copies": len(w.caches)}
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--sparsity", type=float, default=0.4)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--sub-steps", type=int, default=20, help="timed steps of each secondary workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="headline workload only (no per-config records)")
    ap.add_argument("--calib-copy", action="store_true", help="also run a plain 1 GiB copy kernel (PMC calibration)")
    ap.add_argument("--write-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                    help="turn two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) of a --calib-copy run "
                         "into the per-launch HBM traffic record and exit")
    ap.add_argument("--only", choices=["tiered", "vrot", "tokgrid", "rope"],
                    help="run only this variant of the config's workload (protected BF16 tiers, rotated values "
                         "with base selection, per-token key grids, or bucket-relative RoPE) and print its record "
                         "(for profiling)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import page_set_amd as pa

    shape = synth.config_shape(args.config, args.seed, args.sparsity)
    n_keep = shape.n_keep
    if args.only:
        fn = {"tiered": tiered_record, "vrot": vrot_record, "tokgrid": tokgrid_record,
              "rope": rope_record}[args.only]
        print(json.dumps(fn(shape, args.seed, pa, torch, args.steps)), flush=True)
        return
    log(f"[bench] workload {shape.name}: B={shape.batch} Hq/Hkv={shape.hq}/{shape.hkv} ctx={max(shape.seq_lens)} "
        f"n_keep={n_keep}")
    t0 = time.time()
    w = Int2Workload(shape, args.seed, pa, torch)
    log(f"[bench] cache built on GPU in {time.time() - t0:.1f}s ({w.caches[0].nbytes() / 1e6:.1f} MB, "
        f"{len(w.caches)} copies)")
    # the step: dqk_select_decode_attn, one call (the selection in the decode
    # kernel's prologue, split decode, merge)
    r = w.time_steps(n_keep, args.steps, args.warmup, args.num_splits, fused=True)
    # for context: the same step as two calls, dqk_select_channels then dqk_decode_attn
    r2 = w.time_steps(n_keep, max(10, args.steps // 2), args.warmup, args.num_splits, fused=False)
    B = shape.batch
    ms_per_step = r["t_step_us"] * 1e-3
    log(f"[bench] {r['t_step_us']:.1f} us/step (one call, {r['decode_us']:.1f} us on the stream, p10 "
        f"{r['decode_p10_us']:.1f}, p90 {r['decode_p90_us']:.1f}); as two calls: {r2['t_step_us']:.1f} us/step "
        f"(select {r2['select_us']:.1f} us, decode call {r2['decode_us']:.1f} us)")

    achieved = r["step_bytes"] / (r["decode_us"] * 1e-6) / 1e9
    achieved_step = r["step_bytes"] / (r["t_step_us"] * 1e-6) / 1e9
    khash = source_hash()
    tr = committed_traffic(khash)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": (tr["hbm_bytes_per_launch"] if tr else None),
            "kernel": "dqk_select_decode_attn (decode kernel with the selection in its prologue, then merge), "
                      "HIP events on its stream",
            "algorithmic_bytes_per_launch": int(r["step_bytes"]),
            "bytes_per_token_head": round(r["bytes_per_token_head"], 3),
            "avg_launch_us": round(r["decode_us"], 2),
            "step_definition": "dqk_select_decode_attn (selection + split decode + merge), wall clock per step",
            "algorithmic_bytes_per_step": int(r["step_bytes"]),
            "achieved_step": round(achieved_step, 1), "frac_step": round(achieved_step / PEAK_HBM_GBS, 4),
            "two_call_step": {"entries": "dqk_select_channels + dqk_decode_attn",
                              "t_step_us": round(r2["t_step_us"], 2), "select_us": round(r2["select_us"], 2),
                              "decode_call_us": round(r2["decode_us"], 2),
                              "frac_step": round(r2["step_bytes"] / (r2["t_step_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                                 4)},
            "kernel_source_hash": khash}
    roof["stream_read_gbs"] = round(stream_read_gbs(torch, pa, int(r["decode_bytes"])), 1)
    roof["frac_of_stream_read"] = round(achieved / roof["stream_read_gbs"], 4)
    app = append_roofline(w.append_s, w.append_tokens, w.prob.num_pages, shape.hkv)
    app["workload"] = f"prefill of {shape.seq_lens[0]} tokens x {shape.hkv} KV heads per call, {shape.batch} calls"

    if args.calib_copy:
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        del x, y

    rec = {"metric": METRIC, "value": round(B / (ms_per_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int2-kv/fp32-accumulate",
           "data": "synthetic (seeded Gaussian q/k/v, 4 outlier key channels x10, channel-0 offset +3)",
           "config": {"workload": shape.name, "batch": B, "q_heads": shape.hq, "kv_heads": shape.hkv,
                      "head_dim": 128, "context": max(shape.seq_lens), "n_keep": n_keep, "sparsity": args.sparsity,
                      "cache_copies": len(w.caches), "num_splits": args.num_splits or "auto"},
           "roofline": roof, "append_roofline": app}

    if not args.no_configs and args.config == 3:
        configs = {}
        sub = args.sub_steps
        sweep = {}
        for nk in (128, 103, 77, 52):
            rs = w.time_steps(nk, sub, 100, fused=True)
            sweep[str(nk)] = _summary(shape.name, w, rs, nk)
            log(f"[bench] sweep n_keep {nk}: {rs['t_step_us']:.1f} us/step")
        configs["3_sparsity_sweep"] = sweep
        del w
        torch.cuda.empty_cache()
        # group sizes other than 4 (config 0 is MHA): the same MFMA decode over sets of four query heads
        s0 = synth.config_shape(0, args.seed)
        w0 = Int2Workload(s0, args.seed, pa, torch)
        configs["0"] = _summary(s0.name, w0, w0.time_steps(s0.n_keep, sub, 100, fused=True), s0.n_keep)
        configs["0"]["kernel"] = ("decode_blk_kernel (one set of four query heads per KV head, three of them "
                                  "padding) + merge, after select_kernel_g<1>")
        log(f"[bench] config 0: {configs['0']['t_step_us']} us/step")
        del w0
        gen = {}
        for hq in (16, 64):
            sg = synth.Shape(4, hq, 8, [32768] * 4, 77, name=f"gqa{hq}x8-32k-b4")
            wg = Int2Workload(sg, args.seed, pa, torch)
            gen[f"g{hq // 8}"] = _summary(sg.name, wg, wg.time_steps(77, sub, 100, fused=True), 77)
            gen[f"g{hq // 8}"]["kernel"] = "decode_blk_kernel over sets of four query heads + merge, after select_kernel_g"
            log(f"[bench] group {hq // 8}: {gen[f'g{hq // 8}']['t_step_us']} us/step")
            del wg
        configs["other_groups"] = gen
        torch.cuda.empty_cache()
        s1 = synth.config_shape(1, args.seed)
        w1 = Int2Workload(s1, args.seed, pa, torch)
        configs["1"] = _summary(s1.name, w1, w1.time_steps(s1.n_keep, sub, 100, fused=True), s1.n_keep)
        log(f"[bench] config 1: {configs['1']['t_step_us']} us/step")
        del w1
        s2 = synth.config_shape(2, args.seed)
        w2 = Int2Workload(s2, args.seed, pa, torch)
        c2 = {"int2_40": _summary(s2.name, w2, w2.time_steps(77, sub, 100, fused=True), 77),
              "int2_0": _summary(s2.name, w2, w2.time_steps(128, sub, 100, fused=True), 128)}
        prob2 = w2.prob
        del w2
        torch.cuda.empty_cache()
        kp, vp = build_bf16_pages(prob2, s2, torch)
        qd = torch.from_numpy(prob2.q.view(np.int16)).to("cuda")
        ptd = torch.from_numpy(prob2.page_table).to("cuda")
        sld = torch.from_numpy(prob2.seq_lens).to("cuda")
        out = torch.empty((s2.batch, s2.hq, 128), dtype=torch.float32, device="cuda")
        ws = torch.empty(pa.dqk_decode_workspace_size(s2.batch, s2.hq, s2.hkv, ptd.shape[1], 0) // 4 + 4,
                         dtype=torch.float32, device="cuda")
        for _ in range(3):
            pa.dqk_decode_attn_bf16(kp, vp, qd, ptd, sld, prob2.sm_scale, workspace=ws, out=out, want_lse=False)
        torch.cuda.synchronize()
        tb = time.perf_counter()
        for _ in range(sub):
            pa.dqk_decode_attn_bf16(kp, vp, qd, ptd, sld, prob2.sm_scale, workspace=ws, out=out, want_lse=False)
        torch.cuda.synchronize()
        t_bf = (time.perf_counter() - tb) / sub
        from page_set_amd import traffic
        bf_bytes = traffic.bf16_cache_bytes(prob2.seq_lens, s2.hkv)
        c2["bf16_dense"] = {"workload": s2.name, "t_step_us": round(t_bf * 1e6, 2),
                            "tokens_per_s": round(s2.batch / t_bf, 1), "algorithmic_bytes_per_step": int(bf_bytes),
                            "achieved_step_gbs": round(bf_bytes / t_bf / 1e9, 1),
                            "frac_step": round(bf_bytes / t_bf / 1e9 / PEAK_HBM_GBS, 4),
                            "kernel": "dqk_decode_attn_bf16 (unpruned BF16, split decode + merge)"}
        c2["int2_40_vs_bf16_speedup"] = round(t_bf * 1e6 / c2["int2_40"]["t_step_us"], 3)
        c2["int2_0_vs_bf16_speedup"] = round(t_bf * 1e6 / c2["int2_0"]["t_step_us"], 3)
        c2["bf16_vs_int2_40_read_ratio"] = round(bf_bytes / c2["int2_40"]["algorithmic_bytes_per_step"], 3)
        configs["2"] = c2
        log(f"[bench] config 2: INT2 40% {c2['int2_40']['t_step_us']} us, BF16 {c2['bf16_dense']['t_step_us']} us")
        del kp, vp
        torch.cuda.empty_cache()
        s4 = synth.config_shape(4, args.seed)
        w4 = Int2Workload(s4, args.seed, pa, torch, one_call=True)
        c4 = _summary(s4.name, w4, w4.time_steps(s4.n_keep, sub, 100, fused=True), s4.n_keep)
        c4["total_tokens"] = int(np.sum(s4.seq_lens))
        c4["append"] = append_roofline(w4.append_s, w4.append_tokens, w4.prob.num_pages, s4.hkv)
        c4["append"]["workload"] = f"one call over the ragged batch ({c4['total_tokens']} tokens, shuffled pages)"
        configs["4"] = c4
        log(f"[bench] config 4: {c4['t_step_us']} us/step")
        del w4
        torch.cuda.empty_cache()
        configs["3_tiered"] = tiered_record(shape, args.seed, pa, torch, sub)
        log(f"[bench] config 3 tiered: {configs['3_tiered']['t_step_us']} us/step, append token "
            f"{configs['3_tiered']['append_token_us']} us")
        torch.cuda.empty_cache()
        configs["3_tokgrid"] = tokgrid_record(shape, args.seed, pa, torch, sub)
        log(f"[bench] config 3 per-token key grids: {configs['3_tokgrid']['t_step_us']} us/step, append "
            f"{configs['3_tokgrid']['append']['seconds'] * 1e6:.0f} us")
        torch.cuda.empty_cache()
        configs["3_vrot"] = vrot_record(shape, args.seed, pa, torch, sub)
        log(f"[bench] config 3 rotated values: {configs['3_vrot']['t_step_us']} us/step one call, "
            f"{configs['3_vrot']['three_calls']['t_step_us']} us as three calls, append "
            f"{configs['3_vrot']['append']['seconds'] * 1e6:.0f} us")
        torch.cuda.empty_cache()
        configs["3_rope"] = rope_record(shape, args.seed, pa, torch, sub)
        log(f"[bench] config 3 bucket-relative RoPE: {configs['3_rope']['t_step_us']} us/step one call, "
            f"{configs['3_rope']['two_calls']['t_step_us']} us as two calls, append "
            f"{configs['3_rope']['append']['seconds'] * 1e6:.0f} us")
        rec["configs"] = configs

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline(shape, args.seed, n_keep)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
