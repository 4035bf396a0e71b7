#!/usr/bin/env python3
"""Benchmark of the exact-attention library on one MI355X.

One step = one forward call (fa_fwd) over B1 H32 N8192 d128 bf16 causal
inputs already resident in HBM (the Llama-7B attention shape at 8K).  The
timed region is K such calls bracketed by torch.cuda.synchronize(); each call
is also bracketed by HIP events on the launch stream (torch's current
stream, which the binding passes to the library), which gives the average
duration of the one kernel a call launches.

FLOP convention: 4*B*H*N^2*d for the forward, halved for causal; 2.5x the
forward for the backward; window/varlen workloads count 4*d*H*(visible
query-key pairs).  Peaks: dense bf16 MFMA 2516.6 TFLOP/s (256 CUs x 2.4 GHz x
4096 FLOP/clk/CU), dense fp8 5033.2 TFLOP/s, HBM 8 TB/s.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 5033.2
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_flops(b, h, n, d, causal):
    f = 4.0 * b * h * n * n * d
    return f / 2 if causal else f


def visible_pairs_varlen(lengths, causal, window):
    tot = 0
    for L in lengths:
        for_rows = 0
        if causal and window > 0:
            # row i sees min(i + 1, window) keys
            w = min(window, L)
            for_rows = w * (w + 1) // 2 + (L - w) * w
        elif causal:
            for_rows = L * (L + 1) // 2
        else:
            for_rows = L * L
        tot += for_rows
    return tot


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_attention_24_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def time_calls(fn, warmup, steps, torch):
    """Run fn warmup times, then steps times; return (wall_ms_total, per-call ms list)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return wall, [e0.elapsed_time(e1) for e0, e1 in evs]


def traffic_from_profile(kernel_sha):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "fwd_bf16_llama_n8192_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha") != kernel_sha:
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_info():
    """The host the oracle runs on: CPU model, CPUs in this process's
    affinity mask, and the BLAS thread count (the threads its matmuls use)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)), "blas_threads": blas}


def cpu_baseline(budget_s=15.0):
    """The fp64 oracle on a bounded sample of the same workload: whole heads of
    the causal N=8192 d=128 forward, one after another, until budget_s."""
    import numpy as np  # noqa: F401
    import oracle
    from exact_attention_24_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS["llama_n8192"]
    t = workload_inputs("llama_n8192")
    q, k, v = (t[x].to(dtype=__import__("torch").float64).numpy() for x in ("q", "k", "v"))
    heads, t0 = 0, time.perf_counter()
    while heads < w.heads and time.perf_counter() - t0 < budget_s:
        oracle.attention_fwd(q[0, :, heads], k[0, :, heads], v[0, :, heads], w.scale, True, 0)
        heads += 1
    el = time.perf_counter() - t0
    info = cpu_info()
    flops = fwd_flops(1, heads, w.seqlen, w.head_dim, True)
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": info["blas_threads"] or 1,
            "kind": "oracle",
            "sample": f"{heads} of 32 heads of the B1 H32 N8192 d128 causal forward, fp64 NumPy, {el:.1f} s",
            "seconds": round(el, 2), **info}


def counters_from_profile(name, sha):
    """MFMA-busy % per kernel from a committed SQ counter summary, if it was
    taken on the current kernel source (its sha line); else None."""
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            text = f.read()
    except OSError:
        return None
    if f"sha {sha}" not in text:
        return None
    out, kernel = {}, None
    for ln in text.splitlines():
        if ln.startswith("fa::"):
            kernel = ln.strip()
        m = re.search(r"MFMA_busy_pct=([0-9.]+)", ln)
        if m and kernel:
            out[kernel] = float(m.group(1))
    return out or None


def _errors(got, ref):
    import numpy as np
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(d.max()), float(d.mean())


def _oracle_timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0


def config_rows(torch, fa, steps, headline_cpu):
    """One record per configuration of the hot path, plus the extra rows:
    flops and compulsory HBM bytes per call, median and minimum call time
    (HIP events on the launch stream), TFLOP/s and % of peak, bytes / time,
    MFMA busy % from the committed counter summary of the same kernel source
    (null when there is none), max / mean abs error against the fp64 oracle
    on sampled rows, and the oracle timed on a bounded sample of the config."""
    import numpy as np
    import oracle
    from exact_attention_24_amd.inputs import WORKLOADS, workload_inputs

    rows = {}
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731

    def timed(fn):
        _, ms = time_calls(fn, 2, steps, torch)
        ms = sorted(ms)
        return ms[len(ms) // 2], ms[0]

    def mfma_row(name, fn, flops, nbytes, peak, err, oracle_s, oracle_flops, sample, counters=None, extra=None):
        med, mn = timed(fn)
        r = {"flops": flops, "bytes": nbytes, "median_us": round(med * 1e3, 1), "min_us": round(mn * 1e3, 1),
             "tflops": round(flops / med / 1e9, 1), "pct_peak": round(100 * flops / med / 1e9 / peak, 2),
             "gbs": round(nbytes / med / 1e6, 1), "mfma_busy_pct": counters,
             "err_max": None if err is None else float(f"{err[0]:.3e}"),
             "err_mean": None if err is None else float(f"{err[1]:.3e}"),
             "oracle": None if oracle_s is None else {"seconds": round(oracle_s, 3), "sample": sample,
                                                       "gflops": round(oracle_flops / oracle_s / 1e9, 3)}}
        if extra:
            r.update(extra)
        rows[name] = r
        log(f"[bench] {name}: {json.dumps(r)}")

    def hbm_row(name, fn, nbytes):
        med, mn = timed(fn)
        rows[name] = {"bytes": nbytes, "median_us": round(med * 1e3, 1), "min_us": round(mn * 1e3, 1),
                      "gbs": round(nbytes / med / 1e6, 1), "pct_hbm_peak": round(100 * nbytes / med / 1e6 / PEAK_HBM_GBS, 2)}
        log(f"[bench] {name}: {json.dumps(rows[name])}")

    fsha = src_hash("fa_fwd.hip", "fa_device.h", "fa_internal.h")
    bsha = src_hash("fa_bwd.hip", "fa_device.h", "fa_internal.h")
    psha = src_hash("fa_fp8.hip", "fa_device.h", "fa_internal.h")

    # configuration 1: B1 H1 N256 d64 fp32, non-causal (whole output checked)
    w = WORKLOADS["tiny_fp32"]
    t = workload_inputs("tiny_fp32")
    q, k, v = (t[x].cuda() for x in ("q", "k", "v"))
    o, lse1 = fa.fa_fwd(q, k, v, causal=False)
    (ro, _), secs = _oracle_timed(lambda: oracle.mha_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), w.scale, False, 0))
    F = fwd_flops(1, 1, 256, 64, False)
    o1 = torch.empty_like(o)  # outputs allocated once, as in the timed headline step
    mfma_row("cfg1_fwd_fp32_b1_h1_n256_d64", lambda: fa.fa_fwd(q, k, v, causal=False, out=o1, lse=lse1), F,
             4 * (4 * 256 * 64) + 4 * 256, 157.3, _errors(f64(o), ro), secs, F, "the whole config",
             extra={"note": "fp32 FMA kernel; peak is the fp32 vector rate 157.3 TFLOP/s; launch-bound"})

    # configuration 2: B2 H16 N1024 d64 bf16 causal (whole output checked)
    w = WORKLOADS["b2_h16_n1024"]
    t = workload_inputs("b2_h16_n1024")
    q, k, v = (t[x].cuda() for x in ("q", "k", "v"))
    o, lse2 = fa.fa_fwd(q, k, v, causal=True)
    (ro, _), secs = _oracle_timed(lambda: oracle.mha_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), w.scale, True, 0))
    F = fwd_flops(2, 16, 1024, 64, True)
    o2 = torch.empty_like(o)  # outputs allocated once, as in the timed headline step
    mfma_row("cfg2_fwd_bf16_b2_h16_n1024_d64_causal", lambda: fa.fa_fwd(q, k, v, causal=True, out=o2, lse=lse2), F,
             2 * (4 * 2 * 1024 * 16 * 64) + 4 * 2 * 16 * 1024, PEAK_BF16_TFLOPS, _errors(f64(o), ro), secs, F,
             "the whole config")

    # configuration 3: B1 H32 N8192 d128 bf16, causal (headline) and non-causal
    w = WORKLOADS["llama_n8192"]
    t = workload_inputs("llama_n8192")
    q, k, v = (t[x].cuda() for x in ("q", "k", "v"))
    qh, kh, vh = f64(t["q"]), f64(t["k"]), f64(t["v"])
    nbytes = 2 * (4 * 8192 * 32 * 128) + 4 * 32 * 8192
    srows = np.unique(np.concatenate([[0, 1, 63, 64, 255, 256, 8191], np.random.default_rng(3).choice(8192, 25, False)]))
    for causal in (True, False):
        o, _ = fa.fa_fwd(q, k, v, causal=causal)
        o64 = f64(o)
        errs = []
        for h in (0, 11, 22, 31):
            ro, _ = oracle.attention_fwd(qh[0, srows, h], kh[0, :, h], vh[0, :, h], w.scale, causal, 0, q_pos=srows,
                                         nq=8192)
            errs.append(_errors(o64[0, srows, h], ro))
        err = (max(e[0] for e in errs), float(np.mean([e[1] for e in errs])))
        F = fwd_flops(1, 32, 8192, 128, causal)
        if causal and headline_cpu:
            secs, nh = headline_cpu["seconds"], int(headline_cpu["sample"].split()[0])
        else:
            _, secs = _oracle_timed(lambda: oracle.attention_fwd(qh[0, :, 0], kh[0, :, 0], vh[0, :, 0], w.scale, causal,
                                                                 0))
            nh = 1
        name = "cfg3_fwd_bf16_b1_h32_n8192_d128_" + ("causal" if causal else "noncausal")
        prof = "fwd_bf16_n8192_d128_causal.sq_counters.txt" if causal else "fwd_bf16_n8192_d128_noncausal.sq_counters.txt"
        mfma_row(name, lambda c=causal: fa.fa_fwd(q, k, v, causal=c), F, nbytes, PEAK_BF16_TFLOPS, err, secs,
                 fwd_flops(1, nh, 8192, 128, causal), f"{nh} of 32 heads, fp64", counters_from_profile(prof, fsha))
    # the same causal call with the inputs evicted from the 256 MB last-level
    # cache (MALL) before every call: two input sets (402 MB) in turn
    t2 = workload_inputs("llama_n8192_noncausal")
    q2, k2, v2 = (x.cuda() * 1 for x in (t2["q"], t2["k"], t2["v"]))
    sets = [(q, k, v), (q2, k2, v2)]
    state = {"i": 0}

    def alternate():
        qq, kk, vv = sets[state["i"] & 1]
        state["i"] += 1
        fa.fa_fwd(qq, kk, vv, causal=True)

    med, mn = timed(alternate)
    F = fwd_flops(1, 32, 8192, 128, True)
    rows["cfg3_fwd_causal_two_input_sets"] = {
        "median_us": round(med * 1e3, 1), "min_us": round(mn * 1e3, 1), "tflops": round(F / med / 1e9, 1),
        "note": "Q/K/V of one call are 201 MB and stay resident in the 256 MB MALL between repeated calls; "
                "alternating two input sets (402 MB) makes every call read them from HBM"}
    log(f"[bench] cfg3_fwd_causal_two_input_sets: {json.dumps(rows['cfg3_fwd_causal_two_input_sets'])}")
    del q2, k2, v2, sets

    # configuration 5 (fp8): the same shape in e4m3 with per-tensor scales, causal
    t8 = workload_inputs("fp8_n8192")
    q8, k8, v8 = (t8[x].cuda() for x in ("q8", "k8", "v8"))
    ds = (t8["q_scale"], t8["k_scale"], t8["v_scale"])
    o, _ = fa.fa_fwd(q8, k8, v8, causal=True, descale=ds)
    o64 = f64(o)
    deq = [oracle.fp8_dequant(t8[x].view(torch.uint8).numpy(), sc) for x, sc in zip(("q8", "k8", "v8"), ds)]
    errs = []
    for h in (0, 11, 22, 31):
        ro, _ = oracle.attention_fwd(deq[0][0, srows, h], deq[1][0, :, h], deq[2][0, :, h], w.scale, True, 0,
                                     q_pos=srows, nq=8192)
        errs.append(_errors(o64[0, srows, h], ro))
    err = (max(e[0] for e in errs), float(np.mean([e[1] for e in errs])))
    _, secs = _oracle_timed(lambda: oracle.attention_fwd(deq[0][0, :, 0], deq[1][0, :, 0], deq[2][0, :, 0], w.scale,
                                                         True, 0))
    F = fwd_flops(1, 32, 8192, 128, True)
    mfma_row("cfg5_fwd_fp8_b1_h32_n8192_d128_causal", lambda: fa.fa_fwd(q8, k8, v8, causal=True, descale=ds), F,
             3 * 8192 * 32 * 128 + 2 * 8192 * 32 * 128 + 4 * 32 * 8192, PEAK_FP8_TFLOPS, err, secs,
             fwd_flops(1, 1, 8192, 128, True), "1 of 32 heads, fp64 on the dequantised inputs",
             counters_from_profile("fwd_fp8_n8192_d128_causal.sq_counters.txt", psha))
    del q8, k8, v8, deq

    # configuration 5 (backward): B1 H32 N8192 d128 bf16 causal, fp32 gradients
    w = WORKLOADS["bwd_n8192"]
    t = workload_inputs("bwd_n8192")
    qb, kb, vb, dob = (t[x].cuda() for x in ("q", "k", "v", "dout"))
    o, lse = fa.fa_fwd(qb, kb, vb, causal=True)
    dq, dk, dv = (torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in (qb, kb, vb))
    bwd = lambda: fa.fa_bwd(dob, qb, kb, vb, o, lse, causal=True, dq=dq, dk=dk, dv=dv)  # noqa: E731
    bwd()
    g64 = [f64(x)[0, :, 0] for x in (dq, dk, dv)]
    ref, secs = _oracle_timed(lambda: oracle.attention_bwd(*(f64(t[x])[0, :, 0] for x in ("q", "k", "v", "dout")),
                                                           w.scale, True, 0))
    errs = [_errors(g, r) for g, r in zip(g64, ref)]
    err = (max(e[0] for e in errs), float(np.mean([e[1] for e in errs])))
    F = 2.5 * fwd_flops(1, 32, 8192, 128, True)
    mfma_row("cfg5_bwd_bf16_b1_h32_n8192_d128_causal", bwd, F,
             5 * 2 * 8192 * 32 * 128 + 4 * 32 * 8192 + 3 * 4 * 8192 * 32 * 128, PEAK_BF16_TFLOPS, err, secs,
             2.5 * fwd_flops(1, 1, 8192, 128, True), "head 0 of 32 (all its dQ, dK, dV), fp64",
             counters_from_profile("bwd_bf16_n8192_d128_causal.sq_counters.txt", bsha))
    # dropout (p = 0.1) forward and backward at the same shape
    kw = dict(causal=True, dropout_p=0.1, seed=1234, offset=0)
    od, lsed = fa.fa_fwd(qb, kb, vb, **kw)
    F = fwd_flops(1, 32, 8192, 128, True)
    mfma_row("fwd_bf16_n8192_causal_dropout0.1", lambda: fa.fa_fwd(qb, kb, vb, **kw), F,
             2 * (4 * 8192 * 32 * 128) + 4 * 32 * 8192, PEAK_BF16_TFLOPS, None, None, 0, None)
    mfma_row("bwd_bf16_n8192_causal_dropout0.1",
             lambda: fa.fa_bwd(dob, qb, kb, vb, od, lsed, dq=dq, dk=dk, dv=dv, **kw), 2.5 * F,
             5 * 2 * 8192 * 32 * 128 + 4 * 32 * 8192 + 3 * 4 * 8192 * 32 * 128, PEAK_BF16_TFLOPS, None, None, 0,
             None)
    del qb, kb, vb, dob, o, lse, od, lsed, dq, dk, dv

    # configuration 4: packed varlen, 32768 tokens, H28 d128, causal + window 4096; and its backward
    w = WORKLOADS["varlen_32k"]
    t = workload_inputs("varlen_bwd_32k")
    q, k, v, do, cu = (t[x].cuda() for x in ("q", "k", "v", "dout", "cu_seqlens"))
    mx = max(t["lengths"])
    o, lse = fa.fa_varlen_fwd(q, k, v, cu, mx, causal=True, window=w.window)
    o64 = f64(o)
    cuh = t["cu_seqlens"].numpy()
    qh, kh, vh = f64(t["q"]), f64(t["k"]), f64(t["v"])
    errs, osecs = [], 0.0
    for s_ in range(len(t["lengths"])):
        a_, b_ = int(cuh[s_]), int(cuh[s_ + 1])
        rr = np.unique(np.concatenate([[0, b_ - a_ - 1], np.random.default_rng(s_).choice(b_ - a_, 6, False)]))
        for h in (0, 27):
            ro, _ = oracle.attention_fwd(qh[a_ + rr, h], kh[a_:b_, h], vh[a_:b_, h], w.scale, True, w.window,
                                         q_pos=rr, nq=b_ - a_)
            errs.append(_errors(o64[a_ + rr, h], ro))
        _, sec = _oracle_timed(lambda: oracle.attention_fwd(qh[a_:b_, 0], kh[a_:b_, 0], vh[a_:b_, 0], w.scale, True,
                                                            w.window))
        osecs += sec
    err = (max(e[0] for e in errs), float(np.mean([e[1] for e in errs])))
    pairs = visible_pairs_varlen(t["lengths"], True, w.window)
    F = 4.0 * w.head_dim * w.heads * pairs
    mfma_row("cfg4_varlen_fwd_bf16_32k_h28_d128_causal_w4096",
             lambda: fa.fa_varlen_fwd(q, k, v, cu, mx, causal=True, window=w.window), F,
             2 * (4 * 32768 * 28 * 128) + 4 * 28 * 32768, PEAK_BF16_TFLOPS, err, osecs, 4.0 * 128 * pairs,
             "head 0 of 28, all sequences, fp64", counters_from_profile("varlen_fwd_bf16_32k_h28_w4096.sq_counters.txt", fsha),
             extra={"lengths": t["lengths"]})
    dq, dk, dv = (torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in (q, k, v))
    mfma_row("varlen_bwd_bf16_32k_h28_d128_causal_w4096",
             lambda: fa.fa_varlen_bwd(do, q, k, v, o, lse, cu, mx, causal=True, window=w.window, dq=dq, dk=dk, dv=dv),
             2.5 * F, 5 * 2 * 32768 * 28 * 128 + 4 * 28 * 32768 + 3 * 4 * 32768 * 28 * 128, PEAK_BF16_TFLOPS, None,
             None, 0, None, counters_from_profile("varlen_bwd_bf16_32k_h28_w4096.sq_counters.txt", bsha))
    del q, k, v, do, o, lse, dq, dk, dv

    # HBM-bound rows: partial-result merge, KV-cache decode steps
    o_p, lse_p, out, lse, nbytes = merge_inputs(torch)
    hbm_row("merge_8parts_f32_b1_n8192_h32_d128", lambda: fa.fa_merge(o_p, lse_p, out=out, lse=lse), nbytes)
    del o_p, lse_p, out, lse
    fn, nbytes = kvcache_step(torch, fa)
    hbm_row("kvcache_decode_b8_h32_d128_8k", fn, nbytes)
    fn, nbytes = kvcache_step(torch, fa, page=256)
    hbm_row("kvcache_paged256_decode_b8_h32_d128_8k", fn, nbytes)
    return rows


MERGE_PARTS = 8


def merge_inputs(torch):
    """8 fp32 partial results of the B1 N8192 H32 d128 forward (ring-attention
    shape: one per key segment), seeded, resident in HBM."""
    g = torch.Generator(device="cuda").manual_seed(1006)
    o_p = torch.randn(MERGE_PARTS, 1, 8192, 32, 128, generator=g, device="cuda")
    lse_p = 4.0 * torch.randn(MERGE_PARTS, 1, 32, 8192, generator=g, device="cuda")
    out = torch.empty(1, 8192, 32, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, 32, 8192, dtype=torch.float32, device="cuda")
    nbytes = o_p.numel() * 4 + lse_p.numel() * 4 + out.numel() * 2 + lse.numel() * 4
    return o_p, lse_p, out, lse, nbytes


def kvcache_step(torch, fa, page=0):
    """One decode step at B8 H32 d128 with 8191 cached tokens + 1 new: the
    step function (idempotent: it appends at the same row each time) and the
    bytes it must move (every cached K/V row once, plus q, the new rows and O).
    page > 0: the caches are cut into pages of that many rows, stored in a
    seeded random order and addressed through a block table."""
    from exact_attention_24_amd.inputs import WORKLOADS, kvcache_inputs
    w = WORKLOADS["kvcache_b8_h32"]
    q, kc, vc, kn, vn = (x.cuda() for x in kvcache_inputs(w.batch, w.seqlen, w.heads, w.head_dim, 1, seed=w.seed))
    table = None
    if page:
        mb = w.seqlen // page
        perm = torch.randperm(w.batch * mb, generator=torch.Generator().manual_seed(9)).cuda()
        table = perm.reshape(w.batch, mb).to(torch.int32)
        shape = (w.batch * mb, page, w.heads, w.head_dim)
        kb, vb = torch.empty(shape, dtype=kc.dtype, device="cuda"), torch.empty(shape, dtype=kc.dtype, device="cuda")
        kb[perm] = kc.reshape(shape)
        vb[perm] = vc.reshape(shape)
        kc, vc = kb, vb
    seq = torch.full((w.batch,), w.seqlen - 1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(w.batch, w.heads, 1, dtype=torch.float32, device="cuda")
    row = w.batch * w.heads * w.head_dim * 2
    nbytes = 2 * w.seqlen * row + 4 * row + w.batch * w.heads * 4
    fn = lambda: fa.fa_fwd_kvcache(q, kc, vc, kn, vn, cache_seqlens=seq, causal=True, out=out, lse=lse,
                                   block_table=table)
    return fn, nbytes


WORKLOAD_CHOICES = ("fwd_causal", "fwd_noncausal", "fwd_short", "bwd", "varlen", "varlen_bwd", "fp8", "merge",
                    "kvcache")


def make_step(name, torch, fa):
    """(step fn, work per step, description, dtype, peak, kernel source, unit) of a workload, inputs
    generated and moved to HBM before timing; work is FLOPs (unit TFLOP/s) or bytes (unit GB/s)."""
    from exact_attention_24_amd.inputs import WORKLOADS, workload_inputs
    if name in ("fwd_causal", "fwd_noncausal"):
        causal = name == "fwd_causal"
        w = WORKLOADS["llama_n8192"]
        t = workload_inputs("llama_n8192")
        q, k, v = (t[x].cuda() for x in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((1, w.heads, w.seqlen), dtype=torch.float32, device="cuda")
        desc = f"fwd B1 H32 N8192 d128 bf16 {'causal' if causal else 'non-causal'} (Llama-7B attention shape)"
        return (lambda: fa.fa_fwd(q, k, v, causal=causal, out=o, lse=lse),
                fwd_flops(1, 32, 8192, 128, causal), desc, "bf16", PEAK_BF16_TFLOPS, "fa_fwd.hip", "TFLOP/s")
    if name == "fwd_short":
        t = workload_inputs("b2_h16_n1024")
        q, k, v = (t[x].cuda() for x in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((2, 16, 1024), dtype=torch.float32, device="cuda")
        return (lambda: fa.fa_fwd(q, k, v, causal=True, out=o, lse=lse), fwd_flops(2, 16, 1024, 64, True),
                "fwd B2 H16 N1024 d64 bf16 causal (the MindSpore API example; split-key launch)", "bf16",
                PEAK_BF16_TFLOPS, "fa_fwd_split.hip", "TFLOP/s")
    if name == "bwd":
        t = {k_: v_.cuda() for k_, v_ in workload_inputs("bwd_n8192").items()}
        o, lse = fa.fa_fwd(t["q"], t["k"], t["v"], causal=True)
        dq, dk, dv = (torch.empty(t[x].shape, dtype=torch.float32, device="cuda") for x in ("q", "k", "v"))
        return (lambda: fa.fa_bwd(t["dout"], t["q"], t["k"], t["v"], o, lse, causal=True, dq=dq, dk=dk, dv=dv),
                2.5 * fwd_flops(1, 32, 8192, 128, True), "bwd B1 H32 N8192 d128 bf16 causal, fp32 gradients",
                "bf16", PEAK_BF16_TFLOPS, "fa_bwd.hip", "TFLOP/s")
    if name == "varlen":
        w = WORKLOADS["varlen_32k"]
        t = workload_inputs("varlen_32k")
        q, k, v, cu = (t[x].cuda() for x in ("q", "k", "v", "cu_seqlens"))
        mx = max(t["lengths"])
        f = 4.0 * w.head_dim * w.heads * visible_pairs_varlen(t["lengths"], True, w.window)
        return (lambda: fa.fa_varlen_fwd(q, k, v, cu, mx, causal=True, window=w.window), f,
                "varlen fwd 32768 tokens H28 d128 bf16 causal window 4096", "bf16", PEAK_BF16_TFLOPS, "fa_fwd.hip",
                "TFLOP/s")
    if name == "varlen_bwd":
        w = WORKLOADS["varlen_bwd_32k"]
        t = workload_inputs("varlen_bwd_32k")
        q, k, v, do, cu = (t[x].cuda() for x in ("q", "k", "v", "dout", "cu_seqlens"))
        mx = max(t["lengths"])
        o, lse = fa.fa_varlen_fwd(q, k, v, cu, mx, causal=True, window=w.window)
        dq, dk, dv = (torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in (q, k, v))
        f = 2.5 * 4.0 * w.head_dim * w.heads * visible_pairs_varlen(t["lengths"], True, w.window)
        return (lambda: fa.fa_varlen_bwd(do, q, k, v, o, lse, cu, mx, causal=True, window=w.window, dq=dq, dk=dk,
                                         dv=dv), f,
                "varlen bwd 32768 tokens H28 d128 bf16 causal window 4096, fp32 gradients", "bf16",
                PEAK_BF16_TFLOPS, "fa_bwd.hip", "TFLOP/s")
    if name == "kvcache":
        fn, nbytes = kvcache_step(torch, fa)
        return (fn, nbytes, "KV-cache decode step B8 H32 d128, 8191 cached + 1 new token, causal", "bf16",
                PEAK_HBM_GBS, "fa_decode.hip", "GB/s")
    if name == "merge":
        o_p, lse_p, out, lse, nbytes = merge_inputs(torch)
        return (lambda: fa.fa_merge(o_p, lse_p, out=out, lse=lse), nbytes,
                "merge of 8 fp32 partial results, B1 N8192 H32 d128 -> bf16", "f32", PEAK_HBM_GBS, "fa_merge.hip",
                "GB/s")
    t = workload_inputs("fp8_n8192")
    q8, k8, v8 = (t[x].cuda() for x in ("q8", "k8", "v8"))
    ds = (t["q_scale"], t["k_scale"], t["v_scale"])
    return (lambda: fa.fa_fwd(q8, k8, v8, causal=True, descale=ds), fwd_flops(1, 32, 8192, 128, True),
            "fwd B1 H32 N8192 d128 fp8-e4m3 causal", "fp8_e4m3", PEAK_FP8_TFLOPS, "fa_fp8.hip", "TFLOP/s")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the timed oracle sample")
    ap.add_argument("--no-rows", action="store_true", help="skip the other hot-path rows")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (HBM-counter calibration)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--workload", default="fwd_causal",
                    help="what one step runs: " + ", ".join(WORKLOAD_CHOICES) +
                         " (default fwd_causal, the headline; the others are for profiling runs)")
    args = ap.parse_args()

    if args.workload not in WORKLOAD_CHOICES:
        ap.error(f"--workload must be one of {WORKLOAD_CHOICES}")
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_24_amd as fa
    from exact_attention_24_amd.inputs import WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa.lib()  # fail loudly if the HIP library is missing
    headline = args.workload == "fwd_causal"
    step, work, desc, dtype, peak, src, unit = make_step(args.workload, torch, fa)
    log(f"[bench] {torch.cuda.get_device_name(0)}; workload {desc}")

    wall_ms, per_call = time_calls(step, args.warmup, args.steps, torch)
    ms_per_step = wall_ms / args.steps
    kernel_ms = sum(per_call) / len(per_call)
    per_unit = 1e12 if unit == "TFLOP/s" else 1e9
    value = work / (ms_per_step * 1e-3) / per_unit
    achieved = work / (kernel_ms * 1e-3) / per_unit
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step (wall), per-call avg {kernel_ms:.4f} ms, "
        f"{achieved:.1f} {unit}")

    if args.calib_copy:
        src_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst_buf = torch.empty_like(src_buf)
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        log("[bench] calibration copy of 1 GiB done")

    # the kernel's code depends on its source file and the shared device headers
    sha = src_hash(src, "fa_device.h", "fa_internal.h")
    cpu = None if (args.no_cpu_baseline or not headline) else cpu_baseline(args.cpu_budget)
    rows = {} if (args.no_rows or not headline) else config_rows(torch, fa, max(5, min(args.steps, 20)), cpu)

    out = {
        "metric": "attention fwd TFLOP/s + % MFMA peak, bf16 causal N=8192 d=128, 1 GPU" if headline else
                  f"{args.workload} {unit} (profiling workload, not the headline)",
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) inputs (see exact_attention_24_amd/inputs.py)",
        "config": {"workload": desc, "parallelism": "none (1 GPU)",
                   "inputs": "resident in HBM; the 201 MB of Q/K/V also stay in the 256 MB MALL between calls "
                             "(rows.cfg3_fwd_causal_two_input_sets times the same call with them evicted)"},
        "pct_mfma_peak" if unit == "TFLOP/s" else "pct_hbm_peak": round(100 * value / peak, 2),
        "roofline": {"bound": "mfma" if unit == "TFLOP/s" else "hbm", "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic_from_profile(sha) if headline else None, "kernel_src_sha": sha},
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
