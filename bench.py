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
import math
import os
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


def cpu_baseline(budget_s=15.0):
    """The fp64 oracle on a bounded sample of the same workload: whole heads of
    the causal N=8192 d=128 forward, one after another, until budget_s."""
    import numpy as np
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
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    cores = threads or len(os.sched_getaffinity(0))
    flops = fwd_flops(1, heads, w.seqlen, w.head_dim, True)
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of 32 heads of the B1 H32 N8192 d128 causal forward, fp64 NumPy, {el:.1f} s",
            "seconds": round(el, 2)}


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


def extra_rows(torch, fa, steps):
    """Timings of the other hot-path rows (median per call, HIP events)."""
    from exact_attention_24_amd.inputs import WORKLOADS, workload_inputs
    rows = {}

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2]

    # non-causal forward
    t = {k_: v_.cuda() for k_, v_ in workload_inputs("llama_n8192").items()}
    _, ms = time_calls(lambda: fa.fa_fwd(t["q"], t["k"], t["v"], causal=False), 2, steps, torch)
    f = fwd_flops(1, 32, 8192, 128, False)
    rows["fwd_noncausal_n8192"] = {"ms": round(med(ms), 4), "tflops": round(f / med(ms) / 1e9, 1)}
    # backward
    try:
        w = WORKLOADS["bwd_n8192"]
        t = {k_: v_.cuda() for k_, v_ in workload_inputs("bwd_n8192").items() if hasattr(v_, "cuda")}
        o, lse = fa.fa_fwd(t["q"], t["k"], t["v"], causal=True)
        _, ms = time_calls(lambda: fa.fa_bwd(t["dout"], t["q"], t["k"], t["v"], o, lse, causal=True), 2, steps,
                           torch)
        f = 2.5 * fwd_flops(1, 32, 8192, 128, True)
        rows["bwd_causal_n8192"] = {"ms": round(med(ms), 4), "tflops": round(f / med(ms) / 1e9, 1)}
    except Exception as e:  # not available in this build
        rows["bwd_causal_n8192"] = {"error": str(e)[:120]}
    # dropout (p = 0.1) forward and backward at the same shape
    try:
        t = {k_: v_.cuda() for k_, v_ in workload_inputs("bwd_n8192").items() if hasattr(v_, "cuda")}
        kw = dict(causal=True, dropout_p=0.1, seed=1234, offset=0)
        _, ms = time_calls(lambda: fa.fa_fwd(t["q"], t["k"], t["v"], **kw), 2, steps, torch)
        f = fwd_flops(1, 32, 8192, 128, True)
        rows["fwd_causal_dropout0.1_n8192"] = {"ms": round(med(ms), 4), "tflops": round(f / med(ms) / 1e9, 1)}
        o, lse = fa.fa_fwd(t["q"], t["k"], t["v"], **kw)
        _, ms = time_calls(lambda: fa.fa_bwd(t["dout"], t["q"], t["k"], t["v"], o, lse, **kw), 2, steps, torch)
        rows["bwd_causal_dropout0.1_n8192"] = {"ms": round(med(ms), 4), "tflops": round(2.5 * f / med(ms) / 1e9, 1)}
    except Exception as e:
        rows["fwd_causal_dropout0.1_n8192"] = {"error": str(e)[:120]}
    # varlen
    try:
        w = WORKLOADS["varlen_32k"]
        t = workload_inputs("varlen_32k")
        q, k, v, cu = (t[x].cuda() for x in ("q", "k", "v", "cu_seqlens"))
        mx = max(t["lengths"])
        _, ms = time_calls(lambda: fa.fa_varlen_fwd(q, k, v, cu, mx, causal=True, window=w.window), 2, steps,
                           torch)
        f = 4.0 * w.head_dim * w.heads * visible_pairs_varlen(t["lengths"], True, w.window)
        rows["varlen_32k_w4096"] = {"ms": round(med(ms), 4), "tflops": round(f / med(ms) / 1e9, 1)}
    except Exception as e:
        rows["varlen_32k_w4096"] = {"error": str(e)[:120]}
    # varlen backward
    try:
        w = WORKLOADS["varlen_bwd_32k"]
        t = workload_inputs("varlen_bwd_32k")
        q, k, v, do, cu = (t[x].cuda() for x in ("q", "k", "v", "dout", "cu_seqlens"))
        mx = max(t["lengths"])
        o, lse = fa.fa_varlen_fwd(q, k, v, cu, mx, causal=True, window=w.window)
        _, ms = time_calls(lambda: fa.fa_varlen_bwd(do, q, k, v, o, lse, cu, mx, causal=True, window=w.window),
                           2, steps, torch)
        f = 2.5 * 4.0 * w.head_dim * w.heads * visible_pairs_varlen(t["lengths"], True, w.window)
        rows["varlen_bwd_32k_w4096"] = {"ms": round(med(ms), 4), "tflops": round(f / med(ms) / 1e9, 1)}
    except Exception as e:
        rows["varlen_bwd_32k_w4096"] = {"error": str(e)[:120]}
    # merge of partial results
    try:
        o_p, lse_p, out, lse, nbytes = merge_inputs(torch)
        _, ms = time_calls(lambda: fa.fa_merge(o_p, lse_p, out=out, lse=lse), 2, steps, torch)
        gbs = nbytes / med(ms) / 1e6
        rows["merge_8parts_n8192"] = {"ms": round(med(ms), 4), "GB/s": round(gbs, 1),
                                      "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        del o_p, lse_p, out, lse
    except Exception as e:
        rows["merge_8parts_n8192"] = {"error": str(e)[:120]}
    # KV-cache decode step
    try:
        fn, nbytes = kvcache_step(torch, fa)
        _, ms = time_calls(fn, 2, steps, torch)
        gbs = nbytes / med(ms) / 1e6
        rows["kvcache_decode_b8_h32_8k"] = {"ms": round(med(ms), 4), "GB/s": round(gbs, 1),
                                            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    except Exception as e:
        rows["kvcache_decode_b8_h32_8k"] = {"error": str(e)[:120]}
    try:
        fn, nbytes = kvcache_step(torch, fa, page=256)
        _, ms = time_calls(fn, 2, steps, torch)
        gbs = nbytes / med(ms) / 1e6
        rows["kvcache_paged256_decode_b8_h32_8k"] = {"ms": round(med(ms), 4), "GB/s": round(gbs, 1),
                                                     "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    except Exception as e:
        rows["kvcache_paged256_decode_b8_h32_8k"] = {"error": str(e)[:120]}
    # fp8 forward
    try:
        t = workload_inputs("fp8_n8192")
        q8, k8, v8 = (t[x].cuda() for x in ("q8", "k8", "v8"))
        ds = (t["q_scale"], t["k_scale"], t["v_scale"])
        _, ms = time_calls(lambda: fa.fa_fwd(q8, k8, v8, causal=True, descale=ds), 2, steps, torch)
        f = fwd_flops(1, 32, 8192, 128, True)
        rows["fp8_fwd_causal_n8192"] = {"ms": round(med(ms), 4), "tflops": round(f / med(ms) / 1e9, 1),
                                        "frac_fp8_peak": round(f / med(ms) / 1e9 / PEAK_FP8_TFLOPS, 4)}
    except Exception as e:
        rows["fp8_fwd_causal_n8192"] = {"error": str(e)[:120]}
    return rows


WORKLOAD_CHOICES = ("fwd_causal", "fwd_noncausal", "bwd", "varlen", "varlen_bwd", "fp8", "merge", "kvcache")


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
    rows = {} if (args.no_rows or not headline) else extra_rows(torch, fa, max(5, min(args.steps, 20)))
    if rows:
        log(f"[bench] rows: {json.dumps(rows)}")
    cpu = None if (args.no_cpu_baseline or not headline) else cpu_baseline(args.cpu_budget)

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
        "config": {"workload": desc, "parallelism": "none (1 GPU)"},
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
