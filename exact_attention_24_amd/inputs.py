"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module only draws random numbers and casts them to the storage types the
kernels read; it holds none of the attention arithmetic.  Both sides of every
parity check receive the very same tensors from here.

Workloads (the shapes of the pages' examples and model configurations):
  tiny_fp32      B1 H1 N256 d64, fp32, non-causal
  b2_h16_n1024   B2 H16 N1024 d64, bf16, causal (the packed-QKV API example
                 of the MindSpore page, "核心API与使用示例", without dropout)
  llama_n8192    B1 H32 N8192 d128, bf16 (Llama-7B attention shape at 8K)
  varlen_32k     28 heads, d128, 32768 packed tokens, lengths U{512..8192},
                 causal + window 4096 (packing of mixed lengths, ms-swift
                 long-text page section 5.1)
  bwd_n8192      B1 H32 N8192 d128, bf16 Q/K/V/dO, causal
  varlen_bwd_32k the varlen_32k packing (same seed, so the same lengths and
                 Q/K/V) plus a bf16 dO, for the packed backward
  fp8_n8192      same shape, e4m3 Q/K/V with per-tensor scales, causal
  kvcache_b2_h16 the KV-cache decode loop of the MindSpore page (推理优化与KV缓存):
                 B2, cache 2048, H16, d64, one new token per step, causal
  kvcache_b8_h32 one decode step at the Llama-7B shape: B8, H32, d128, 8191
                 cached tokens + 1 new (cache 8192), causal

Recipe: one ``torch.Generator('cpu')`` per workload seeded with its seed;
Q, K, V (then dO) drawn in that order as i.i.d. N(0, 1) float32 and cast to
the storage dtype with round-to-nearest-even.  Varlen lengths come from
``numpy.random.default_rng(seed)``: integers in [512, 8192] drawn until their
sum reaches the token total, the last one truncated so the sum is exact.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seqlen: int
    head_dim: int
    dtype: str            # "f32" | "bf16" | "fp8"
    causal: bool
    window: int = 0
    seed: int = 0
    varlen_total: int = 0  # > 0: packed varlen workload with this many tokens
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 256, 64, "f32", False, seed=1001),
    "b2_h16_n1024": Workload("b2_h16_n1024", 2, 16, 1024, 64, "bf16", True, seed=1002),
    "llama_n8192": Workload("llama_n8192", 1, 32, 8192, 128, "bf16", True, seed=1003),
    "llama_n8192_noncausal": Workload("llama_n8192_noncausal", 1, 32, 8192, 128, "bf16", False, seed=1003),
    "varlen_32k": Workload("varlen_32k", 1, 28, 8192, 128, "bf16", True, window=4096, seed=1004,
                           varlen_total=32768),
    "bwd_n8192": Workload("bwd_n8192", 1, 32, 8192, 128, "bf16", True, seed=1005),
    "varlen_bwd_32k": Workload("varlen_bwd_32k", 1, 28, 8192, 128, "bf16", True, window=4096, seed=1004,
                               varlen_total=32768),
    "fp8_n8192": Workload("fp8_n8192", 1, 32, 8192, 128, "fp8", True, seed=1005),
    "kvcache_b2_h16": Workload("kvcache_b2_h16", 2, 16, 2048, 64, "bf16", True, seed=1007),
    "kvcache_b8_h32": Workload("kvcache_b8_h32", 8, 32, 8192, 128, "bf16", True, seed=1008),
}

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}

FP8_MAX = 448.0  # largest finite OCP e4m3 value


def randn(gen: torch.Generator, shape, dtype: str) -> torch.Tensor:
    """N(0,1) float32 draw cast to the storage dtype ("f32" or "bf16")."""
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x.to(_TORCH_DT[dtype])


def dense_inputs(batch, seqlen, heads, head_dim, dtype="bf16", seed=0, with_dout=False,
                 seqlen_k=None):
    """Q [B,Nq,H,d], K/V [B,Nk,H,d] (and dO [B,Nq,H,d]) on the CPU, seeded."""
    gen = torch.Generator("cpu").manual_seed(seed)
    nk = seqlen if seqlen_k is None else seqlen_k
    q = randn(gen, (batch, seqlen, heads, head_dim), dtype)
    k = randn(gen, (batch, nk, heads, head_dim), dtype)
    v = randn(gen, (batch, nk, heads, head_dim), dtype)
    if not with_dout:
        return q, k, v
    do = randn(gen, (batch, seqlen, heads, head_dim), dtype)
    return q, k, v, do


def varlen_lengths(total: int, seed: int, lo: int = 512, hi: int = 8192) -> list:
    """Integer lengths U{lo..hi} drawn until they reach ``total``; last truncated."""
    rng = np.random.default_rng(seed)
    out, acc = [], 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return out


def cu_seqlens_of(lengths) -> torch.Tensor:
    """int32 prefix offsets [num_seqs + 1] with cu[0] = 0."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return torch.from_numpy(cu.astype(np.int32))


def varlen_inputs(lengths, heads, head_dim, dtype="bf16", seed=0, with_dout=False):
    """Packed Q/K/V [total, H, d] and cu_seqlens for the given lengths (then dO)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    total = int(sum(lengths))
    q = randn(gen, (total, heads, head_dim), dtype)
    k = randn(gen, (total, heads, head_dim), dtype)
    v = randn(gen, (total, heads, head_dim), dtype)
    if not with_dout:
        return q, k, v, cu_seqlens_of(lengths)
    do = randn(gen, (total, heads, head_dim), dtype)
    return q, k, v, cu_seqlens_of(lengths), do


def kvcache_inputs(batch, cache_len, heads, head_dim, nq, seed=0):
    """KV-cache decode inputs on the CPU: q, k_cache, v_cache, k_new, v_new,
    drawn in that order (the caches whole, every row random)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = randn(gen, (batch, nq, heads, head_dim), "bf16")
    kc = randn(gen, (batch, cache_len, heads, head_dim), "bf16")
    vc = randn(gen, (batch, cache_len, heads, head_dim), "bf16")
    kn = randn(gen, (batch, nq, heads, head_dim), "bf16")
    vn = randn(gen, (batch, nq, heads, head_dim), "bf16")
    return q, kc, vc, kn, vn


def spike_keys(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float, every: int = 1024,
               phase: int = 300, group: int = 8, level: float = 9.0, voff: float = 0.3, rest: float = 0.1):
    """Inputs whose row maximum of the logits jumps in the middle of the key loop.

    q, k, v: [..., seqlen, heads, d] (token axis -3).  Every query gets first
    coordinate 1 and its other coordinates scaled by ``rest``; every key gets
    first coordinate 0 except the spike keys, groups of ``group`` consecutive
    keys starting at phase (mod every), which get level / (scale log2 e).  A
    spike key's logit then exceeds the others' by about ``level`` in base-2
    units (the rest spread by about rest sqrt(d) scale log2 e around 0), so a
    row's running maximum rises by more than 8 when the row reaches its first
    spike group after its first key tile.  A group's weight (group 2^level)
    is of the order of that of the ~1000 ordinary keys before it, and no key
    carries much of a row's weight.  V rows of ordinary keys are shifted by
    +voff, those of spike keys by -voff (alternating in sign along the head
    dimension), so the output depends strongly on how the weights before and
    after the jump are combined.  Returns new q, k, v of the input dtypes."""
    qf, kf, vf = q.float().clone(), k.float().clone(), v.float().clone()
    qf[..., 1:] *= rest
    qf[..., 0] = 1.0
    n = kf.shape[-3]
    j = torch.arange(n)
    hit = ((j - phase) % every) < group
    amp = torch.where(hit, level / (scale * 1.4426950408889634), 0.0)
    sign = torch.where(hit, -voff, voff)
    shape = [1] * (kf.dim() - 1)
    shape[-2] = n
    kf[..., 0] = amp.reshape(shape).expand(kf.shape[:-1])
    d = vf.shape[-1]
    pattern = torch.where(torch.arange(d) % 2 == 0, 1.0, -1.0)
    vf += sign.reshape(shape + [1]) * pattern
    return qf.to(q.dtype), kf.to(k.dtype), vf.to(v.dtype)


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor e4m3 quantisation done by the caller before the fp8 forward.

    scale = amax|x| / 448 (fp32); codes = RNE cast of x / scale to
    torch.float8_e4m3fn (the OCP format).  Returns (codes, scale) where the
    tensor represents codes * scale.
    """
    xf = x.float()
    amax = float(xf.abs().max())
    scale = float(np.float32(amax / FP8_MAX)) if amax > 0 else 1.0
    codes = (xf / scale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, scale


def workload_inputs(name: str, seqlen: int | None = None, heads: int | None = None):
    """The tensors of a named workload (optionally with fewer tokens/heads).

    Returns a dict with CPU tensors: q, k, v (and dout for the backward
    workload; q8/k8/v8 + scales for fp8; cu_seqlens + lengths for varlen).
    """
    w = WORKLOADS[name]
    n = w.seqlen if seqlen is None else seqlen
    h = w.heads if heads is None else heads
    with_do = "bwd" in name
    if w.varlen_total:
        total = w.varlen_total if seqlen is None else seqlen
        lengths = varlen_lengths(total, w.seed)
        t = varlen_inputs(lengths, h, w.head_dim, w.dtype, w.seed, with_dout=with_do)
        d = {"q": t[0], "k": t[1], "v": t[2], "cu_seqlens": t[3], "lengths": lengths}
        if with_do:
            d["dout"] = t[4]
        return d
    if w.dtype == "fp8":
        q, k, v = dense_inputs(w.batch, n, h, w.head_dim, "bf16", w.seed)
        q8, sq = quantize_e4m3(q)
        k8, sk = quantize_e4m3(k)
        v8, sv = quantize_e4m3(v)
        return {"q8": q8, "k8": k8, "v8": v8, "q_scale": sq, "k_scale": sk, "v_scale": sv}
    t = dense_inputs(w.batch, n, h, w.head_dim, w.dtype, w.seed, with_dout=with_do)
    d = {"q": t[0], "k": t[1], "v": t[2]}
    if with_do:
        d["dout"] = t[3]
    return d
