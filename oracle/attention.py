"""CPU fp64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it and shares no code with it: the two meet only on the seeded
inputs that ``exact_attention_24_amd.inputs`` generates.

What is computed, and where the pages define it
------------------------------------------------
* Forward: O = softmax(scale * Q K^T + mask) V, with the N x N score matrix
  S written out in full.  Definition: the attention formula at the top of
  "Flash-Attention 2/3在ms-swift中的集成与性能提升" (bxzpzcl.cn), the formula in
  section 一 of the adg.csdn.net flash_attn/Qwen page, and the standard flow of
  "FlashAttention优化Transformer显存与计算效率" (jsqmd.com) section 2.1.
  The method is exact, not an approximation (ms-swift long-text page, section
  3.3; adg.csdn.net page, section 三; MindSpore page, "技术背景与核心优势"), so the
  plain definition is the oracle.
* Masks: causal and sliding window are the structured masks of the FA-3
  paragraph of the ms-swift integration page; ``causal=True`` appears on every
  API example of the MindSpore page.
* LSE = m + ln(sum exp(S - m)) per row: the only forward residual the
  recomputing backward needs ("重计算" in the ms-swift integration page and in
  section 三 of the adg.csdn.net page).
* Backward: the pages only say that S is recomputed rather than stored, so the
  gradients are the textbook chain rule of L = sum(dO * O), written out with
  this module's own fp64 P and O.
* ``blocked_fwd``: the blockwise softmax of jsqmd.com section 2.2.2 (per-block
  max m and exponent sum l, combined in a numerically stable way), with the
  tile loop of section 2.2.1.  It exists to pin that the tiled recombination
  equals the direct softmax; it is not the GPU algorithm.
* ``merge_partials``: attention results over disjoint key subsets, each
  normalised over its own keys and carried as (O_p, LSE_p), combined into the
  result over the union.  This is the stable combination of per-block max m
  and exponent sum l of jsqmd.com section 2.2.2, with each part written as
  LSE_p = m_p + ln l_p; it is also the step that joins the local results of
  ring attention (the Ring-Attention paragraph of the ms-swift integration
  page).
* ``kvcache_fwd``: incremental decoding against a KV cache, the
  ``flash_attn_with_kvcache(q, k_cache, v_cache, k, v, cache_seqlens, causal)``
  example of the MindSpore page (推理优化与KV缓存): the new k, v are written into
  the cache at position cache_seqlens, then q attends over the cache up to and
  including them.
* ``kvcache_paged_fwd``: the same step with the caches stored in fixed-size
  pages (the paged storage of the same section): logical row j of batch entry
  b is row j mod P of page block_table[b, j div P].
* Dropout on the attention probabilities (``dropout_p`` on every API
  signature of the MindSpore page; fused with softmax and mask in the FA-2
  paragraph of the ms-swift integration page): O = (P * keep * s) V with
  LSE unchanged.  The keep mask comes from the counter-based generator
  Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
  as 1, 2, 3", SC 2011), written here from that paper's definition, so the
  backward can regenerate it instead of storing it:
    - one random byte per (query row i, key j) of head slot
      b * heads + h: byte (j mod 4) of word ((j mod 32) div 8) of
      Philox(counter = (2 (j div 32) + ((j div 4) mod 2), i, slot, offset),
      key = (seed mod 2^32, seed div 2^32));
    - the element is kept iff its byte < K = round(256 (1 - p)) (at least 1),
      and kept values are scaled by s = 256 / K, so p is in effect rounded to
      a multiple of 1/256 and the expectation of O is the undropped O.
  The backward is the chain rule through the same mask: dV = (P keep s)^T
  dO, dP = keep s (dO V^T), D = rowsum(dO * O), dS = P (dP - D).
* fp8: ``e4m3_decode`` follows the OCP 8-bit floating point specification for
  E4M3 (bias 7, no infinities, S.1111.111 is NaN, max finite 448); the fp8
  forward is the plain definition applied to code * per-tensor scale (FA-3 FP8
  paragraph of the ms-swift integration page).

Readings where the pages are silent
-----------------------------------
* ``scale`` is applied as given; callers pass 1/sqrt(d) for the pages' default.
* ``window = W > 0``: a query at aligned position p sees keys j with
  p - W < j (W keys including itself); a left bound only.
* Causal with Nq != Nk is bottom-right aligned: query i sits at key position
  i + Nk - Nq.
* A query row with no visible key gets O = 0 and LSE = -inf.
* KV cache: with new keys, batch b sees keys 0 .. cache_seqlens[b] + Nq - 1
  (the Nq new ones last); without, keys 0 .. cache_seqlens[b] - 1.  The Nq
  queries are the last Nq positions (bottom-right causal).  Cache rows past
  that length are never read.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, hand-derived golden values, finite differences, invariants and
torch's CPU attention routine.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "visible",
    "attention_fwd",
    "attention_probs",
    "attention_bwd",
    "blocked_fwd",
    "mha_fwd",
    "mha_bwd",
    "varlen_fwd",
    "varlen_bwd",
    "philox4x32",
    "dropout_index",
    "dropout_bytes",
    "dropout_keep",
    "merge_partials",
    "kvcache_fwd",
    "paged_gather",
    "kvcache_paged_fwd",
    "e4m3_decode",
    "fp8_dequant",
]


def visible(q_pos, nk, causal, window, offset=0):
    """Boolean [len(q_pos), nk] matrix: may query q_pos[a] see key j?

    q_pos are query indices in [0, Nq); offset = Nk - Nq aligns them to key
    positions (bottom-right).  Causal: j <= p.  Window W > 0: j > p - W.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    p = (q_pos + offset)[:, None]
    j = np.arange(nk, dtype=np.int64)[None, :]
    ok = np.ones((q_pos.shape[0], nk), dtype=bool)
    if causal:
        ok &= j <= p
    if window > 0:
        ok &= j > p - window
    return ok


def _scores(q, k, scale, causal, window, q_pos, nq):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if q_pos is None:
        q_pos = np.arange(q.shape[0])
    if nq is None:
        nq = q.shape[0]
    s = float(scale) * (q @ k.T)
    ok = visible(q_pos, k.shape[0], causal, window, offset=k.shape[0] - nq)
    return np.where(ok, s, -np.inf)


def _softmax_rows(s):
    """Stable row softmax of masked scores; returns (P, m, l)."""
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 on masked entries
    l = p.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(l[:, None] > 0, p / l[:, None], 0.0)
    return p, m_safe, l


def attention_probs(q, k, scale, causal=False, window=0, q_pos=None, nq=None):
    """P = softmax(scale * Q K^T + mask), row by row (fp64)."""
    p, _, _ = _softmax_rows(_scores(q, k, scale, causal, window, q_pos, nq))
    return p


def attention_fwd(q, k, v, scale, causal=False, window=0, q_pos=None, nq=None, drop=None):
    """One head: q [nq_sel, d], k [nk, d], v [nk, dv] -> (O [nq_sel, dv], LSE [nq_sel]).

    ``q_pos`` (default 0..nq_sel-1) gives the index of each given row in a
    query sequence of length ``nq`` (default nq_sel), so that sampled rows of a
    long sequence can be checked one by one.  LSE is natural-log.
    ``drop`` = (keep [nq_sel, nk] bool, s): dropout of the probabilities.
    """
    s = _scores(q, k, scale, causal, window, q_pos, nq)
    p, m, l = _softmax_rows(s)
    if drop is not None:
        p = p * drop[0] * drop[1]
    o = p @ np.asarray(v, dtype=np.float64)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(l), -np.inf)
    return o, lse


def attention_bwd(q, k, v, dout, scale, causal=False, window=0, drop=None):
    """One head, all rows: gradients of L = sum(dout * O) w.r.t. q, k, v (fp64).

    D_i = sum_c dO_ic O_ic;  dV = P^T dO;  dP = dO V^T;  dS = P * (dP - D);
    dQ = scale dS K;  dK = scale dS^T Q.  With ``drop`` = (keep, s) the
    forward used P keep s, so dV = (P keep s)^T dO and dP = keep s (dO V^T).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    p = attention_probs(q, k, scale, causal, window)
    ks = np.ones_like(p) if drop is None else drop[0] * float(drop[1])
    o = (p * ks) @ v
    d_row = (do * o).sum(axis=1)
    dv = (p * ks).T @ do
    dp = (do @ v.T) * ks
    ds = p * (dp - d_row[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def blocked_fwd(q, k, v, scale, causal=False, window=0, br=16, bc=16):
    """Blockwise online softmax over key blocks (jsqmd.com section 2.2.2).

    For each block of ``br`` query rows, keep per row a running max m, a
    running exponent sum l and an unnormalised output acc.  Each key block of
    ``bc`` keys that the mask leaves at least partly visible updates them:
      m' = max(m, rowmax S_blk);  alpha = exp(m - m') (0 while m = -inf);
      P~ = exp(S_blk - m') (0 where masked);  l = alpha l + rowsum P~;
      acc = alpha acc + P~ V_blk;  m = m'.
    Key blocks the mask hides entirely for the whole row block are skipped.
    At the end O = acc / l and LSE = m + ln l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk, dv = q.shape[0], k.shape[0], v.shape[1]
    o = np.zeros((nq, dv))
    lse = np.full(nq, -np.inf)
    for r0 in range(0, nq, br):
        rows = np.arange(r0, min(r0 + br, nq))
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, dv))
        for c0 in range(0, nk, bc):
            cols = np.arange(c0, min(c0 + bc, nk))
            ok = visible(rows, nk, causal, window, offset=nk - nq)[:, cols]
            if not ok.any():
                continue  # tile skipping: nothing visible in this block
            s = float(scale) * (q[rows] @ k[cols].T)
            s = np.where(ok, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            finite = np.isfinite(m_new)
            m_ref = np.where(finite, m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
            pt = np.exp(s - m_ref[:, None])
            l = alpha * l + pt.sum(axis=1)
            acc = alpha[:, None] * acc + pt @ v[cols]
            m = m_new
        has = l > 0
        o[rows[has]] = acc[has] / l[has, None]
        lse[rows[has]] = m[has] + np.log(l[has])
    return o, lse


def philox4x32(counter, key, rounds=10):
    """Philox4x32 (Salmon et al., SC 2011): counter [..., 4], key (k0, k1) of
    unsigned 32-bit words -> [..., 4] uint32.

    Each round multiplies words 0 and 2 by 0xD2511F53 and 0xCD9E8D57 into
    64-bit products (hi, lo) and forms (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1,
    lo0); between rounds the key is bumped by the Weyl constants 0x9E3779B9
    and 0xBB67AE85 (mod 2^32).
    """
    m32 = np.uint64(0xFFFFFFFF)
    c = np.asarray(counter, dtype=np.uint64) & m32
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    for r in range(rounds):
        if r:
            k0 = (k0 + np.uint64(0x9E3779B9)) & m32
            k1 = (k1 + np.uint64(0xBB67AE85)) & m32
        p0 = np.uint64(0xD2511F53) * c0
        p1 = np.uint64(0xCD9E8D57) * c2
        c0, c1, c2, c3 = (p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & m32, (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & m32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def dropout_index(slot, q_rows, nk, offset):
    """Where the random byte of each element (query row i, key j) of head slot
    ``slot`` comes from: (counter [len(q_rows), nk, 4], word [len(q_rows), nk],
    byte [len(q_rows), nk]) -- the Philox counter (2 (j div 32) + (j div 4)
    mod 2, i, slot, offset), word (j mod 32) div 8 of its output, byte j mod 4
    of that word (see the module docstring)."""
    i = np.asarray(q_rows, dtype=np.uint64)[:, None]
    j = np.arange(nk, dtype=np.uint64)[None, :]
    ctr = np.stack(np.broadcast_arrays(2 * (j >> np.uint64(5)) + ((j >> np.uint64(2)) & np.uint64(1)), i,
                                       np.uint64(slot), np.uint64(offset & 0xFFFFFFFF)), axis=-1)
    shape = ctr.shape[:2]
    word = np.broadcast_to(((j & np.uint64(31)) >> np.uint64(3)).astype(np.int64), shape)
    byte = np.broadcast_to((j & np.uint64(3)).astype(np.int64), shape)
    return ctr, word, byte


def dropout_bytes(slot, q_rows, nk, seed, offset):
    """Random bytes [len(q_rows), nk] of head slot ``slot``: byte ``byte`` of
    word ``word`` of Philox4x32-10 at ``counter`` (dropout_index)."""
    ctr, word, byte = dropout_index(slot, q_rows, nk, offset)
    words = philox4x32(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))   # [rows, nk, 4]
    w = np.take_along_axis(words, word[..., None], axis=-1)[..., 0]
    return ((w >> (np.uint32(8) * byte.astype(np.uint32))) & np.uint32(0xFF)).astype(np.uint8)


def dropout_keep(slot, q_rows, nk, seed, offset, p):
    """(keep [len(q_rows), nk] bool, s): keep iff byte < K = round(256 (1 - p)), s = 256 / K."""
    kthr = max(1, int(round(256.0 * (1.0 - float(p)))))
    return dropout_bytes(slot, q_rows, nk, seed, offset) < kthr, 256.0 / kthr


def mha_fwd(q, k, v, scale, causal=False, window=0, heads=None, dropout=None):
    """Dense multi-head forward in [B, N, H, d] layout.

    Returns O [B, Nq, H, dv] and LSE [B, H, Nq].  ``heads`` restricts the
    computation to a list of (b, h) pairs (others are left NaN), for large
    shapes where only sampled heads are checked.  ``dropout`` = (p, seed,
    offset): head slot b * H + h.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, nq, h_, _ = q.shape
    o = np.full((b_, nq, h_, v.shape[3]), np.nan)
    lse = np.full((b_, h_, nq), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(b_) for h in range(h_)]
    for b, h in pairs:
        drop = None if dropout is None else dropout_keep(b * h_ + h, range(nq), k.shape[1], dropout[1], dropout[2],
                                                         dropout[0])
        o[b, :, h], lse[b, h] = attention_fwd(q[b, :, h], k[b, :, h], v[b, :, h], scale, causal, window, drop=drop)
    return o, lse


def mha_bwd(q, k, v, dout, scale, causal=False, window=0, heads=None, dropout=None):
    """Dense multi-head backward in [B, N, H, d] layout -> (dq, dk, dv)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    b_, _, h_, _ = q.shape
    pairs = heads if heads is not None else [(b, h) for b in range(b_) for h in range(h_)]
    for b, h in pairs:
        drop = None if dropout is None else dropout_keep(b * h_ + h, range(q.shape[1]), k.shape[1], dropout[1],
                                                         dropout[2], dropout[0])
        dq[b, :, h], dk[b, :, h], dv[b, :, h] = attention_bwd(
            q[b, :, h], k[b, :, h], v[b, :, h], dout[b, :, h], scale, causal, window, drop=drop)
    return dq, dk, dv


def varlen_fwd(q, k, v, cu_seqlens, scale, causal=False, window=0, heads=None, seqs=None, dropout=None):
    """Packed sequences: q/k/v [total, H, d]; sequence s spans rows
    cu_seqlens[s]:cu_seqlens[s+1] and attends only within itself.

    Returns O [total, H, dv] and LSE [H, total].  ``heads`` / ``seqs`` restrict
    the work to sampled heads / sequences (others left NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    total, h_, _ = q.shape
    o = np.full((total, h_, v.shape[2]), np.nan)
    lse = np.full((h_, total), np.nan)
    hs = range(h_) if heads is None else heads
    ss = range(cu.size - 1) if seqs is None else seqs
    for s in ss:
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in hs:
            drop = None if dropout is None else dropout_keep(s * h_ + h, range(b - a), b - a, dropout[1], dropout[2],
                                                             dropout[0])
            o[a:b, h], lse[h, a:b] = attention_fwd(q[a:b, h], k[a:b, h], v[a:b, h], scale, causal, window, drop=drop)
    return o, lse


def varlen_bwd(q, k, v, dout, cu_seqlens, scale, causal=False, window=0, heads=None, seqs=None, dropout=None):
    """Gradients for packed sequences (the same layout as ``varlen_fwd``).

    Each sequence is an independent attention problem, so its gradients are
    the chain rule of ``attention_bwd`` applied within the sequence; rows of
    other sequences get exactly zero from it.  Returns dq, dk, dv
    [total, H, d]; ``heads`` / ``seqs`` restrict the work (others NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    total, h_, _ = q.shape
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    hs = range(h_) if heads is None else heads
    ss = range(cu.size - 1) if seqs is None else seqs
    for s in ss:
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in hs:
            drop = None if dropout is None else dropout_keep(s * h_ + h, range(b - a), b - a, dropout[1], dropout[2],
                                                             dropout[0])
            dq[a:b, h], dk[a:b, h], dv[a:b, h] = attention_bwd(q[a:b, h], k[a:b, h], v[a:b, h], dout[a:b, h],
                                                               scale, causal, window, drop=drop)
    return dq, dk, dv


def merge_partials(o_parts, lse_parts):
    """Combine P partial results: o_parts [P, ..., dv], lse_parts [P, ...].

    Part p is attention over its own key subset: O_p normalised over those
    keys, LSE_p = m_p + ln l_p (natural log).  Over the union of the subsets,
    LSE = ln sum_p exp(LSE_p) and O = sum_p exp(LSE_p - LSE) O_p, evaluated
    relative to the largest LSE_p so that no exponent overflows.  Parts with
    LSE_p = -inf saw no key and add nothing; if every part is -inf, O = 0 and
    LSE = -inf.  Returns (O [..., dv], LSE [...]).
    """
    o = np.asarray(o_parts, dtype=np.float64)
    lse = np.asarray(lse_parts, dtype=np.float64)
    m = lse.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse - m_safe[None])          # [P, ...]; 0 for -inf parts
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse_out = np.where(tot > 0, m_safe + np.log(tot), -np.inf)
        frac = np.where(tot[None] > 0, w / tot[None], 0.0)
    o_out = (frac[..., None] * np.where(frac[..., None] > 0, o, 0.0)).sum(axis=0)
    return o_out, lse_out


def kvcache_fwd(q, k_cache, v_cache, cache_seqlens, scale, causal=False, window=0, k_new=None, v_new=None):
    """Decode step against a KV cache, dense [B, N, H, d] layout.

    q [B, Nq, H, d]; k_cache, v_cache [B, Lmax, H, d]; cache_seqlens [B] ints.
    With k_new, v_new [B, Nq, H, d]: copies of the caches get them at rows
    cache_seqlens[b] .. cache_seqlens[b] + Nq - 1, and batch b attends over
    the first cache_seqlens[b] + Nq rows; without, over the first
    cache_seqlens[b].  Returns (O [B, Nq, H, dv], LSE [B, H, Nq], k_cache',
    v_cache').
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    b_, nq, h_, _ = q.shape
    lens = np.asarray(cache_seqlens, dtype=np.int64).reshape(-1)
    if k_new is not None:
        kn = np.asarray(k_new, dtype=np.float64)
        vn = np.asarray(v_new, dtype=np.float64)
        for b in range(b_):
            kc[b, lens[b]:lens[b] + nq] = kn[b]
            vc[b, lens[b]:lens[b] + nq] = vn[b]
    o = np.zeros((b_, nq, h_, vc.shape[3]))
    lse = np.zeros((b_, h_, nq))
    for b in range(b_):
        nk = int(lens[b]) + (nq if k_new is not None else 0)
        for h in range(h_):
            o[b, :, h], lse[b, h] = attention_fwd(q[b, :, h], kc[b, :nk, h], vc[b, :nk, h], scale, causal, window)
    return o, lse, kc, vc


def paged_gather(blocks, block_table, page):
    """Logical caches [B, max_blocks * page, H, d] from pages [num_blocks, page, H, d]:
    row j of entry b is blocks[block_table[b, j // page], j % page]."""
    blocks = np.asarray(blocks)
    table = np.asarray(block_table, dtype=np.int64)
    b_, mb = table.shape
    out = np.empty((b_, mb * page) + blocks.shape[2:], dtype=blocks.dtype)
    for b in range(b_):
        for j in range(mb * page):
            out[b, j] = blocks[table[b, j // page], j % page]
    return out


def kvcache_paged_fwd(q, k_blocks, v_blocks, block_table, page, cache_seqlens, scale, causal=False, window=0,
                      k_new=None, v_new=None):
    """kvcache_fwd on paged caches.  Returns (O, LSE, k_blocks', v_blocks'):
    the pages after the new rows were written to the rows they map to."""
    kc = paged_gather(np.asarray(k_blocks, dtype=np.float64), block_table, page)
    vc = paged_gather(np.asarray(v_blocks, dtype=np.float64), block_table, page)
    o, lse, kc2, vc2 = kvcache_fwd(q, kc, vc, cache_seqlens, scale, causal, window, k_new, v_new)
    kb = np.array(k_blocks, dtype=np.float64)
    vb = np.array(v_blocks, dtype=np.float64)
    if k_new is not None:
        table = np.asarray(block_table, dtype=np.int64)
        nq = np.asarray(q).shape[1]
        for b, t in enumerate(np.asarray(cache_seqlens, dtype=np.int64).reshape(-1)):
            for j in range(int(t), int(t) + nq):
                kb[table[b, j // page], j % page] = kc2[b, j]
                vb[table[b, j // page], j % page] = vc2[b, j]
    return o, lse, kb, vb


def e4m3_decode(codes):
    """OCP E4M3 byte codes -> fp64 values.

    Layout s.eeee.mmm, exponent bias 7.  e = 0: subnormal, (-1)^s 2^-6 (m/8).
    Otherwise (-1)^s 2^(e-7) (1 + m/8), except e = 15 and m = 7, which is NaN
    (the format has no infinities; max finite = 2^8 * 1.75 = 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    val = sign * val
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)


def fp8_dequant(codes, scale):
    """Value an fp8 tensor stands for: decoded code times its per-tensor scale."""
    return e4m3_decode(codes) * float(scale)
