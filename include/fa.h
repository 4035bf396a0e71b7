/*
 * fa.h -- C ABI of the exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(softmax_scale * Q K^T + mask) V
 * by tiling Q, K and V through on-chip memory with an online (running max,
 * running sum) softmax, so the N x N score matrix never reaches HBM, and the
 * backward pass that recomputes the scores from the saved log-sum-exp.
 *
 * Where each operation is defined:
 *   - the attention formula: top of "Flash-Attention 2/3在ms-swift中的集成与性能提升"
 *     (bxzpzcl.cn); section 一 of the adg.csdn.net flash_attn/Qwen page;
 *     section 2.1 of "FlashAttention优化Transformer显存与计算效率" (jsqmd.com);
 *   - tiling, blockwise softmax and fusion: jsqmd.com sections 2.2.1-2.2.3;
 *     section 三 of the adg.csdn.net page;
 *   - recomputation in the backward: the three techniques listed in the
 *     ms-swift integration page; section 三 (step 5) of the adg.csdn.net page;
 *   - causal and sliding-window masks, FP8 operands: the FA-3 paragraph of the
 *     ms-swift integration page; causal=True in every API example of
 *     "突破AI算力瓶颈：FlashAttention与MindSpore 2.0全场景融合方案" (核心API与使用示例);
 *   - packed variable-length sequences: flash_attn_varlen_func and --packing
 *     in "ms-swift长文本训练优化，Flash-Attention显存省一半" sections 4.3 and 5.1;
 *   - the [batch, seqlen, nheads, headdim] layout and packed QKV
 *     (batch, seqlen, 3, nheads, headdim): the MindSpore page, 核心API与使用示例;
 *   - the precision recipe (bf16 operands, fp32 softmax accumulation, convert
 *     at output): jsqmd.com section 3.2;
 *   - error conventions (mixed dtypes -> "same dtype" error, missing GPU build
 *     -> runtime error): ms-swift long-text page section 4.3.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; every call only enqueues kernels
 *     on `stream` (a hipStream_t; NULL = the default stream) and returns.
 *   - Strides are in ELEMENTS; the last (head_dim) dimension must be
 *     contiguous (stride 1) and every row must start 16-byte aligned.
 *   - head_dim must be 64 or 128.  softmax_scale is applied as given and
 *     must be finite and >= 0 (callers pass 1/sqrt(head_dim) for the usual
 *     default; 0 gives every visible key the same weight, so O is the mean of
 *     V over the visible keys and LSE = ln(number of visible keys)).
 *   - causal: key j is visible to query i iff j <= i + (Nk - Nq)
 *     (bottom-right alignment; for Nq == Nk this is j <= i).
 *   - window W > 0: additionally j > i + (Nk - Nq) - W, i.e. each query sees
 *     at most W keys ending at its own position; W = 0 means unlimited.
 *   - A query row that sees no key gets O = 0 and LSE = -inf.
 *   - LSE is the natural-log log-sum-exp of the scaled, masked scores, fp32.
 *   - Dropout (dropout_p > 0; bf16 only): the attention probabilities are
 *     dropped after the softmax (LSE is of the undropped softmax), as the
 *     dropout_p argument of every API example of the MindSpore page and the
 *     fused softmax/mask/dropout of the ms-swift integration page describe.
 *     Element (query row i, key j) of head slot b * heads + h (b: batch entry
 *     or packed sequence; i, j counted within it) draws byte (j & 3) of word
 *     ((j & 31) >> 3) of Philox4x32-10 (Salmon et al., "Parallel random
 *     numbers: as easy as 1, 2, 3", SC 2011) with counter (2 (j >> 5) +
 *     ((j >> 2) & 1), i, slot, dropout_offset) and key (dropout_seed mod
 *     2^32, dropout_seed >> 32).  It is kept iff that byte < K =
 *     round(256 (1 - dropout_p)) (at least 1), and kept values are scaled by
 *     256 / K, so dropout_p is in effect rounded to a multiple of 1/256
 *     (below 1/512 it is no dropout).  The backward regenerates the same
 *     mask from the same (seed, offset).
 *   - Errors: a non-FA_OK status is returned and fa_last_error() describes it.
 *     FA_ERR_INVALID_ARGUMENT and FA_ERR_DTYPE_MISMATCH are detected on the
 *     host before anything is launched; kernel faults surface at the caller's
 *     next synchronisation.
 *   - Calls on different streams may run concurrently; the library keeps no
 *     state between calls other than the thread-local error message and a
 *     per-device architecture check.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 7

typedef enum {
  FA_F32 = 0,       /* IEEE binary32 */
  FA_BF16 = 1,      /* bfloat16 */
  FA_FP8_E4M3 = 2   /* OCP FP8 E4M3 (max finite 448, no infinities) */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size/stride/flag/scale */
  FA_ERR_DTYPE_MISMATCH = 2,   /* q/k/v (and o) dtypes are not an allowed combination */
  FA_ERR_UNSUPPORTED = 3,      /* head_dim not 64/128, device not gfx950, fp8 backward */
  FA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} fa_status;

/* Dense forward.
 *   q [batch, seqlen_q, heads, head_dim]; k, v [batch, seqlen_k, heads, head_dim];
 *   o [batch, seqlen_q, heads, head_dim]; lse [batch, heads, seqlen_q] fp32,
 *   contiguous, or NULL when the caller does not need it.
 *   x_stride = {batch, token, head} element strides of each tensor.
 *   Allowed dtypes (qkv_dtype, o_dtype): (F32, F32), (BF16, BF16),
 *   (FP8_E4M3, BF16).  For fp8 the values are code * descale (per tensor);
 *   for the other dtypes the descales must be 1.
 *   Packed QKV (batch, seqlen, 3, heads, head_dim) is expressed by pointing
 *   q, k, v at slices 0, 1, 2 of one buffer with token stride 3*heads*head_dim.
 *   The kernels read rows with 32-bit byte offsets from the start of each
 *   (batch, head) slice: (seqlen + 256) * token stride * element size must
 *   be below 2^31 for every tensor, else FA_ERR_INVALID_ARGUMENT. */
typedef struct {
  const void *q, *k, *v;
  void *o;
  float *lse;
  fa_dtype qkv_dtype, o_dtype;
  int32_t batch, seqlen_q, seqlen_k, heads, head_dim;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  float softmax_scale;
  int32_t causal;  /* 0 or 1 */
  int32_t window;  /* 0 = unlimited, W > 0 = sliding window of W keys */
  float q_descale, k_descale, v_descale;
  float dropout_p;          /* 0 <= p < 1; 0 = no dropout */
  uint32_t dropout_offset;  /* Philox counter word 3 */
  uint64_t dropout_seed;    /* Philox key */
} fa_fwd_params;

/* Packed variable-length forward (self-attention within each sequence).
 *   q, k, v, o [total_tokens, heads, head_dim]; x_stride = {token, head}.
 *   Sequence s occupies tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 and attends
 *   only to itself (its own positions start at 0 for the masks).
 *   cu_seqlens: DEVICE int32 [num_seqs + 1], cu_seqlens[0] = 0,
 *   non-decreasing, cu_seqlens[num_seqs] = total_tokens.  Every length must be
 *   <= max_seqlen, which sizes the launch grid.  These device-side contracts
 *   are not checked: violating them reads or writes out of bounds.  Rows are
 *   addressed from each sequence's own start, so the 2^31-byte bound of
 *   fa_fwd applies with max_seqlen in place of seqlen, whatever total_tokens.
 *   lse [heads, total_tokens] fp32 contiguous, or NULL. */
typedef struct {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *cu_seqlens;
  fa_dtype qkv_dtype, o_dtype;
  int32_t num_seqs, total_tokens, max_seqlen, heads, head_dim;
  int64_t q_stride[2], k_stride[2], v_stride[2], o_stride[2];
  float softmax_scale;
  int32_t causal, window;
  float q_descale, k_descale, v_descale;
  float dropout_p;
  uint32_t dropout_offset;
  uint64_t dropout_seed;
} fa_varlen_fwd_params;

/* Dense backward (recomputation from the saved LSE).
 *   q, k, v, o, dout: as in the forward (qkv_dtype BF16: all five bf16);
 *   lse [batch, heads, seqlen_q] fp32 from the forward of the same inputs.
 *   dq [batch, seqlen_q, heads, head_dim], dk, dv [batch, seqlen_k, heads,
 *   head_dim] in grad_dtype (FA_F32, the default of the Python layer, or
 *   FA_BF16).  deterministic (0 or 1, the pages' deterministic= argument):
 *   both settings run the same atomic-free kernels -- dQ has a kernel of its
 *   own rather than a cross-work-group reduction -- so repeated calls always
 *   give bitwise identical gradients.
 *   workspace: device memory of fa_bwd_workspace_bytes(p) bytes, 256-byte
 *   aligned, owned by the caller; its contents on entry are ignored. */
typedef struct {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  fa_dtype qkv_dtype, grad_dtype;
  int32_t batch, seqlen_q, seqlen_k, heads, head_dim;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3], do_stride[3];
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  float softmax_scale;
  int32_t causal, window, deterministic;
  float dropout_p;          /* the forward's dropout: same p, seed, offset */
  uint32_t dropout_offset;
  uint64_t dropout_seed;
} fa_bwd_params;

/* Packed variable-length backward: the gradients of fa_varlen_fwd, by the
 * same recomputation as fa_bwd (packed sequences: ms-swift long-text page
 * sections 4.3 and 5.1; recomputation: ms-swift integration page).
 *   q, k, v, o, dout [total_tokens, heads, head_dim] bf16; x_stride = {token, head}.
 *   lse [heads, total_tokens] fp32 contiguous, as written by fa_varlen_fwd.
 *   dq, dk, dv [total_tokens, heads, head_dim] in grad_dtype (FA_F32 or FA_BF16).
 *   cu_seqlens, max_seqlen: as in fa_varlen_fwd, with the same unchecked
 *   device-side contracts.  Every token of every sequence gets its dq, dk,
 *   dv written (zero for a token that neither sees nor is seen by any other).
 *   deterministic: as in fa_bwd (no atomics either way; repeated calls are
 *   bitwise identical).
 *   workspace: fa_varlen_bwd_workspace_bytes(p) bytes of device memory,
 *   256-byte aligned, owned by the caller; contents on entry are ignored. */
typedef struct {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  const int32_t *cu_seqlens;
  fa_dtype qkv_dtype, grad_dtype;
  int32_t num_seqs, total_tokens, max_seqlen, heads, head_dim;
  int64_t q_stride[2], k_stride[2], v_stride[2], o_stride[2], do_stride[2];
  int64_t dq_stride[2], dk_stride[2], dv_stride[2];
  float softmax_scale;
  int32_t causal, window, deterministic;
  float dropout_p;
  uint32_t dropout_offset;
  uint64_t dropout_seed;
} fa_varlen_bwd_params;

/* Merge of partial results: attention over disjoint key subsets p, each
 * normalised over its own keys, combined into the result over their union,
 *     LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p
 * (the stable combination of per-block max and exponent sum of jsqmd.com
 * section 2.2.2; the step that joins the per-segment results of ring
 * attention, Ring-Attention paragraph of the ms-swift integration page).
 *   o_parts [num_parts, batch, seqlen, heads, head_dim] in parts_dtype (FA_F32
 *   or FA_BF16); parts_stride = {part, batch, token, head} element strides.
 *   lse_parts [num_parts, batch, heads, seqlen] fp32 contiguous (natural log).
 *   o [batch, seqlen, heads, head_dim] in o_dtype (FA_F32 or FA_BF16),
 *   o_stride = {batch, token, head}; lse [batch, heads, seqlen] fp32
 *   contiguous, or NULL.
 * A part with LSE_p = -inf (it saw no key) adds nothing and its O_p row is
 * not read; a row where every part is -inf (or num_parts = 0) gets O = 0 and
 * LSE = -inf.  o must not overlap o_parts. */
typedef struct {
  const void *o_parts;
  const float *lse_parts;
  void *o;
  float *lse;
  fa_dtype parts_dtype, o_dtype;
  int32_t num_parts, batch, seqlen, heads, head_dim;
  int64_t parts_stride[4], o_stride[3];
} fa_merge_params;

/* KV-cache decode step (flash_attn_with_kvcache of the MindSpore page,
 * 推理优化与KV缓存): optional new rows k_new, v_new are first written into the
 * caches at rows cache_seqlens[b] .. cache_seqlens[b] + seqlen_q - 1; then
 * the seqlen_q query rows of batch entry b, taken as the last seqlen_q
 * positions, attend over cache rows 0 .. L_b - 1 with
 * L_b = cache_seqlens[b] + (k_new ? seqlen_q : 0), with the causal /
 * window rules of every other entry point (bottom-right aligned).
 *   q [batch, seqlen_q, heads, head_dim] bf16, 1 <= seqlen_q <= 8 (0: no-op).
 *   k_cache, v_cache [batch, cache_len, heads, head_dim] bf16, written only
 *   at the appended rows.  k_new, v_new [batch, seqlen_q, heads, head_dim]
 *   bf16, both or neither.
 *   cache_seqlens: DEVICE int32 [batch]; unchecked contract:
 *   0 <= cache_seqlens[b] and L_b <= cache_len.
 *   o [batch, seqlen_q, heads, head_dim] bf16; lse [batch, heads, seqlen_q]
 *   fp32 contiguous, or NULL.  A query row that sees no key gets O = 0 and
 *   LSE = -inf.
 *   num_splits: key ranges per (batch, head) processed by separate
 *   work-groups and merged as fa_merge does; 0 lets the library choose from
 *   batch * heads and cache_len.  It fixes the workspace size.
 *   workspace: fa_kvcache_workspace_bytes(p) bytes of device memory,
 *   256-byte aligned (0 bytes when one split is used). */
typedef struct {
  const void *q;
  void *k_cache, *v_cache;
  const void *k_new, *v_new;
  const int32_t *cache_seqlens;
  void *o;
  float *lse;
  fa_dtype qkv_dtype;
  int32_t batch, seqlen_q, cache_len, heads, head_dim;
  int64_t q_stride[3], kc_stride[3], vc_stride[3], kn_stride[3], vn_stride[3], o_stride[3];
  float softmax_scale;
  int32_t causal, window, num_splits;
  /* Paged caches (the paged storage of the same section), or NULL: then
   * k_cache, v_cache are [num_blocks, page_block_size, heads, head_dim] with
   * kc_stride / vc_stride = {block, token, head}, and logical row j of batch
   * entry b is row j % page_block_size of block block_table[b][j /
   * page_block_size].  block_table: DEVICE int32 [batch, max_blocks_per_seq],
   * row-major.  page_block_size is a power of two; cache_len (the logical
   * capacity) must be <= max_blocks_per_seq * page_block_size.  Unchecked
   * contract: every entry for a row below L_b names an existing block, and no
   * two appended rows map to the same physical row. */
  const int32_t *block_table;
  int32_t page_block_size, max_blocks_per_seq;
} fa_kvcache_params;

/* Host-only validation: never touches a device.  Returns the status the
 * corresponding entry point would return before launching anything. */
fa_status fa_check_fwd(const fa_fwd_params *p);
fa_status fa_check_varlen_fwd(const fa_varlen_fwd_params *p);
fa_status fa_check_bwd(const fa_bwd_params *p);
fa_status fa_check_varlen_bwd(const fa_varlen_bwd_params *p);
fa_status fa_check_merge(const fa_merge_params *p);
fa_status fa_check_kvcache(const fa_kvcache_params *p);

/* Enqueue the forward: writes o (and lse when non-NULL). */
fa_status fa_fwd(const fa_fwd_params *p, void *stream);

/* Enqueue the packed variable-length forward. */
fa_status fa_varlen_fwd(const fa_varlen_fwd_params *p, void *stream);

/* Bytes of device workspace fa_bwd needs for these parameters (0 on invalid
 * parameters; see fa_last_error). */
size_t fa_bwd_workspace_bytes(const fa_bwd_params *p);

/* Enqueue the backward: writes dq, dk, dv. */
fa_status fa_bwd(const fa_bwd_params *p, void *workspace, size_t workspace_bytes, void *stream);

/* fa_bwd without any allocation, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels and results as fa_bwd, with the
 * workspace taken from a static device array of FA_BWD_SCRATCH_BYTES that
 * the library holds on each device it runs on until the process ends.  The
 * caller passes every input and output as for fa_bwd.  Calls that need more
 * than FA_BWD_SCRATCH_BYTES (8 bytes per row of batch x heads x seqlen_q,
 * i.e. more than 2^20 such rows) return FA_ERR_INVALID_ARGUMENT before
 * anything is launched.  Nothing in the array has to start at any value
 * (every call writes what it reads), but all calls on one device share it:
 * calls that overlap in time on one device (different streams) race. */
#define FA_BWD_SCRATCH_BYTES ((size_t)8 << 20)
fa_status fa_bwd_noalloc(const fa_bwd_params *p, void *stream);

/* Bytes of device workspace fa_varlen_bwd needs (0 on invalid parameters). */
size_t fa_varlen_bwd_workspace_bytes(const fa_varlen_bwd_params *p);

/* Enqueue the packed variable-length backward: writes dq, dk, dv. */
fa_status fa_varlen_bwd(const fa_varlen_bwd_params *p, void *workspace, size_t workspace_bytes, void *stream);

/* Enqueue the merge: writes o (and lse when non-NULL). */
fa_status fa_merge(const fa_merge_params *p, void *stream);

/* Bytes of device workspace fa_fwd_kvcache needs (0 on invalid parameters
 * and when one split is used). */
size_t fa_kvcache_workspace_bytes(const fa_kvcache_params *p);

/* Enqueue the KV-cache decode step: appends k_new, v_new (if given), writes o
 * (and lse when non-NULL). */
fa_status fa_fwd_kvcache(const fa_kvcache_params *p, void *workspace, size_t workspace_bytes, void *stream);

/* Thread-local description of the last non-FA_OK status ("" if none). */
const char *fa_last_error(void);

/* FA_ABI_VERSION of the loaded library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
