// Internal declarations shared by the C-ABI layer (fa_api.cpp) and the
// kernel translation units.  Not part of the public interface (include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Kernel-side view of one forward call.  Dense and packed-varlen calls share
// it: for varlen, batch = number of sequences, the batch strides are 0 and
// each work-group reads its sequence's token offset from cu_seqlens.
struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *cu_seqlens;  // null for dense calls
  int64_t q_sb, q_st, q_sh;   // element strides: batch, token, head
  int64_t k_sb, k_st, k_sh;
  int64_t v_sb, v_st, v_sh;
  int64_t o_sb, o_st, o_sh;
  int64_t lse_sb, lse_sh;     // lse element strides: batch, head (token stride 1)
  int32_t batch, heads, nq, nk;  // varlen: nq = nk = max_seqlen (grid sizing only)
  int32_t nqt;                   // query tiles per (batch, head)
  int32_t br;                    // query rows per tile (fwd_block_rows)
  int32_t causal, window;
  float scale_log2;              // softmax_scale * log2(e) (* q, k descales for fp8)
  float v_descale;               // fp8 only, 1 otherwise
  // dropout (drop_k == 0: none): element kept iff its random byte < drop_k,
  // kept probabilities scaled by drop_scale = 256 / drop_k
  uint32_t drop_k, seed_lo, seed_hi, drop_offset;
  float drop_scale;
  // the running row max moves only when a tile's max exceeds it by more than
  // this (base-2 units); 0 keeps it exact
  float lazy;
  int32_t persist;               // persistent launch (set by the launcher): 1 dense schedule, 2 packed varlen schedule
};

// Kernel-side view of one backward call.  Packed varlen calls set
// cu_seqlens, zero batch strides, batch = number of sequences and
// nq = nk = max_seqlen (grid sizing only).
struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  const int32_t *cu_seqlens;  // null for dense calls
  float *dpsum;      // workspace: D_i = rowsum(dO * O), laid out like lse
  float *lse2;       // workspace: LSE_i * log2(e) (+inf for rows that see no key), laid out like lse
  int64_t lse_sb, lse_sh;  // lse / dpsum / lse2 element strides: batch, head (token stride 1)
  int64_t q_sb, q_st, q_sh, k_sb, k_st, k_sh, v_sb, v_st, v_sh, o_sb, o_st, o_sh;
  int64_t do_sb, do_st, do_sh, dq_sb, dq_st, dq_sh, dk_sb, dk_st, dk_sh, dv_sb, dv_st, dv_sh;
  int32_t batch, heads, nq, nk;
  int32_t causal, window, deterministic, grad_f32;
  float scale, scale_log2;
  uint32_t drop_k, seed_lo, seed_hi, drop_offset;  // dropout, as in FwdArgs
  float drop_scale;
  int32_t persist;   // dK/dV or dQ kernel: persistent launch over a static schedule (set by the launcher)
};

// Kernel-side view of one merge of partial results (O_p, LSE_p).
struct MergeArgs {
  const void *o_parts;     // [num_parts, batch, seqlen, heads, head_dim], fp32 or bf16
  const float *lse_parts;  // [num_parts, batch, heads, seqlen] fp32, parts lse_sp elements apart
  void *o;                 // [batch, seqlen, heads, head_dim], fp32 or bf16
  float *lse;              // [batch, heads, seqlen] fp32, or null
  int64_t p_sp, p_sb, p_st, p_sh;  // o_parts element strides: part, batch, token, head
  int64_t lse_sp;
  int64_t o_sb, o_st, o_sh;
  int32_t num_parts, batch, seqlen, heads;
  int32_t parts_f32, out_f32;
};

// Kernel-side view of one KV-cache decode call.
struct DecodeArgs {
  const void *q;                    // [batch, nq, heads, d] bf16
  void *k_cache, *v_cache;          // [batch, cache_len, heads, d] bf16
  const void *k_new, *v_new;        // [batch, nq, heads, d] bf16, or null
  const int32_t *cache_seqlens;     // [batch]
  void *o;                          // [batch, nq, heads, d] bf16 (num_splits == 1)
  float *lse;                       // [batch, heads, nq], or null (num_splits == 1)
  float *o_parts, *lse_parts;       // workspace (num_splits > 1): [splits, batch, nq, heads, d], [splits, batch, heads, nq]
  int64_t q_sb, q_st, q_sh, kc_sb, kc_st, kc_sh, vc_sb, vc_st, vc_sh;
  int64_t kn_sb, kn_st, kn_sh, vn_sb, vn_st, vn_sh, o_sb, o_st, o_sh;
  int32_t batch, nq, cache_len, heads;
  int32_t causal, window, num_splits, split_len;
  float scale_log2;
  const int32_t *block_table;       // paged caches: [batch, max_blocks] (else null; strides above are then
  int32_t page_shift, max_blocks;   // {block, token, head} of [num_blocks, 2^page_shift, heads, d])
};

// Launchers (defined in the kernel translation units).  Each returns the
// HIP status of its launch(es).
hipError_t launch_fwd_bf16(const FwdArgs &a, int head_dim, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs &a, int head_dim, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdArgs &a, int head_dim, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs &a, int head_dim, hipStream_t s);
size_t bwd_workspace_bytes(int batch, int heads, int nq, int head_dim, int deterministic);
// Device scratch that replaces the backward's workspace in fa_bwd_noalloc
// (one static copy per device); bwd_scratch() gives this device's address.
constexpr size_t kBwdScratchBytes = (size_t)8 << 20;
hipError_t bwd_scratch(void **ptr);
// Backward calls that run the exact fp32 kernels of a narrow causal window
// (every row sees at most 64 keys); their launches take one work-group per
// 32 query rows and per 32 keys of each (batch, head).
bool bwd_band(int causal, int window);
hipError_t launch_merge(const MergeArgs &a, int head_dim, hipStream_t s);
hipError_t launch_kv_append(const DecodeArgs &a, int head_dim, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int head_dim, hipStream_t s);

// Work-groups of a persistent launch on the current device: its CU count
// rounded down to a multiple of the 8 XCDs (0 if it cannot be read).
int persistent_groups();

// Query rows per work-group of the forward for a call (the tile table):
// bf16 calls take 256 rows (the ping-pong kernel) when that launch has at
// least one unit of work per CU (a causal dense unit is a pair of tiles),
// else 128 rows (4 waves) if that gives one work-group per CU, else 64 (2
// waves), so that short sequences still spread over the chip; packed calls
// count sequences x heads tiles of max_seqlen rows.  fp8 takes 256, fp32
// 16.  `cus` is the device's CU count (0: unknown).
int fwd_block_rows(int qkv_dtype, int head_dim, int64_t batch_heads, int64_t nq, bool causal, bool varlen,
                   int cus);
// Smallest tile a call may take (bounds of the host checks): 64 rows for
// bf16 and fp8 inputs, 16 for the fp32 kernel.
constexpr int kFwdMinBlockRows = 64;
constexpr int kFwdF32BlockRows = 16;
inline int fwd_min_block_rows(int qkv_dtype) { return qkv_dtype == 0 ? kFwdF32BlockRows : kFwdMinBlockRows; }

}  // namespace fa
