// C ABI of the exact-attention library (declared in include/fa.h).
//
// Host side only: argument validation that never touches a device, the
// per-device architecture check, translation of the public parameter structs
// into the kernels' argument structs, and launches on the caller's stream.
// Error classes mirror the pages' conventions (ms-swift long-text page,
// section 4.3): mixed dtypes are a "same dtype" error, a missing or
// unsupported GPU build is a runtime error.

#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "fa_internal.h"
#include "fa_split.h"

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fa_status ok() {
  g_last_error.clear();
  return FA_OK;
}

constexpr float kLog2e = 1.4426950408889634f;

// The kernels' exponent factor scale * log2(e) (* fp8 descales).  At scale 0
// it is the smallest normal float instead: every finite score then still
// gives 2^(s c - m) = 1 exactly in fp32 (|s c| < 2^-100), as scale 0 does,
// while masked scores (-inf) stay -inf rather than becoming -inf * 0 = NaN.
float exp2_factor(float scale, float descale) {
  const float c = scale * kLog2e * descale;
  return c > 0.f ? c : FLT_MIN;
}

bool valid_dtype(int d) { return d == FA_F32 || d == FA_BF16 || d == FA_FP8_E4M3; }

int dtype_bytes(fa_dtype d) { return d == FA_F32 ? 4 : d == FA_BF16 ? 2 : 1; }

// Common checks of the forward parameters shared by the dense and varlen
// entry points.
fa_status check_fwd_common(fa_dtype qkv, fa_dtype o, int32_t heads, int32_t head_dim,
                           float scale, int32_t causal, int32_t window, float qd, float kd,
                           float vd) {
  if (!valid_dtype(qkv) || !valid_dtype(o))
    return fail(FA_ERR_INVALID_ARGUMENT, "unknown dtype code (qkv_dtype=%d, o_dtype=%d)", (int)qkv, (int)o);
  const bool combo = (qkv == FA_F32 && o == FA_F32) || (qkv == FA_BF16 && o == FA_BF16) ||
                     (qkv == FA_FP8_E4M3 && o == FA_BF16);
  if (!combo)
    return fail(FA_ERR_DTYPE_MISMATCH,
                "Input and output tensors must have the same dtype (fp8 inputs give bf16 output); "
                "got qkv_dtype=%d o_dtype=%d", (int)qkv, (int)o);
  if (heads < 0) return fail(FA_ERR_INVALID_ARGUMENT, "heads must be >= 0 (got %d)", heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  // applied as given; 0 gives every visible key the same weight.  The kernels
  // take the row max of the unscaled scores, so a negative scale is refused.
  if (!(std::isfinite(scale) && scale >= 0.f))
    return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0 (got %g)", (double)scale);
  if (causal != 0 && causal != 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  if (window < 0) return fail(FA_ERR_INVALID_ARGUMENT, "window must be >= 0 (got %d)", window);
  if (qkv == FA_FP8_E4M3) {
    if (!(std::isfinite(qd) && qd > 0.f && std::isfinite(kd) && kd > 0.f && std::isfinite(vd) && vd > 0.f))
      return fail(FA_ERR_INVALID_ARGUMENT, "fp8 descales must be finite and > 0 (got %g, %g, %g)",
                  (double)qd, (double)kd, (double)vd);
  } else if (qd != 1.f || kd != 1.f || vd != 1.f) {
    return fail(FA_ERR_INVALID_ARGUMENT, "descales must be 1 for non-fp8 inputs (got %g, %g, %g)",
                (double)qd, (double)kd, (double)vd);
  }
  return FA_OK;
}

// Row alignment: every row the kernels load with 16-byte accesses must start
// 16-byte aligned, i.e. pointer and all token/head/batch strides.
fa_status check_tensor(const char *name, const void *ptr, const int64_t *stride, int nstride,
                       int elem_bytes, bool empty, int64_t rows = 0, int head_dim = 0) {
  if (empty) return FA_OK;
  if (!ptr) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  for (int i = 0; i < nstride; ++i)
    if (stride[i] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "%s stride[%d] must be >= 0 (got %lld)",
                                   name, i, (long long)stride[i]);
  // rows are addressed with 32-bit byte offsets from the start of each
  // (batch, head) slice, and rows past the end read as zeros only if rows do
  // not overlap: token stride >= head_dim whenever there is more than one row
  const int64_t tok = stride[nstride == 3 ? 1 : 0];
  if (rows > 1 && tok < head_dim)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s token stride (%lld) must be >= head_dim (%d)", name,
                (long long)tok, head_dim);
  if ((rows + 256) * tok * elem_bytes >= (int64_t)1 << 31)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: one (batch, head) slice spans more than 2 GiB", name);
  const int64_t a = 16 / elem_bytes;
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  for (int i = 0; i < nstride; ++i)
    if (stride[i] % a)
      return fail(FA_ERR_INVALID_ARGUMENT, "%s stride[%d] must be a multiple of %lld elements (got %lld)",
                  name, i, (long long)a, (long long)stride[i]);
  return FA_OK;
}

// Per-device architecture check, cached.
std::mutex g_arch_mu;
int g_arch_ok[64];  // 0 unknown, 1 gfx950, -1 other

fa_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(FA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    g_arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (g_arch_ok[dev] < 0)
      return fail(FA_ERR_UNSUPPORTED, "this library is built for gfx950 only (device %d is %s)", dev,
                  prop.gcnArchName);
  }
  if (g_arch_ok[dev] < 0) return fail(FA_ERR_UNSUPPORTED, "this library is built for gfx950 only");
  return FA_OK;
}

fa_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Dropout: validate p for the dtype and fill the kernel-side fields.
fa_status check_dropout(float p, fa_dtype qkv) {
  if (!(std::isfinite(p) && p >= 0.f && p < 1.f))
    return fail(FA_ERR_INVALID_ARGUMENT, "dropout_p must be in [0, 1) (got %g)", (double)p);
  if (p > 0.f && qkv != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dropout is available for bf16 inputs only (got qkv_dtype=%d)", (int)qkv);
  return FA_OK;
}

// Lazy running max of the forward kernels: 8 (log2 units), or exact where
// every row sees at most 64 keys (causal mask with a window of at most 64):
// the weights of such rows can sit on a few keys, whose unnormalised
// probabilities are then kept at 1 rather than rounded from up to 2^8.
float lazy_threshold(int causal, int window) { return causal && window > 0 && window <= 64 ? 0.f : 8.f; }

template <class Args>
void set_dropout(Args &a, float p, uint64_t seed, uint32_t offset) {
  const long kthr = std::max(1L, std::lround(256.0 * (1.0 - (double)p)));
  a.drop_k = kthr >= 256 ? 0u : (uint32_t)kthr;  // p < 1/512: nothing is dropped
  a.drop_scale = a.drop_k ? 256.f / (float)a.drop_k : 1.f;
  a.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  a.seed_hi = (uint32_t)(seed >> 32);
  a.drop_offset = offset;
}

// Checks shared by the dense and packed backward.
fa_status check_bwd_common(fa_dtype qkv, fa_dtype grad, int heads, int head_dim, float scale, int causal,
                           int window, int deterministic) {
  if (!valid_dtype(qkv) || !valid_dtype(grad))
    return fail(FA_ERR_INVALID_ARGUMENT, "unknown dtype code (qkv_dtype=%d, grad_dtype=%d)", (int)qkv, (int)grad);
  if (qkv == FA_FP8_E4M3) return fail(FA_ERR_UNSUPPORTED, "the backward pass is not available for fp8 inputs");
  if (qkv != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "the backward pass takes bf16 q/k/v/o/dout (got qkv_dtype=%d)", (int)qkv);
  if (grad != FA_F32 && grad != FA_BF16)
    return fail(FA_ERR_DTYPE_MISMATCH, "gradients must be fp32 or bf16 (got grad_dtype=%d)", (int)grad);
  if (heads < 0) return fail(FA_ERR_INVALID_ARGUMENT, "heads must be >= 0 (got %d)", heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  // applied as given; 0 gives every visible key the same weight.  The kernels
  // take the row max of the unscaled scores, so a negative scale is refused.
  if (!(std::isfinite(scale) && scale >= 0.f))
    return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0 (got %g)", (double)scale);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  if (window < 0) return fail(FA_ERR_INVALID_ARGUMENT, "window must be >= 0 (got %d)", window);
  if (deterministic != 0 && deterministic != 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "deterministic must be 0 or 1 (got %d)", deterministic);
  return FA_OK;
}

// Key splits per (batch, head) of a KV-cache decode: enough work-groups for
// two per CU, but no split shorter than 512 keys.
int kvcache_splits(const fa_kvcache_params *p) {
  if (p->num_splits > 0) return p->num_splits;
  const int64_t bh = std::max<int64_t>(1, (int64_t)p->batch * p->heads);
  const int64_t want = (512 + bh - 1) / bh;
  const int64_t cap = std::max<int64_t>(1, ((int64_t)p->cache_len + 511) / 512);
  return (int)std::max<int64_t>(1, std::min<int64_t>(std::min(want, cap), 64));
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

size_t kvcache_ws(const fa_kvcache_params *p, int splits) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)splits * p->batch * p->seqlen_q * p->heads;
  return round256(rows * p->head_dim * sizeof(float)) + round256(rows * sizeof(float));
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char *fa_last_error(void) { return g_last_error.c_str(); }

fa_status fa_check_fwd(const fa_fwd_params *p) {
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "params is NULL");
  fa_status st = check_fwd_common(p->qkv_dtype, p->o_dtype, p->heads, p->head_dim, p->softmax_scale,
                                  p->causal, p->window, p->q_descale, p->k_descale, p->v_descale);
  if (st != FA_OK) return st;
  if ((st = check_dropout(p->dropout_p, p->qkv_dtype)) != FA_OK) return st;
  if (p->batch < 0 || p->seqlen_q < 0 || p->seqlen_k < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 0 (batch=%d seqlen_q=%d seqlen_k=%d)", p->batch,
                p->seqlen_q, p->seqlen_k);
  const bool q_empty = (int64_t)p->batch * p->seqlen_q * p->heads == 0;
  const bool k_empty = (int64_t)p->batch * p->seqlen_k * p->heads == 0;
  const int eb = dtype_bytes(p->qkv_dtype), ob = dtype_bytes(p->o_dtype);
  const int hd = p->head_dim;
  if ((st = check_tensor("q", p->q, p->q_stride, 3, eb, q_empty, p->seqlen_q, hd)) != FA_OK) return st;
  if ((st = check_tensor("k", p->k, p->k_stride, 3, eb, k_empty, p->seqlen_k, hd)) != FA_OK) return st;
  if ((st = check_tensor("v", p->v, p->v_stride, 3, eb, k_empty, p->seqlen_k, hd)) != FA_OK) return st;
  if ((st = check_tensor("o", p->o, p->o_stride, 3, ob, q_empty, p->seqlen_q, hd)) != FA_OK) return st;
  const int64_t items = ceil_div(p->seqlen_q, fa::fwd_min_block_rows(p->qkv_dtype)) * (int64_t)p->heads * p->batch;
  if (items > INT32_MAX) return fail(FA_ERR_INVALID_ARGUMENT, "problem too large for one launch");
  return ok();
}

fa_status fa_check_varlen_fwd(const fa_varlen_fwd_params *p) {
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "params is NULL");
  fa_status st = check_fwd_common(p->qkv_dtype, p->o_dtype, p->heads, p->head_dim, p->softmax_scale,
                                  p->causal, p->window, p->q_descale, p->k_descale, p->v_descale);
  if (st != FA_OK) return st;
  if ((st = check_dropout(p->dropout_p, p->qkv_dtype)) != FA_OK) return st;
  if (p->num_seqs < 0 || p->total_tokens < 0 || p->max_seqlen < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 0 (num_seqs=%d total_tokens=%d max_seqlen=%d)",
                p->num_seqs, p->total_tokens, p->max_seqlen);
  if (p->max_seqlen > p->total_tokens)
    return fail(FA_ERR_INVALID_ARGUMENT, "max_seqlen (%d) exceeds total_tokens (%d)", p->max_seqlen,
                p->total_tokens);
  const bool empty = (int64_t)p->total_tokens * p->heads == 0 || p->num_seqs == 0;
  if (!empty && !p->cu_seqlens) return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  const int eb = dtype_bytes(p->qkv_dtype), ob = dtype_bytes(p->o_dtype);
  // the kernels address each sequence's rows from its own start (64-bit
  // pointer arithmetic), so the 32-bit offset bound applies per sequence
  const int hd = p->head_dim, ms = p->max_seqlen;
  if ((st = check_tensor("q", p->q, p->q_stride, 2, eb, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("k", p->k, p->k_stride, 2, eb, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("v", p->v, p->v_stride, 2, eb, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("o", p->o, p->o_stride, 2, ob, empty, ms, hd)) != FA_OK) return st;
  const int64_t items =
      ceil_div(p->max_seqlen, fa::fwd_min_block_rows(p->qkv_dtype)) * (int64_t)p->heads * p->num_seqs;
  if (items > INT32_MAX) return fail(FA_ERR_INVALID_ARGUMENT, "problem too large for one launch");
  return ok();
}

fa_status fa_check_bwd(const fa_bwd_params *p) {
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "params is NULL");
  fa_status st0 = check_bwd_common(p->qkv_dtype, p->grad_dtype, p->heads, p->head_dim, p->softmax_scale,
                                   p->causal, p->window, p->deterministic);
  if (st0 != FA_OK) return st0;
  if ((st0 = check_dropout(p->dropout_p, p->qkv_dtype)) != FA_OK) return st0;
  if (p->batch < 0 || p->seqlen_q < 0 || p->seqlen_k < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 0 (batch=%d seqlen_q=%d seqlen_k=%d heads=%d)",
                p->batch, p->seqlen_q, p->seqlen_k, p->heads);
  const bool q_empty = (int64_t)p->batch * p->seqlen_q * p->heads == 0;
  const bool k_empty = (int64_t)p->batch * p->seqlen_k * p->heads == 0;
  const int gb = dtype_bytes(p->grad_dtype);
  fa_status st;
  const int hd = p->head_dim, nq = p->seqlen_q, nk = p->seqlen_k;
  if ((st = check_tensor("q", p->q, p->q_stride, 3, 2, q_empty, nq, hd)) != FA_OK) return st;
  if ((st = check_tensor("k", p->k, p->k_stride, 3, 2, k_empty, nk, hd)) != FA_OK) return st;
  if ((st = check_tensor("v", p->v, p->v_stride, 3, 2, k_empty, nk, hd)) != FA_OK) return st;
  if ((st = check_tensor("o", p->o, p->o_stride, 3, 2, q_empty, nq, hd)) != FA_OK) return st;
  if ((st = check_tensor("dout", p->dout, p->do_stride, 3, 2, q_empty, nq, hd)) != FA_OK) return st;
  if ((st = check_tensor("dq", p->dq, p->dq_stride, 3, gb, q_empty, nq, hd)) != FA_OK) return st;
  if ((st = check_tensor("dk", p->dk, p->dk_stride, 3, gb, k_empty, nk, hd)) != FA_OK) return st;
  if ((st = check_tensor("dv", p->dv, p->dv_stride, 3, gb, k_empty, nk, hd)) != FA_OK) return st;
  if (!q_empty && !p->lse) return fail(FA_ERR_INVALID_ARGUMENT, "lse is NULL");
  if (ceil_div(std::max(nq, nk), 128) * (int64_t)p->heads * p->batch > INT32_MAX ||
      (fa::bwd_band(p->causal, p->window) &&
       ceil_div(std::max(nq, nk), 32) * (int64_t)p->heads * p->batch * 256 > (int64_t)UINT32_MAX))
    return fail(FA_ERR_INVALID_ARGUMENT, "problem too large for one launch");
  return ok();
}

fa_status fa_check_varlen_bwd(const fa_varlen_bwd_params *p) {
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "params is NULL");
  fa_status st = check_bwd_common(p->qkv_dtype, p->grad_dtype, p->heads, p->head_dim, p->softmax_scale,
                                  p->causal, p->window, p->deterministic);
  if (st != FA_OK) return st;
  if ((st = check_dropout(p->dropout_p, p->qkv_dtype)) != FA_OK) return st;
  if (p->num_seqs < 0 || p->total_tokens < 0 || p->max_seqlen < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 0 (num_seqs=%d total_tokens=%d max_seqlen=%d)",
                p->num_seqs, p->total_tokens, p->max_seqlen);
  if (p->max_seqlen > p->total_tokens)
    return fail(FA_ERR_INVALID_ARGUMENT, "max_seqlen (%d) exceeds total_tokens (%d)", p->max_seqlen,
                p->total_tokens);
  const bool empty = (int64_t)p->total_tokens * p->heads == 0 || p->num_seqs == 0;
  if (!empty && !p->cu_seqlens) return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  const int gb = dtype_bytes(p->grad_dtype);
  // per-sequence 32-bit offsets, as in the packed forward
  const int hd = p->head_dim, ms = p->max_seqlen;
  if ((st = check_tensor("q", p->q, p->q_stride, 2, 2, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("k", p->k, p->k_stride, 2, 2, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("v", p->v, p->v_stride, 2, 2, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("o", p->o, p->o_stride, 2, 2, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("dout", p->dout, p->do_stride, 2, 2, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("dq", p->dq, p->dq_stride, 2, gb, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("dk", p->dk, p->dk_stride, 2, gb, empty, ms, hd)) != FA_OK) return st;
  if ((st = check_tensor("dv", p->dv, p->dv_stride, 2, gb, empty, ms, hd)) != FA_OK) return st;
  if (!empty && !p->lse) return fail(FA_ERR_INVALID_ARGUMENT, "lse is NULL");
  if (ceil_div(p->max_seqlen, 128) * (int64_t)p->heads * p->num_seqs > INT32_MAX ||
      (fa::bwd_band(p->causal, p->window) &&
       ceil_div(p->max_seqlen, 32) * (int64_t)p->heads * p->num_seqs * 256 > (int64_t)UINT32_MAX))
    return fail(FA_ERR_INVALID_ARGUMENT, "problem too large for one launch");
  return ok();
}

fa_status fa_fwd(const fa_fwd_params *p, void *stream) {
  fa_status st = fa_check_fwd(p);
  if (st != FA_OK) return st;
  if ((int64_t)p->batch * p->heads * p->seqlen_q == 0) return ok();
  if ((st = check_device()) != FA_OK) return st;
  fa::FwdArgs a{};
  a.q = p->q; a.k = p->k; a.v = p->v; a.o = p->o; a.lse = p->lse; a.cu_seqlens = nullptr;
  a.q_sb = p->q_stride[0]; a.q_st = p->q_stride[1]; a.q_sh = p->q_stride[2];
  a.k_sb = p->k_stride[0]; a.k_st = p->k_stride[1]; a.k_sh = p->k_stride[2];
  a.v_sb = p->v_stride[0]; a.v_st = p->v_stride[1]; a.v_sh = p->v_stride[2];
  a.o_sb = p->o_stride[0]; a.o_st = p->o_stride[1]; a.o_sh = p->o_stride[2];
  a.lse_sb = (int64_t)p->heads * p->seqlen_q; a.lse_sh = p->seqlen_q;
  a.batch = p->batch; a.heads = p->heads; a.nq = p->seqlen_q; a.nk = p->seqlen_k;
  a.br = fa::fwd_block_rows(p->qkv_dtype, p->head_dim, (int64_t)p->batch * p->heads, p->seqlen_q, p->causal,
                            false, fa::persistent_groups());
  a.nqt = (int32_t)ceil_div(p->seqlen_q, a.br);
  a.causal = p->causal; a.window = p->window;
  a.scale_log2 = exp2_factor(p->softmax_scale, p->q_descale * p->k_descale);
  a.v_descale = p->v_descale;
  a.lazy = lazy_threshold(p->causal, p->window);
  set_dropout(a, p->dropout_p, p->dropout_seed, p->dropout_offset);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // short causal calls (a table choice below 256 rows): the keys of each
  // 32-row block split over the work-group's waves
  if (p->qkv_dtype == FA_BF16 && a.br < 256 &&
      fa::fwd_split_keys(p->causal, p->window, a.drop_k, p->seqlen_q, p->seqlen_k, (int64_t)p->batch * p->heads,
                         fa::persistent_groups())) {
    a.br = fa::kFwdSplitRows;
    a.nqt = (int32_t)ceil_div(p->seqlen_q, a.br);
    return launched(fa::launch_fwd_bf16_split(a, p->head_dim, s));
  }
  switch (p->qkv_dtype) {
    case FA_F32: return launched(fa::launch_fwd_f32(a, p->head_dim, s));
    case FA_BF16: return launched(fa::launch_fwd_bf16(a, p->head_dim, s));
    default: return launched(fa::launch_fwd_fp8(a, p->head_dim, s));
  }
}

fa_status fa_varlen_fwd(const fa_varlen_fwd_params *p, void *stream) {
  fa_status st = fa_check_varlen_fwd(p);
  if (st != FA_OK) return st;
  if ((int64_t)p->num_seqs * p->heads * p->max_seqlen == 0) return ok();
  if ((st = check_device()) != FA_OK) return st;
  fa::FwdArgs a{};
  a.q = p->q; a.k = p->k; a.v = p->v; a.o = p->o; a.lse = p->lse; a.cu_seqlens = p->cu_seqlens;
  a.q_sb = 0; a.q_st = p->q_stride[0]; a.q_sh = p->q_stride[1];
  a.k_sb = 0; a.k_st = p->k_stride[0]; a.k_sh = p->k_stride[1];
  a.v_sb = 0; a.v_st = p->v_stride[0]; a.v_sh = p->v_stride[1];
  a.o_sb = 0; a.o_st = p->o_stride[0]; a.o_sh = p->o_stride[1];
  a.lse_sb = 0; a.lse_sh = p->total_tokens;
  a.batch = p->num_seqs; a.heads = p->heads; a.nq = p->max_seqlen; a.nk = p->max_seqlen;
  a.br = fa::fwd_block_rows(p->qkv_dtype, p->head_dim, (int64_t)p->num_seqs * p->heads, p->max_seqlen, p->causal,
                            true, fa::persistent_groups());
  a.nqt = (int32_t)ceil_div(p->max_seqlen, a.br);
  a.causal = p->causal; a.window = p->window;
  a.scale_log2 = exp2_factor(p->softmax_scale, p->q_descale * p->k_descale);
  a.v_descale = p->v_descale;
  a.lazy = lazy_threshold(p->causal, p->window);
  set_dropout(a, p->dropout_p, p->dropout_seed, p->dropout_offset);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (p->qkv_dtype) {
    case FA_F32: return launched(fa::launch_fwd_f32(a, p->head_dim, s));
    case FA_BF16: return launched(fa::launch_fwd_bf16(a, p->head_dim, s));
    default: return launched(fa::launch_fwd_fp8(a, p->head_dim, s));
  }
}

size_t fa_bwd_workspace_bytes(const fa_bwd_params *p) {
  if (fa_check_bwd(p) != FA_OK) return 0;
  return fa::bwd_workspace_bytes(p->batch, p->heads, p->seqlen_q, p->head_dim, p->deterministic);
}

fa_status fa_bwd(const fa_bwd_params *p, void *workspace, size_t workspace_bytes, void *stream) {
  fa_status st = fa_check_bwd(p);
  if (st != FA_OK) return st;
  const size_t need = fa::bwd_workspace_bytes(p->batch, p->heads, p->seqlen_q, p->head_dim, p->deterministic);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace too small (%zu bytes, need %zu)", workspace_bytes, need);
  if (need && !workspace) return fail(FA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if ((int64_t)p->batch * p->heads * (p->seqlen_q + (int64_t)p->seqlen_k) == 0) return ok();
  if ((st = check_device()) != FA_OK) return st;
  fa::BwdArgs a{};
  a.q = p->q; a.k = p->k; a.v = p->v; a.o = p->o; a.dout = p->dout; a.lse = p->lse;
  a.dq = p->dq; a.dk = p->dk; a.dv = p->dv; a.cu_seqlens = nullptr;
  const size_t dsz = need / 2;
  a.dpsum = static_cast<float *>(workspace);
  a.lse2 = reinterpret_cast<float *>(static_cast<char *>(workspace) + dsz);
  a.lse_sb = (int64_t)p->heads * p->seqlen_q; a.lse_sh = p->seqlen_q;
  a.q_sb = p->q_stride[0]; a.q_st = p->q_stride[1]; a.q_sh = p->q_stride[2];
  a.k_sb = p->k_stride[0]; a.k_st = p->k_stride[1]; a.k_sh = p->k_stride[2];
  a.v_sb = p->v_stride[0]; a.v_st = p->v_stride[1]; a.v_sh = p->v_stride[2];
  a.o_sb = p->o_stride[0]; a.o_st = p->o_stride[1]; a.o_sh = p->o_stride[2];
  a.do_sb = p->do_stride[0]; a.do_st = p->do_stride[1]; a.do_sh = p->do_stride[2];
  a.dq_sb = p->dq_stride[0]; a.dq_st = p->dq_stride[1]; a.dq_sh = p->dq_stride[2];
  a.dk_sb = p->dk_stride[0]; a.dk_st = p->dk_stride[1]; a.dk_sh = p->dk_stride[2];
  a.dv_sb = p->dv_stride[0]; a.dv_st = p->dv_stride[1]; a.dv_sh = p->dv_stride[2];
  a.batch = p->batch; a.heads = p->heads; a.nq = p->seqlen_q; a.nk = p->seqlen_k;
  a.causal = p->causal; a.window = p->window; a.deterministic = p->deterministic;
  a.grad_f32 = p->grad_dtype == FA_F32;
  a.scale = p->softmax_scale;
  a.scale_log2 = exp2_factor(p->softmax_scale, 1.f);
  set_dropout(a, p->dropout_p, p->dropout_seed, p->dropout_offset);
  return launched(fa::launch_bwd_bf16(a, p->head_dim, reinterpret_cast<hipStream_t>(stream)));
}

fa_status fa_bwd_noalloc(const fa_bwd_params *p, void *stream) {
  fa_status st = fa_check_bwd(p);
  if (st != FA_OK) return st;
  const size_t need = fa::bwd_workspace_bytes(p->batch, p->heads, p->seqlen_q, p->head_dim, p->deterministic);
  if (need > fa::kBwdScratchBytes)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "fa_bwd_noalloc: this call needs %zu bytes of scratch, more than the library's static %zu "
                "(8 bytes per row of batch x heads x seqlen_q); use fa_bwd with a workspace",
                need, (size_t)fa::kBwdScratchBytes);
  if ((int64_t)p->batch * p->heads * (p->seqlen_q + (int64_t)p->seqlen_k) == 0) return ok();
  if ((st = check_device()) != FA_OK) return st;
  void *ws = nullptr;
  const hipError_t e = fa::bwd_scratch(&ws);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "device scratch lookup failed: %s", hipGetErrorString(e));
  return fa_bwd(p, ws, fa::kBwdScratchBytes, stream);
}

size_t fa_varlen_bwd_workspace_bytes(const fa_varlen_bwd_params *p) {
  if (fa_check_varlen_bwd(p) != FA_OK) return 0;
  return fa::bwd_workspace_bytes(1, p->heads, p->total_tokens, p->head_dim, p->deterministic);
}

fa_status fa_varlen_bwd(const fa_varlen_bwd_params *p, void *workspace, size_t workspace_bytes, void *stream) {
  fa_status st = fa_check_varlen_bwd(p);
  if (st != FA_OK) return st;
  const size_t need = fa::bwd_workspace_bytes(1, p->heads, p->total_tokens, p->head_dim, p->deterministic);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace too small (%zu bytes, need %zu)", workspace_bytes, need);
  if (need && !workspace) return fail(FA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if ((int64_t)p->num_seqs * p->heads * p->max_seqlen == 0) return ok();
  if ((st = check_device()) != FA_OK) return st;
  fa::BwdArgs a{};
  a.q = p->q; a.k = p->k; a.v = p->v; a.o = p->o; a.dout = p->dout; a.lse = p->lse;
  a.dq = p->dq; a.dk = p->dk; a.dv = p->dv; a.cu_seqlens = p->cu_seqlens;
  a.dpsum = static_cast<float *>(workspace);
  a.lse2 = reinterpret_cast<float *>(static_cast<char *>(workspace) + need / 2);
  a.lse_sb = 0; a.lse_sh = p->total_tokens;
  a.q_sb = 0; a.q_st = p->q_stride[0]; a.q_sh = p->q_stride[1];
  a.k_sb = 0; a.k_st = p->k_stride[0]; a.k_sh = p->k_stride[1];
  a.v_sb = 0; a.v_st = p->v_stride[0]; a.v_sh = p->v_stride[1];
  a.o_sb = 0; a.o_st = p->o_stride[0]; a.o_sh = p->o_stride[1];
  a.do_sb = 0; a.do_st = p->do_stride[0]; a.do_sh = p->do_stride[1];
  a.dq_sb = 0; a.dq_st = p->dq_stride[0]; a.dq_sh = p->dq_stride[1];
  a.dk_sb = 0; a.dk_st = p->dk_stride[0]; a.dk_sh = p->dk_stride[1];
  a.dv_sb = 0; a.dv_st = p->dv_stride[0]; a.dv_sh = p->dv_stride[1];
  a.batch = p->num_seqs; a.heads = p->heads; a.nq = p->max_seqlen; a.nk = p->max_seqlen;
  a.causal = p->causal; a.window = p->window; a.deterministic = p->deterministic;
  a.grad_f32 = p->grad_dtype == FA_F32;
  a.scale = p->softmax_scale;
  a.scale_log2 = exp2_factor(p->softmax_scale, 1.f);
  set_dropout(a, p->dropout_p, p->dropout_seed, p->dropout_offset);
  return launched(fa::launch_bwd_bf16(a, p->head_dim, reinterpret_cast<hipStream_t>(stream)));
}

fa_status fa_check_merge(const fa_merge_params *p) {
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "params is NULL");
  if (!valid_dtype(p->parts_dtype) || !valid_dtype(p->o_dtype))
    return fail(FA_ERR_INVALID_ARGUMENT, "unknown dtype code (parts_dtype=%d, o_dtype=%d)", (int)p->parts_dtype,
                (int)p->o_dtype);
  if ((p->parts_dtype != FA_F32 && p->parts_dtype != FA_BF16) || (p->o_dtype != FA_F32 && p->o_dtype != FA_BF16))
    return fail(FA_ERR_DTYPE_MISMATCH, "partial and merged O must be fp32 or bf16 (got parts_dtype=%d o_dtype=%d)",
                (int)p->parts_dtype, (int)p->o_dtype);
  if (p->num_parts < 0 || p->batch < 0 || p->seqlen < 0 || p->heads < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 0 (num_parts=%d batch=%d seqlen=%d heads=%d)",
                p->num_parts, p->batch, p->seqlen, p->heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  const int64_t rows = (int64_t)p->batch * p->seqlen * p->heads;
  const bool empty = rows == 0;
  const bool no_parts = empty || p->num_parts == 0;
  fa_status st;
  const int pb = dtype_bytes(p->parts_dtype), ob = dtype_bytes(p->o_dtype), hd = p->head_dim;
  if ((st = check_tensor("o_parts", p->o_parts, p->parts_stride + 1, 3, pb, no_parts, p->seqlen, hd)) != FA_OK)
    return st;
  if (!no_parts && (p->parts_stride[0] < 0 || p->parts_stride[0] % (16 / pb)))
    return fail(FA_ERR_INVALID_ARGUMENT, "o_parts part stride must be >= 0 and a multiple of %d elements", 16 / pb);
  if (!no_parts && !p->lse_parts) return fail(FA_ERR_INVALID_ARGUMENT, "lse_parts is NULL");
  if ((st = check_tensor("o", p->o, p->o_stride, 3, ob, empty, p->seqlen, hd)) != FA_OK) return st;
  if ((rows + 255) / 256 * (hd / 4) > INT32_MAX) return fail(FA_ERR_INVALID_ARGUMENT, "problem too large for one launch");
  return ok();
}

fa_status fa_merge(const fa_merge_params *p, void *stream) {
  fa_status st = fa_check_merge(p);
  if (st != FA_OK) return st;
  if ((int64_t)p->batch * p->seqlen * p->heads == 0) return ok();
  if ((st = check_device()) != FA_OK) return st;
  fa::MergeArgs a{};
  a.o_parts = p->o_parts; a.lse_parts = p->lse_parts; a.o = p->o; a.lse = p->lse;
  a.p_sp = p->parts_stride[0]; a.p_sb = p->parts_stride[1]; a.p_st = p->parts_stride[2]; a.p_sh = p->parts_stride[3];
  a.lse_sp = (int64_t)p->batch * p->heads * p->seqlen;
  a.o_sb = p->o_stride[0]; a.o_st = p->o_stride[1]; a.o_sh = p->o_stride[2];
  a.num_parts = p->num_parts; a.batch = p->batch; a.seqlen = p->seqlen; a.heads = p->heads;
  a.parts_f32 = p->parts_dtype == FA_F32;
  a.out_f32 = p->o_dtype == FA_F32;
  return launched(fa::launch_merge(a, p->head_dim, reinterpret_cast<hipStream_t>(stream)));
}

fa_status fa_check_kvcache(const fa_kvcache_params *p) {
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "params is NULL");
  if (!valid_dtype(p->qkv_dtype)) return fail(FA_ERR_INVALID_ARGUMENT, "unknown dtype code (qkv_dtype=%d)", (int)p->qkv_dtype);
  if (p->qkv_dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "the KV-cache decode takes bf16 q and caches (got qkv_dtype=%d)", (int)p->qkv_dtype);
  if (p->batch < 0 || p->seqlen_q < 0 || p->cache_len < 0 || p->heads < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 0 (batch=%d seqlen_q=%d cache_len=%d heads=%d)", p->batch,
                p->seqlen_q, p->cache_len, p->heads);
  if (p->seqlen_q > 8)
    return fail(FA_ERR_UNSUPPORTED, "the KV-cache decode takes at most 8 query rows (got %d)", p->seqlen_q);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale >= 0.f))
    return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0 (got %g)", (double)p->softmax_scale);
  if (p->causal != 0 && p->causal != 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", p->causal);
  if (p->window < 0) return fail(FA_ERR_INVALID_ARGUMENT, "window must be >= 0 (got %d)", p->window);
  if (p->num_splits < 0 || p->num_splits > 256)
    return fail(FA_ERR_INVALID_ARGUMENT, "num_splits must be in [0, 256] (got %d)", p->num_splits);
  if ((p->k_new == nullptr) != (p->v_new == nullptr))
    return fail(FA_ERR_INVALID_ARGUMENT, "k_new and v_new must be given together");
  const bool empty = (int64_t)p->batch * p->seqlen_q * p->heads == 0;
  fa_status st;
  const int hd = p->head_dim;
  if ((st = check_tensor("q", p->q, p->q_stride, 3, 2, empty, p->seqlen_q, hd)) != FA_OK) return st;
  if ((st = check_tensor("o", p->o, p->o_stride, 3, 2, empty, p->seqlen_q, hd)) != FA_OK) return st;
  const bool no_cache = empty || p->cache_len == 0;
  int64_t cache_rows = p->cache_len;
  if (p->block_table) {
    const int pg = p->page_block_size;
    if (pg <= 0 || (pg & (pg - 1)))
      return fail(FA_ERR_INVALID_ARGUMENT, "page_block_size must be a power of two (got %d)", pg);
    if (p->max_blocks_per_seq < 0 || (int64_t)p->cache_len > (int64_t)p->max_blocks_per_seq * pg)
      return fail(FA_ERR_INVALID_ARGUMENT, "cache_len (%d) exceeds max_blocks_per_seq (%d) * page_block_size (%d)",
                  p->cache_len, p->max_blocks_per_seq, pg);
    cache_rows = pg;
  }
  if ((st = check_tensor("k_cache", p->k_cache, p->kc_stride, 3, 2, no_cache, cache_rows, hd)) != FA_OK) return st;
  if ((st = check_tensor("v_cache", p->v_cache, p->vc_stride, 3, 2, no_cache, cache_rows, hd)) != FA_OK) return st;
  if (p->k_new) {
    if (p->cache_len < p->seqlen_q)
      return fail(FA_ERR_INVALID_ARGUMENT, "cache_len (%d) cannot hold the %d new rows", p->cache_len, p->seqlen_q);
    if ((st = check_tensor("k_new", p->k_new, p->kn_stride, 3, 2, empty, p->seqlen_q, hd)) != FA_OK) return st;
    if ((st = check_tensor("v_new", p->v_new, p->vn_stride, 3, 2, empty, p->seqlen_q, hd)) != FA_OK) return st;
  }
  if (!empty && !p->cache_seqlens) return fail(FA_ERR_INVALID_ARGUMENT, "cache_seqlens is NULL");
  if ((int64_t)p->batch * p->heads * kvcache_splits(p) > INT32_MAX)
    return fail(FA_ERR_INVALID_ARGUMENT, "problem too large for one launch");
  return ok();
}

size_t fa_kvcache_workspace_bytes(const fa_kvcache_params *p) {
  if (fa_check_kvcache(p) != FA_OK) return 0;
  return kvcache_ws(p, kvcache_splits(p));
}

fa_status fa_fwd_kvcache(const fa_kvcache_params *p, void *workspace, size_t workspace_bytes, void *stream) {
  fa_status st = fa_check_kvcache(p);
  if (st != FA_OK) return st;
  const int splits = kvcache_splits(p);
  const size_t need = kvcache_ws(p, splits);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace too small (%zu bytes, need %zu)", workspace_bytes, need);
  if (need && !workspace) return fail(FA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if ((int64_t)p->batch * p->seqlen_q * p->heads == 0) return ok();
  if ((st = check_device()) != FA_OK) return st;
  fa::DecodeArgs a{};
  a.q = p->q; a.k_cache = p->k_cache; a.v_cache = p->v_cache; a.k_new = p->k_new; a.v_new = p->v_new;
  a.cache_seqlens = p->cache_seqlens; a.o = p->o; a.lse = p->lse;
  a.q_sb = p->q_stride[0]; a.q_st = p->q_stride[1]; a.q_sh = p->q_stride[2];
  a.kc_sb = p->kc_stride[0]; a.kc_st = p->kc_stride[1]; a.kc_sh = p->kc_stride[2];
  a.vc_sb = p->vc_stride[0]; a.vc_st = p->vc_stride[1]; a.vc_sh = p->vc_stride[2];
  a.kn_sb = p->kn_stride[0]; a.kn_st = p->kn_stride[1]; a.kn_sh = p->kn_stride[2];
  a.vn_sb = p->vn_stride[0]; a.vn_st = p->vn_stride[1]; a.vn_sh = p->vn_stride[2];
  a.o_sb = p->o_stride[0]; a.o_st = p->o_stride[1]; a.o_sh = p->o_stride[2];
  a.batch = p->batch; a.nq = p->seqlen_q; a.cache_len = p->cache_len; a.heads = p->heads;
  a.causal = p->causal; a.window = p->window; a.num_splits = splits;
  a.split_len = splits == 1 ? p->cache_len : (int)((((int64_t)p->cache_len + splits - 1) / splits + 63) / 64 * 64);
  a.scale_log2 = exp2_factor(p->softmax_scale, 1.f);
  a.block_table = p->block_table;
  if (p->block_table) {
    a.max_blocks = p->max_blocks_per_seq;
    while ((1 << a.page_shift) < p->page_block_size) ++a.page_shift;
  }
  const size_t rows = (size_t)splits * p->batch * p->seqlen_q * p->heads;
  if (splits > 1) {
    a.o_parts = static_cast<float *>(workspace);
    a.lse_parts = reinterpret_cast<float *>(static_cast<char *>(workspace) + round256(rows * p->head_dim * 4));
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (p->k_new) e = fa::launch_kv_append(a, p->head_dim, s);
  if (e == hipSuccess) e = fa::launch_decode(a, p->head_dim, s);
  if (e == hipSuccess && splits > 1) {
    fa::MergeArgs m{};
    m.o_parts = a.o_parts; m.lse_parts = a.lse_parts; m.o = p->o; m.lse = p->lse;
    const int64_t hd = p->head_dim;
    m.p_sh = hd; m.p_st = hd * p->heads; m.p_sb = m.p_st * p->seqlen_q; m.p_sp = m.p_sb * p->batch;
    m.lse_sp = (int64_t)p->batch * p->heads * p->seqlen_q;
    m.o_sb = p->o_stride[0]; m.o_st = p->o_stride[1]; m.o_sh = p->o_stride[2];
    m.num_parts = splits; m.batch = p->batch; m.seqlen = p->seqlen_q; m.heads = p->heads;
    m.parts_f32 = 1; m.out_f32 = 0;
    e = fa::launch_merge(m, p->head_dim, s);
  }
  return launched(e);
}

}  // extern "C"
