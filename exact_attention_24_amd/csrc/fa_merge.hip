// Merge of partial attention results.
//
// Attention over disjoint key subsets p, each normalised over its own keys
// and carried as (O_p, LSE_p), combines into the result over their union:
//   LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p,
// evaluated relative to the largest LSE_p.  This is the stable combination
// of per-block max and exponent sum of "FlashAttention优化Transformer显存与计算效率"
// (jsqmd.com) section 2.2.2, with each block written as LSE_p = m_p + ln l_p,
// and the step that joins the per-segment results of ring attention (the
// Ring-Attention paragraph of "Flash-Attention 2/3在ms-swift中的集成与性能提升").
// The split-K/V decode kernel uses it to join its key splits.
//
// HBM-bound: each output row reads num_parts rows of O_p and writes one row.
// D / 4 lanes per row, 4 elements per lane (16-byte fp32 or 8-byte bf16
// loads, coalesced along the head dimension); rows are (batch, token, head)
// with the head fastest, the order of the tensors in memory.  Parts with
// LSE_p = -inf are skipped without reading their O_p.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// 4 consecutive elements of a partial O row, read once (non-temporal).
template <bool F32>
__device__ __forceinline__ f32x4 load4(const void *base, int64_t off) {
  if constexpr (F32) {
    return __builtin_nontemporal_load((const f32x4 *)((const float *)base + off));
  } else {
    const u32x2 v = __builtin_nontemporal_load((const u32x2 *)((const uint16_t *)base + off));
    return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                 __uint_as_float(v.y & 0xffff0000u)};
  }
}

// Parts are taken 8 at a time: their LSEs, then all 8 O_p loads in flight at
// once, then the weighted sums against a running maximum (one batch for up
// to 8 parts, so the usual case rescales nothing).
template <int D, bool F32>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a, int64_t rows) {
  constexpr int LPR = D / 4;      // lanes per row
  constexpr int RPB = 256 / LPR;  // rows per block
  constexpr int U = 8;            // parts per batch
  const int tid = threadIdx.x, sub = tid % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  if (row >= rows) return;
  const int h = (int)(row % a.heads);
  const int64_t bn = row / a.heads;
  const int n = (int)(bn % a.seqlen), b = (int)(bn / a.seqlen);
  const int64_t lrow = ((int64_t)b * a.heads + h) * a.seqlen + n;  // [batch, heads, seqlen]
  const int np = a.num_parts;

  float m = -INFINITY, tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int64_t base = b * a.p_sb + (int64_t)n * a.p_st + h * a.p_sh + sub * 4;
  for (int p0 = 0; p0 < np; p0 += U) {
    float lp[U];
    f32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) lp[u] = p0 + u < np ? a.lse_parts[(p0 + u) * a.lse_sp + lrow] : -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)  // a part that saw no key is not read
      x[u] = lp[u] != -INFINITY ? load4<F32>(a.o_parts, (p0 + u) * a.p_sp + base) : f32x4{0.f, 0.f, 0.f, 0.f};
    float mb = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mb = fmaxf(mb, lp[u]);
    if (mb == -INFINITY) continue;  // nothing seen so far
    const float r = expf(m - mb);   // 0 on the first batch with a key (m = -inf)
    tot *= r;
    acc *= r;
    m = mb;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = lp[u] != -INFINITY ? expf(lp[u] - m) : 0.f;
      tot += w;
      acc.x = __builtin_fmaf(w, x[u].x, acc.x);
      acc.y = __builtin_fmaf(w, x[u].y, acc.y);
      acc.z = __builtin_fmaf(w, x[u].z, acc.z);
      acc.w = __builtin_fmaf(w, x[u].w, acc.w);
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int64_t oo = b * a.o_sb + (int64_t)n * a.o_st + h * a.o_sh + sub * 4;
  if (a.out_f32) {
    *(f32x4 *)((float *)a.o + oo) = acc * inv;
  } else {
    const uint2 v = {pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv)};
    *(uint2 *)((uint16_t *)a.o + oo) = v;
  }
  if (a.lse && sub == 0) a.lse[lrow] = tot > 0.f ? m + logf(tot) : -INFINITY;
}

template <int D>
hipError_t launch_merge_d(const MergeArgs &a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.seqlen * a.heads;
  if (rows == 0) return hipSuccess;
  constexpr int RPB = 256 / (D / 4);
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  if (a.parts_f32) hipLaunchKernelGGL((merge_kernel<D, true>), grid, dim3(256), 0, s, a, rows);
  else hipLaunchKernelGGL((merge_kernel<D, false>), grid, dim3(256), 0, s, a, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_merge_d<128>(a, s) : launch_merge_d<64>(a, s);
}

}  // namespace fa
