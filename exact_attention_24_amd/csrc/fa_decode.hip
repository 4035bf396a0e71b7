// KV-cache incremental decoding.
//
// flash_attn_with_kvcache(q, k_cache, v_cache, k, v, cache_seqlens, causal)
// of "突破AI算力瓶颈：FlashAttention与MindSpore 2.0全场景融合方案" (推理优化与KV缓存):
// the new k, v rows are written into the cache at position cache_seqlens[b],
// then the nq query rows, which are the last nq positions, attend over the
// cache up to and including them (bottom-right causal, optional window).
//
// One decoding step reads each batch entry's cache prefix once for a handful
// of query rows, about 2 nq FLOPs per byte, so it is bound by HBM and the
// arithmetic stays on the VALU: v_dot2c_f32_bf16 for q.k, fp32 FMAs for P.V.
// The keys of each (batch, head) are cut into num_splits ranges of split_len
// keys, one work-group each (split-K), so that a small batch still fills 256
// CUs; with more than one split each work-group writes a partial (O, LSE)
// that the merge kernel joins.
//
// Inside a work-group (4 waves), a key row of d bf16 is read by d/8 lanes,
// 16 bytes each, so one wave-wide load covers 64/(d/8) keys; every lane group
// keeps its own online-softmax state (running max m, sum l, its 8 columns of
// O) per query, and the states of the groups, then of the waves, are joined
// at the end.  Loads run one step ahead of the arithmetic.  Paged caches
// (fixed-size pages named by a block table, the paged storage of the same
// section) differ only in how a logical row is addressed.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;  // the running max moves only when a score exceeds it by 2^8

// ---------------------------------------------------------------------------
// Append: k_new, v_new rows (b, i, h) go to cache row cache_seqlens[b] + i.
// ---------------------------------------------------------------------------
// Element offset of logical cache row j of batch entry b (block and token
// strides sb, st): contiguous, or through the block table.
template <bool PAGED>
__device__ __forceinline__ int64_t cache_row(const DecodeArgs &a, int b, int j, int64_t sb, int64_t st) {
  if constexpr (PAGED) {
    const int blk = a.block_table[(int64_t)b * a.max_blocks + (j >> a.page_shift)];
    return blk * sb + (int64_t)(j & ((1 << a.page_shift) - 1)) * st;
  } else {
    return b * sb + (int64_t)j * st;
  }
}

template <int D, bool PAGED>
__global__ __launch_bounds__(256) void kv_append_kernel(DecodeArgs a, int64_t rows) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int tid = threadIdx.x, c = tid % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;  // (b, i, h), h fastest
  if (row >= rows) return;
  const int h = (int)(row % a.heads);
  const int64_t bi = row / a.heads;
  const int i = (int)(bi % a.nq), b = (int)(bi / a.nq);
  const int t = a.cache_seqlens[b] + i;
  const uint4 kx = *(const uint4 *)((const uint16_t *)a.k_new + b * a.kn_sb + (int64_t)i * a.kn_st + h * a.kn_sh + c * 8);
  const uint4 vx = *(const uint4 *)((const uint16_t *)a.v_new + b * a.vn_sb + (int64_t)i * a.vn_st + h * a.vn_sh + c * 8);
  *(uint4 *)((uint16_t *)a.k_cache + cache_row<PAGED>(a, b, t, a.kc_sb, a.kc_st) + h * a.kc_sh + c * 8) = kx;
  *(uint4 *)((uint16_t *)a.v_cache + cache_row<PAGED>(a, b, t, a.vc_sb, a.vc_st) + h * a.vc_sh + c * 8) = vx;
}

__device__ __forceinline__ float dot8(const uint32_t (&q)[4], const uint4 &k) {
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[0]), __builtin_bit_cast(bf16x2_t, k.x), 0.f,
                                            false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[1]), __builtin_bit_cast(bf16x2_t, k.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[2]), __builtin_bit_cast(bf16x2_t, k.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[3]), __builtin_bit_cast(bf16x2_t, k.w), s, false);
  return s;
}

// Join online-softmax state (m2, l2, acc2) into (m, l, acc); m in log2 units.
template <int N>
__device__ __forceinline__ void join_state(float &m, float &l, float (&acc)[N], float m2, float l2,
                                           const float (&acc2)[N]) {
  const float mn = fmaxf(m, m2);
  const float a1 = m == -INFINITY ? 0.f : exp2f(m - mn);
  const float a2 = m2 == -INFINITY ? 0.f : exp2f(m2 - mn);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * a1 + acc2[e] * a2;
  m = mn;
}

// ---------------------------------------------------------------------------
// Decode: one work-group per (batch, head, split); NQ >= nq query rows.
// ---------------------------------------------------------------------------
template <int D, int NQ, bool PAGED>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int LPK = D / 8;   // lanes per key row
  constexpr int G = 64 / LPK;  // keys per wave-wide load
  constexpr int U = 4;         // loads per wave per step
  constexpr int KW = G * U;    // keys per wave per step
  constexpr int KS = 4 * KW;   // keys per work-group per step
  __shared__ float s_m[4][NQ], s_l[4][NQ];
  __shared__ float s_acc[4][NQ][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane % LPK, g = lane / LPK;
  const int S = a.num_splits;
  const int split = blockIdx.x % S, bh = blockIdx.x / S;
  const int h = bh % a.heads, b = bh / a.heads;
  const int nq = a.nq, causal = a.causal, window = a.window;
  const int L = a.cache_seqlens[b] + (a.k_new ? nq : 0);  // keys of this batch entry
  const int qpos0 = L - nq;                                // key position of query row 0
  int lo = split * a.split_len;
  const int hi = min(L, lo + a.split_len);
  if (window > 0) lo = max(lo, qpos0 - window + 1);

  uint32_t qv[NQ][4];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    uint4 x = {0u, 0u, 0u, 0u};
    if (i < nq) x = *(const uint4 *)((const uint16_t *)a.q + b * a.q_sb + (int64_t)i * a.q_st + h * a.q_sh + c * 8);
    qv[i][0] = x.x; qv[i][1] = x.y; qv[i][2] = x.z; qv[i][3] = x.w;
  }
  float m[NQ], l[NQ], acc[NQ][8];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  }

  const uint16_t *kb = (const uint16_t *)a.k_cache + h * a.kc_sh + c * 8;
  const uint16_t *vb = (const uint16_t *)a.v_cache + h * a.vc_sh + c * 8;
  const int jw = wave * KW + g;  // this lane group's first key of a step
  // Paged caches: the block-table entries of a step's rows are read one step
  // before its K/V rows (which are read one step before their arithmetic),
  // so the table lookup never stalls a K/V load.
  const int pmask = PAGED ? (1 << a.page_shift) - 1 : 0;
  const int32_t *tbl = PAGED ? a.block_table + (int64_t)b * a.max_blocks : nullptr;
  auto table = [&](int j) __attribute__((always_inline)) -> int {
    return (PAGED && j < hi) ? tbl[j >> a.page_shift] : 0;
  };
  // rows j >= hi read as zeros (and are masked); blk: j's table entry (paged)
  auto load_kv = [&](int j, int blk, uint4 &kx, uint4 &vx) __attribute__((always_inline)) {
    kx = vx = uint4{0u, 0u, 0u, 0u};
    if (j < hi) {
      if constexpr (PAGED) {
        kx = *(const uint4 *)(kb + blk * a.kc_sb + (int64_t)(j & pmask) * a.kc_st);
        vx = *(const uint4 *)(vb + blk * a.vc_sb + (int64_t)(j & pmask) * a.vc_st);
      } else {
        kx = *(const uint4 *)(kb + cache_row<false>(a, b, j, a.kc_sb, a.kc_st));
        vx = *(const uint4 *)(vb + cache_row<false>(a, b, j, a.vc_sb, a.vc_st));
      }
    }
  };
  uint4 kc[U], vc[U];
  int tb_next[U];  // table entries of the next step's rows
#pragma unroll
  for (int u = 0; u < U; ++u) {
    load_kv(lo + jw + u * G, table(lo + jw + u * G), kc[u], vc[u]);
    tb_next[u] = table(lo + KS + jw + u * G);
  }
  for (int base = lo; base < hi; base += KS) {
    uint4 kn[U], vn[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // in flight during this step
      load_kv(base + KS + jw + u * G, tb_next[u], kn[u], vn[u]);
      tb_next[u] = table(base + 2 * KS + jw + u * G);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + jw + u * G;
      float vf[8];
      vf[0] = __uint_as_float(vc[u].x << 16); vf[1] = __uint_as_float(vc[u].x & 0xffff0000u);
      vf[2] = __uint_as_float(vc[u].y << 16); vf[3] = __uint_as_float(vc[u].y & 0xffff0000u);
      vf[4] = __uint_as_float(vc[u].z << 16); vf[5] = __uint_as_float(vc[u].z & 0xffff0000u);
      vf[6] = __uint_as_float(vc[u].w << 16); vf[7] = __uint_as_float(vc[u].w & 0xffff0000u);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        float part = dot8(qv[i], kc[u]);
#pragma unroll
        for (int x = 1; x < LPK; x <<= 1) part += __shfl_xor(part, x);
        const int pos = qpos0 + i;
        const bool vis = j < hi && i < nq && (!causal || j <= pos) && (window <= 0 || j > pos - window);
        if (vis) {  // uniform over the lane group
          const float s = part * a.scale_log2;
          if (s > m[i] + kLazy || m[i] == -INFINITY) {
            const float alpha = exp2f(m[i] - s);  // 0 while nothing was seen
            l[i] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i][e] *= alpha;
            m[i] = s;
          }
          const float p = exp2f(s - m[i]);
          l[i] += p;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] = __builtin_fmaf(p, vf[e], acc[i][e]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kc[u] = kn[u];
      vc[u] = vn[u];
    }
  }

  // join the lane groups of the wave (same columns, other keys), then the waves
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) {
      float acc2[8];
      const float m2 = __shfl_xor(m[i], x), l2 = __shfl_xor(l[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc2[e] = __shfl_xor(acc[i][e], x);
      join_state(m[i], l[i], acc[i], m2, l2, acc2);
    }
    if (g == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][i][c * 8 + e] = acc[i][e];
      if (c == 0) {
        s_m[wave][i] = m[i];
        s_l[wave][i] = l[i];
      }
    }
  }
  __syncthreads();
  if (tid >= NQ * LPK) return;
  const int i = tid / LPK, cc = tid % LPK;
  if (i >= nq) return;
  float mt = s_m[0][i], lt = s_l[0][i], at[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) at[e] = s_acc[0][i][cc * 8 + e];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    float a2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a2[e] = s_acc[w][i][cc * 8 + e];
    join_state(mt, lt, at, s_m[w][i], s_l[w][i], a2);
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (mt + log2f(lt)) * kLn2 : -INFINITY;
  if (S == 1) {
    uint4 w;
    w.x = pack_bf16x2(at[0] * inv, at[1] * inv);
    w.y = pack_bf16x2(at[2] * inv, at[3] * inv);
    w.z = pack_bf16x2(at[4] * inv, at[5] * inv);
    w.w = pack_bf16x2(at[6] * inv, at[7] * inv);
    *(uint4 *)((uint16_t *)a.o + b * a.o_sb + (int64_t)i * a.o_st + h * a.o_sh + cc * 8) = w;
    if (a.lse && cc == 0) a.lse[((int64_t)b * a.heads + h) * nq + i] = lse;
  } else {
    const int64_t prow = (((int64_t)split * a.batch + b) * nq + i) * a.heads + h;
    float *op = a.o_parts + prow * D + cc * 8;
    *(float4 *)op = float4{at[0] * inv, at[1] * inv, at[2] * inv, at[3] * inv};
    *(float4 *)(op + 4) = float4{at[4] * inv, at[5] * inv, at[6] * inv, at[7] * inv};
    if (cc == 0) a.lse_parts[(((int64_t)split * a.batch + b) * a.heads + h) * nq + i] = lse;
  }
}

template <int D, bool PAGED>
hipError_t launch_decode_p(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.batch * a.heads * a.num_splits));
  if (a.nq <= 1) hipLaunchKernelGGL((decode_kernel<D, 1, PAGED>), grid, dim3(256), 0, s, a);
  else if (a.nq <= 2) hipLaunchKernelGGL((decode_kernel<D, 2, PAGED>), grid, dim3(256), 0, s, a);
  else if (a.nq <= 4) hipLaunchKernelGGL((decode_kernel<D, 4, PAGED>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((decode_kernel<D, 8, PAGED>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t s) {
  return a.block_table ? launch_decode_p<D, true>(a, s) : launch_decode_p<D, false>(a, s);
}

template <int D>
hipError_t launch_kv_append_d(const DecodeArgs &a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.nq * a.heads;
  constexpr int RPB = 256 / (D / 8);
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  if (a.block_table) hipLaunchKernelGGL((kv_append_kernel<D, true>), grid, dim3(256), 0, s, a, rows);
  else hipLaunchKernelGGL((kv_append_kernel<D, false>), grid, dim3(256), 0, s, a, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const DecodeArgs &a, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_kv_append_d<128>(a, s) : launch_kv_append_d<64>(a, s);
}

hipError_t launch_decode(const DecodeArgs &a, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_decode_d<128>(a, s) : launch_decode_d<64>(a, s);
}

}  // namespace fa
