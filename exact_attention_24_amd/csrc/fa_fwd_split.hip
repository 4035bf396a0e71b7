// bf16 forward for short causal calls: the keys of a query block are split
// over the work-group's waves.
//
// Under a causal mask the last query tile of a sequence walks every key tile
// on its own, so for short sequences (few tiles per CU) the launch lasts as
// long as that one serial walk.  Here a work-group of 4 waves owns 32 query
// rows; wave w takes the key tiles w, w + 4, w + 8, ... of that range, each
// with its own running max m, exponent sum l and output accumulator, and the
// four partial results are combined at the end the way attention over
// disjoint key sets combines ("FlashAttention优化Transformer显存与计算效率"
// section 2.2.2: O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w with
// M = max_w m_w, where O_w is unnormalised).
//
// Per wave the arithmetic is that of the other bf16 kernels: S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 (each lane owns one query), the online softmax in
// fp32 with the lazy running max, P~ packed to bf16 and O^T += V^T P~^T with
// V^T read transposed from the row-major tile.  Each wave stages its own K
// and V tiles (8 KB each: 64 keys at d = 64, 32 at d = 128) by LDS DMA into
// XOR-swizzled slots, with the P.V product of a tile deferred to the next
// tile's step so that the DMA of both following tiles overlaps the softmax.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_split.h"

namespace fa {
namespace {

using namespace dev;

constexpr int kSplitWaves = 4;

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_split_kernel(FwdArgs a) {
  constexpr int NW = kSplitWaves, BR = kFwdSplitRows;
  constexpr int BC = 4096 / D;                  // keys per tile: 8 KB tiles
  constexpr int NKB = BC / 32, NKS = BC / 16;   // 32-key blocks, 16-key steps
  constexpr int NKK = D / 16, NDB = D / 32;
  constexpr int TS = BC * D;                    // tile elements
  constexpr int NBLK = TS * 2 / 1024;           // 1 KB DMA blocks per tile
  constexpr int RPB = 512 / D;                  // rows per DMA block
  constexpr int NV = 16 * NKB;                  // scores per lane per tile
  constexpr int OP = D + 4;                     // fp32 row pitch of the merge area
  constexpr int TILE_BYTES = NW * 2 * TS * 2, MERGE_BYTES = NW * BR * OP * 4 + 2 * NW * BR * 4;
  static_assert(BR == 32, "one 32-row query block per work-group");
  // per wave a K and a V tile; after the loop the same LDS holds the partial results
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES) / 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hf = lane >> 5;

  // heaviest (last) query block first, XCD-contiguous items
  int b, h, qt;
  fwd_item(blockIdx.x, a.nqt, a.heads, a.batch, false, true, b, h, qt);
  const int nq = a.nq, nk = a.nk;
  const int q0 = qt * BR;
  if (q0 >= nq) return;  // uniform for the whole work-group
  const int off = nk - nq;

  const uint16_t *qbase = (const uint16_t *)a.q + b * a.q_sb + h * a.q_sh;
  const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_sb + h * a.k_sh;
  const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_sb + h * a.v_sh;
  const __amdgpu_buffer_rsrc_t qrs = slice_rsrc(qbase, slice_bytes(nq, a.q_st, D, 2));
  const i32x4 kw = buffer_words(kbase, slice_bytes(nk, a.k_st, D, 2));
  const i32x4 vw = buffer_words(vbase, slice_bytes(nk, a.v_st, D, 2));
  const uint32_t kst2 = (uint32_t)a.k_st * 2, vst2 = (uint32_t)a.v_st * 2;

  // key tiles of the block (causal): 0 .. nt - 1; this wave's: wave, wave + NW, ...
  const int p_hi = min(q0 + BR, nq) - 1 + off;
  const int kv_hi = min(nk, p_hi + 1);
  const int nt = kv_hi > 0 ? (kv_hi + BC - 1) / BC : 0;
  const int my_q = q0 + ql, my_p = my_q + off;
  const VisRange vr = vis_range(0, min(nk - 1, my_p));
  const int p_lo = q0 + off;
  // a mask may cut tile jt for some row of the block: the diagonal or the key tail
  auto edge = [&](int jt) __attribute__((always_inline)) { return jt * BC + BC > nk || jt * BC + BC - 1 > p_lo; };

  uint4 qreg[NKK];
  {
    const uint32_t qoff = (uint32_t)my_q * (uint32_t)a.q_st * 2 + hf * 16;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qreg[kk] = bload16(qrs, qoff + kk * 32);
  }

  // this wave's tiles: DMA lane l of block q fills physical chunk l % (D / 8)
  // of row RPB q + l / (D / 8), i.e. logical chunk (that) ^ swz(row)
  uint16_t *ks = smem + wave * 2 * TS;
  uint16_t *vs = ks + TS;
  const uint32_t kl = lds_addr(ks), vl = lds_addr(vs);
  auto dma_tile = [&](i32x4 w, uint32_t l, uint32_t st2, int jt) __attribute__((always_inline)) {
    const uint32_t g = (uint32_t)(jt * BC) * st2;
#pragma unroll
    for (int q = 0; q < NBLK; ++q) {
      const int r = RPB * q + lane / (D / 8), lc = (lane % (D / 8)) ^ swz<D>(r);
      dma16_at(w, l + q * 1024, g + (uint32_t)r * st2 + lc * 16);
    }
  };
  // operand offsets (as in the ping-pong kernel): K fragment (kb, kk) at
  // (kbase_off ^ 16 kk) + 32 kb D; V^T fragment (cc, db, half) at
  // (vt_off[half] ^ 32 db) + 16 cc D
  const int kbase_off = ql * D + 8 * (swz<D>(ql) ^ hf);
  const int vt_off0 = tr_off<D>(lane, 0, 0), vt_off1 = tr_off<D>(lane, 0, 1);

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = (f32x16){};
  f32x16 s[NKB];
  uint4 pb[NKS];
#pragma unroll
  for (int i = 0; i < NKS; ++i) pb[i] = (uint4){0u, 0u, 0u, 0u};
  // running max from -FLT_MAX: a row's first finite score replaces it, and an
  // all-masked row keeps it with p = 2^(-inf) = 0
  float m = -FLT_MAX, l = 0.f;
  const float c = a.scale_log2;

  auto pv = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < NKS; ++cc)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint2 lo = lds_read_tr16(vs + ((vt_off0 ^ (32 * db)) + cc * 16 * D));
        const uint2 hi = lds_read_tr16(vs + ((vt_off1 ^ (32 * db)) + cc * 16 * D));
        acc[db] = mfma_bf16((uint4){lo.x, lo.y, hi.x, hi.y}, pb[cc], acc[db]);
      }
  };

  // step over this wave's tile jt: S(jt) = K Q^T, the deferred P.V of its
  // previous tile, then the DMA of its next K and of this V, then the softmax
  int jt = wave;
  bool prev = false;  // a P~ waits for its P.V (the V tile of the previous step is in vs)
  if (jt < nt) dma_tile(kw, kl, kst2, jt);
  for (; jt < nt; jt += NW) {
    wait_dma();  // K(jt), and V of this wave's previous tile, in its slots
    // the deferred P.V of the previous tile first, so that the V slot frees
    // (and this tile's V is on its way) before S(jt) is formed
    if (prev) pv();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    dma_tile(vw, vl, vst2, jt);
    // S(jt); then the K slot frees for the next tile's K
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = (f32x16){};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        s[kb] = mfma_bf16(*(const uint4 *)(ks + ((kbase_off ^ (16 * kk)) + kb * 32 * D)), qreg[kk], s[kb]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (jt + NW < nt) dma_tile(kw, kl, kst2, jt + NW);
    if (edge(jt)) {
      const uint32_t vo = vis_offset(vr, jt * BC + 4 * hf);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (!vis(vo, vr, kb * 32 + 8 * (e >> 2) + (e & 3))) s[kb][e] = -INFINITY;
    }
    // row max (two chains of v_max3), lazy running max, exponentials, row sum
    float m0 = max3f(s[0][0], s[0][1], s[0][2]), m1 = max3f(s[0][3], s[0][4], s[0][5]);
#pragma unroll
    for (int i = 6; i + 3 < NV; i += 4) {
      m0 = max3f(m0, s[i >> 4][i & 15], s[(i + 1) >> 4][(i + 1) & 15]);
      m1 = max3f(m1, s[(i + 2) >> 4][(i + 2) & 15], s[(i + 3) >> 4][(i + 3) & 15]);
    }
    m0 = max3f(m0, s[(NV - 2) >> 4][(NV - 2) & 15], s[(NV - 1) >> 4][(NV - 1) & 15]);
    const float mx = swap_max3(max3f(m0, m1, m1)) * c;
    const bool up = mx > m + a.lazy;
    const float alpha = up ? fast_exp2(m - mx) : 1.f;
    m = up ? mx : m;
    float rs[2];
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const float p = fast_exp2(__builtin_fmaf(s[x >> 4][x & 15], c, -m));
      s[x >> 4][x & 15] = p;
      rs[x & 1] = x < 2 ? p : rs[x & 1] + p;
    }
    l = l * alpha + (rs[0] + rs[1]);
    if (__ballot(alpha != 1.f)) {  // rarely taken once the row maxima settle
      float a_r = alpha;
      asm volatile("" : "+v"(a_r));
#pragma unroll
      for (int i = 0; i < NDB; ++i) acc[i] *= a_r;
    }
#pragma unroll
    for (int cc = 0; cc < NKS; ++cc) {
      const int kb = cc >> 1, r0 = (cc & 1) * 8;
      pb[cc].x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
      pb[cc].y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
      pb[cc].z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
      pb[cc].w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
    }
    prev = true;
  }
  if (prev) {
    wait_dma();  // V of the last tile
    pv();
  }

  // combine the four partial results through LDS (every wave is past its
  // last tile read once the barrier has passed)
  __syncthreads();
  float *mo = (float *)smem;                 // [NW][BR][OP] unnormalised O rows
  float *mm = mo + NW * BR * OP;             // [NW][BR] running max (log2 units)
  float *ml = mm + NW * BR;                  // [NW][BR] exponent sums
  const float lt = half_swap_sum(l);
  {
    float *row = mo + (wave * BR + ql) * OP;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) row[db * 32 + 8 * (i >> 2) + 4 * hf + (i & 3)] = acc[db][i];
    if (hf == 0) {
      mm[wave * BR + ql] = m;
      ml[wave * BR + ql] = lt;
    }
  }
  __syncthreads();
  {
    constexpr int TPR = 256 / BR, CPT = D / TPR;  // threads per row, columns per thread
    const int r = tid / TPR, part = tid % TPR;
    float mw[NW], M = -FLT_MAX;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = mm[w * BR + r];
      M = fmaxf(M, mw[w]);
    }
    float f[NW], L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      f[w] = fast_exp2(mw[w] - M);
      L += f[w] * ml[w * BR + r];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int q = q0 + r;
    if (q < nq) {
      uint16_t *orow = (uint16_t *)a.o + b * a.o_sb + (int64_t)q * a.o_st + h * a.o_sh + part * CPT;
#pragma unroll
      for (int c8 = 0; c8 < CPT; c8 += 8) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float t = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) t += f[w] * mo[(w * BR + r) * OP + part * CPT + c8 + j];
          y[j] = t * inv;
        }
        uint4 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        o.z = pack_bf16x2(y[4], y[5]);
        o.w = pack_bf16x2(y[6], y[7]);
        *(uint4 *)(orow + c8) = o;
      }
      if (part == 0 && a.lse)
        a.lse[b * a.lse_sb + h * a.lse_sh + q] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

// At most 4 blocks per CU (two rounds of two resident work-groups): there the
// serial walk of the last tiles sets the launch time, and the split measured
// 12-13% faster (B2 H16 N1024 causal, d 64 and 128).  With more blocks the
// 128-row tiles' shared K/V staging wins (B1 H32 N2048 d128: 61 against 69 us).
bool fwd_split_keys(int causal, int window, uint32_t drop_k, int64_t nq, int64_t nk, int64_t batch_heads, int cus) {
  const int64_t blocks = batch_heads * ((nq + kFwdSplitRows - 1) / kFwdSplitRows);
  return causal && window == 0 && drop_k == 0 && nq <= kFwdSplitMaxRows && nk <= kFwdSplitMaxRows &&
         blocks <= 4 * (int64_t)(cus > 0 ? cus : 256);
}

hipError_t launch_fwd_bf16_split(const FwdArgs &a, int head_dim, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.nqt * a.heads * a.batch));
  if (head_dim == 128) hipLaunchKernelGGL((fwd_bf16_split_kernel<128>), grid, dim3(kSplitWaves * 64), 0, s, a);
  else hipLaunchKernelGGL((fwd_bf16_split_kernel<64>), grid, dim3(kSplitWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
