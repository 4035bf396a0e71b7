// Backward kernels: gradients of exact attention by recomputation.
//
// The forward keeps only O and the per-row log-sum-exp; the backward
// recomputes the scores tile by tile instead of storing S ("重计算" in
// "Flash-Attention 2/3在ms-swift中的集成与性能提升" and step 5 of section 三 of
// the adg.csdn.net flash_attn/Qwen page).  With L = sum(dO * O) and
// P = exp(scale * Q K^T - LSE) (masked entries 0), the chain rule gives
//   D_i  = sum_c dO_ic O_ic            (= sum_j P_ij dP_ij)
//   dV   = P^T dO,   dP = dO V^T,   dS = P * (dP - D),
//   dK   = scale dS^T Q,   dQ = scale dS K.
//
// Three launches on the caller's stream:
//   1. bwd_dsum_kernel  D = rowsum(dO * O) in fp32 (workspace).
//   2. bwd_dkdv_kernel  one work-group per tile of 32*NW keys; loops over the
//      query tiles that see them; per tile S = Q K^T and dP = dO V^T (B
//      operands K, V held in VGPRs), P and dS in fp32 registers, then
//      dV^T += dO^T P and dK^T += Q^T dS with A operands read from transposed
//      copies of the Q / dO tiles in LDS and B operands taken straight from
//      the accumulators.  dK, dV are written once, no atomics.
//   3. bwd_dq_kernel    one work-group per tile of 32*NW queries; loops over
//      key tiles; S^T = K Q^T and dP^T = V dO^T (lane = query, so LSE and D
//      are per-lane scalars), dS^T, then dQ^T += K^T dS^T with K^T from a
//      transposed copy of the key tile.  Written once, no atomics.
// Splitting dQ from dK/dV costs the recomputation of S and dP a second time
// (7 tile products instead of 5) but needs no cross-work-group reduction, so
// the gradients are bitwise reproducible from call to call.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

__device__ __forceinline__ float bf16_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

// Store 4 consecutive gradient values of one row (fp32 or bf16).
__device__ __forceinline__ void store_grad4(void *base, int64_t elem_off, bool f32, float x0, float x1,
                                            float x2, float x3) {
  if (f32) {
    float4 v = {x0, x1, x2, x3};
    *(float4 *)((float *)base + elem_off) = v;
  } else {
    uint2 w = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
    *(uint2 *)((uint16_t *)base + elem_off) = w;
  }
}

// ---------------------------------------------------------------------------
// 1. D_i = sum_c dO_ic O_ic and LSE_i log2(e), [batch, heads, nq] fp32.
//    A row that saw no key (LSE = -inf) gets +inf, so P = 2^(s - lse2) = 0.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;       // lanes per row, 8 bf16 each
  constexpr int RPB = 256 / LPR;   // rows per block
  const int tid = threadIdx.x, sub = tid % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;  // (b, h, q) order
  const int64_t total = (int64_t)a.batch * a.heads * a.nq;
  float acc = 0.f;
  if (row < total) {
    const int q = (int)(row % a.nq);
    const int64_t bh = row / a.nq;
    const int h = (int)(bh % a.heads), b = (int)(bh / a.heads);
    const uint4 ov = *(const uint4 *)((const uint16_t *)a.o + b * a.o_sb + (int64_t)q * a.o_st +
                                      h * a.o_sh + sub * 8);
    const uint4 dv = *(const uint4 *)((const uint16_t *)a.dout + b * a.do_sb + (int64_t)q * a.do_st +
                                      h * a.do_sh + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(bf16_to_f32(u16_at(ov, e)), bf16_to_f32(u16_at(dv, e)), acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < total && sub == 0) {
    a.dpsum[row] = acc;
    const float x = a.lse[row];
    a.lse2[row] = x == -INFINITY ? INFINITY : x * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: key-tile outer, query-tile inner.  One work-group of 4 waves per
//    128 keys (32 per wave, one wave per SIMD); per query tile of 64 rows:
//      phase A: S = Q K^T and dP = dO V^T (K, V held as B operands in
//               AGPRs; Q, dO row fragments read from LDS);
//      phase B: dV^T += dO^T P^T and dK^T += Q^T dS^T (P^T, dS^T straight
//               from the phase-A accumulators of the previous tile; dO^T,
//               Q^T read transposed from the row-major tiles), with the
//               VALU computing P = 2^(s c - lse2) and dS = P (dP - D) of
//               the current tile between the MFMAs.
//    Q, dO, lse2 and D tiles arrive by LDS DMA one tile ahead into three
//    buffers; Q and dO are unpadded with XOR-swizzled 16-byte chunks.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 4, T = NW * 64, BC = 32 * NW, BR = 64;
  constexpr int DCH = D / 8, TS = BR * D;  // Q or dO tile (bf16 elements)
  constexpr int PER = BR * DCH / T;        // 16-byte DMA loads per lane per tile and tensor
  constexpr int NK = D / 16;               // d-steps of S and dP
  constexpr int NA = 4 * NK;               // phase-A MFMAs (S, dP) x (2 query blocks)
  constexpr int NB = (D / 32) * 8;         // phase-B MFMAs (dV, dK) x (D/32) x (4 query chunks)
  constexpr int BUF = 2 * TS * 2 + 2 * 1024;  // bytes per buffer: Q, dO, lse2 (1 KB slot), D (1 KB slot)
  constexpr int RING = 8;                  // operand fragments in flight
  __shared__ __attribute__((aligned(16))) unsigned char smem[3 * BUF];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hf = lane >> 5;
  const int nq = a.nq, nk = a.nk, off = nk - nq;
  const int causal = a.causal, window = a.window;

  const int nkt = (nk + BC - 1) / BC;
  const int item = xcd_item(blockIdx.x, nkt * a.heads * a.batch);
  const int bh = item / nkt, kt = item % nkt;  // causal: low key tiles (most work) first
  const int b = bh / a.heads, h = bh % a.heads;
  const int k0 = kt * BC;
  const int wk0 = k0 + 32 * wave;
  const int my_k = wk0 + ql;

  const uint16_t *qbase = (const uint16_t *)a.q + b * a.q_sb + h * a.q_sh;
  const uint16_t *dobase = (const uint16_t *)a.dout + b * a.do_sb + h * a.do_sh;
  const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_sb + h * a.k_sh;
  const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_sb + h * a.v_sh;
  const i32x4 qw = buffer_words(qbase, slice_bytes(nq, a.q_st, D, 2));
  const i32x4 dow = buffer_words(dobase, slice_bytes(nq, a.do_st, D, 2));
  const i32x4 lw = buffer_words(a.lse2 + (int64_t)bh * nq, (uint32_t)nq * 4);
  const i32x4 dw = buffer_words(a.dpsum + (int64_t)bh * nq, (uint32_t)nq * 4);
  const __amdgpu_buffer_rsrc_t krs = slice_rsrc(kbase, slice_bytes(nk, a.k_st, D, 2));
  const __amdgpu_buffer_rsrc_t vrs = slice_rsrc(vbase, slice_bytes(nk, a.v_st, D, 2));
  const uint32_t qst2 = (uint32_t)a.q_st * 2, dost2 = (uint32_t)a.do_st * 2;

  // this wave's 32 keys: B operands of S = Q K^T and dP = dO V^T (AGPRs)
  u32x4 kreg[NK], vreg[NK];
  {
    const uint32_t ko = (uint32_t)my_k * (uint32_t)a.k_st * 2 + hf * 16;
    const uint32_t vo = (uint32_t)my_k * (uint32_t)a.v_st * 2 + hf * 16;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      kreg[kk] = vec4(bload16(krs, ko + kk * 32));
      vreg[kk] = vec4(bload16(vrs, vo + kk * 32));
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) asm volatile("s_nop 1" : "+a"(kreg[kk]), "+a"(vreg[kk]));
  }

  // query tiles that can see some key of this work-group
  int q_lo = 0, q_hi = nq;
  if (causal) q_lo = max(0, k0 - off);
  if (window > 0) q_hi = min(nq, k0 + BC - 1 - off + window);
  const int it0 = q_lo / BR;
  const int it1 = q_hi > q_lo ? (q_hi + BR - 1) / BR : it0;

  const uint32_t lds0 = lds_addr(smem);
  auto slot = [&](int it) __attribute__((always_inline)) { return (it - it0) % 3; };
  auto qbuf = [&](int it) __attribute__((always_inline)) { return (const uint16_t *)(smem + slot(it) * BUF); };
  auto dobuf = [&](int it) __attribute__((always_inline)) { return qbuf(it) + TS; };
  auto fbuf = [&](int it) __attribute__((always_inline)) {  // lse2[64] at +0, D[64] at +256 floats
    return (const float *)(smem + slot(it) * BUF + 2 * TS * 2);
  };
  uint32_t qgo[PER], dgo[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int sl = i * T + tid, r = sl / DCH, lc = (sl % DCH) ^ swz<D>(r);
    qgo[i] = (uint32_t)r * qst2 + lc * 16;
    dgo[i] = (uint32_t)r * dost2 + lc * 16;
  }
  auto load_tile = [&](int it) __attribute__((always_inline)) {
    const int q0 = it * BR;
    const uint32_t l0 = lds0 + (uint32_t)(slot(it) * BUF + wave * 1024);
    const uint32_t gq = (uint32_t)q0 * qst2, gd = (uint32_t)q0 * dost2;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      dma16_at(qw, l0 + i * T * 16, gq + qgo[i]);
      dma16_at(dow, l0 + TS * 2 + i * T * 16, gd + dgo[i]);
    }
    // 64 lse2 and 64 D values: 16 lanes of one wave each
    if (wave == 0 && lane < 16)
      dma16_at(lw, lds0 + (uint32_t)(slot(it) * BUF + 2 * TS * 2), (uint32_t)q0 * 4 + lane * 16);
    if (wave == 1 && lane < 16)
      dma16_at(dw, lds0 + (uint32_t)(slot(it) * BUF + 2 * TS * 2 + 1024), (uint32_t)q0 * 4 + lane * 16);
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dk[i] = dv[i] = (f32x16){};
  const float c = a.scale_log2;

  f32x16 s[2], dp[2];            // S and dP of the current tile, [query block]; lane = key
  // bf16 P^T, dS^T of the previous tile, [16-query chunk]; zero before the
  // first tile, so its products add nothing and the loop needs no branch
  uint4 pb[4], sb[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) pb[cc] = sb[cc] = (uint4){0u, 0u, 0u, 0u};

  // operand fragments: phase A (j < NA): j = 4 kk + 2 qb + w, w = 0: Q rows, 1: dO rows;
  // phase B (j >= NA): j - NA = 8 db + 2 cc + w, w = 0: dO^T, 1: Q^T
  const int kx = hf ^ swz<D>(ql);
  auto fread = [&](int it, int j) __attribute__((always_inline)) -> uint4 {
    if (j < NA) {
      const int kk = j / 4, qb = (j / 2) % 2, w = j % 2;
      const int o = (qb * 32 + ql) * D + (((2 * kk) ^ kx) << 3);
      return w ? *(const uint4 *)(dobuf(it) + o) : *(const uint4 *)(qbuf(it) + o);
    }
    const int jb = j - NA, db = jb / 8, cc = (jb / 2) % 4, w = jb % 2;
    const int o = cc * 16 * D;
    uint2 lo, hi;
    if (w) {
      lo = lds_read_tr16(qbuf(it) + o + tr_off<D>(lane, db, 0));
      hi = lds_read_tr16(qbuf(it) + o + tr_off<D>(lane, db, 1));
    } else {
      lo = lds_read_tr16(dobuf(it) + o + tr_off<D>(lane, db, 0));
      hi = lds_read_tr16(dobuf(it) + o + tr_off<D>(lane, db, 1));
    }
    return (uint4){lo.x, lo.y, hi.x, hi.y};
  };

  // P, dS of one tile (MASK: causal / window edge); element e = 16 qb + r is
  // query 32 qb + 8 (r / 4) + 4 hf + r % 4 of the tile
  auto one_tile = [&](auto mask_tag, int it) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int q0 = it * BR;
    if (it + 1 < it1) load_tile(it + 1);
    // phase-A fragments come from this tile, phase-B fragments from the
    // previous one (its products are pending; before the first tile they
    // are zero and any resident tile will do)
    const int itp = it > it0 ? it - 1 : it;
    auto frag = [&](int j) __attribute__((always_inline)) { return fread(j < NA ? it : itp, j); };
    uint4 ring[RING];
#pragma unroll
    for (int j = 0; j < RING; ++j) ring[j] = frag(j);
    const float *fl = fbuf(it);
    // ---- phase A
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const uint4 f = ring[j % RING];
      if (j + RING < NA + NB) ring[j % RING] = frag(j + RING);
      const int kk = j / 4, qb = (j / 2) % 2, w = j % 2;
      if (w) {
        if (kk == 0) mfma_v_first(dp[qb], f, vreg[0]);
        else mfma_v(dp[qb], f, vreg[kk]);
      } else {
        if (kk == 0) mfma_v_first(s[qb], f, kreg[0]);
        else mfma_v(s[qb], f, kreg[kk]);
      }
    }
    // lse2 and D of this lane's 32 query rows (4 consecutive rows per float4)
    float4 lse4[8], d4[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int qi = (g / 4) * 32 + 8 * (g % 4) + 4 * hf;
      lse4[g] = *(const float4 *)(fl + qi);
      d4[g] = *(const float4 *)(fl + 256 + qi);
    }
    mfma_drain2_v(s[0], s[1]);
    mfma_drain2_v(dp[0], dp[1]);
    if (MASK) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qpos = q0 + qb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3) + off;
          const bool ok = (!causal || my_k <= qpos) && (window <= 0 || my_k > qpos - window) &&
                          qpos - off < nq;
          if (!ok) s[qb][r] = -INFINITY;
        }
    }
    // ---- phase B: the previous tile's products, this tile's P and dS
    constexpr int EPS = 32 / NB;  // elements started per stage
    static_assert(EPS * NB == 32, "stages must divide the lane's 32 elements");
    auto comp = [](const float4 &v, int i) __attribute__((always_inline)) {
      return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
    };
    // element e = 16 qb + r; its query row's lse2 / D sit in lse4 / d4[e / 4]
    auto elem_fma = [&](int e) __attribute__((always_inline)) {
      s[e / 16][e % 16] = __builtin_fmaf(s[e / 16][e % 16], c, -comp(lse4[e / 4], e % 4));
    };
    auto elem_exp = [&](int e) __attribute__((always_inline)) { s[e / 16][e % 16] = fast_exp2(s[e / 16][e % 16]); };
    auto elem_ds = [&](int e) __attribute__((always_inline)) {
      dp[e / 16][e % 16] = s[e / 16][e % 16] * (dp[e / 16][e % 16] - comp(d4[e / 4], e % 4));
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int jj = NA + j;
      const uint4 f = ring[jj % RING];
      if (jj + RING < NA + NB) ring[jj % RING] = frag(jj + RING);
      {
        const int db = j / 8, cc = (j / 2) % 4, w = j % 2;
        if (j == 0) asm volatile("s_nop 1");
        if (w) mfma_a(dk[db], f, sb[cc]);
        else mfma_a(dv[db], f, pb[cc]);
      }
      // element pipeline over the 32 elements of the lane, EPS per stage:
      // fma at stage e / EPS, exp one stage later, dS two stages later
#pragma unroll
      for (int k = 0; k < EPS; ++k) {
        if (j * EPS + k < 32) elem_fma(j * EPS + k);
        if (j >= 1) elem_exp((j - 1) * EPS + k);
        if (j >= 2) elem_ds((j - 2) * EPS + k);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // tail of the element pipeline
#pragma unroll
    for (int k = 0; k < EPS; ++k) {
      elem_exp((NB - 1) * EPS + k);
      elem_ds((NB - 2) * EPS + k);
      elem_ds((NB - 1) * EPS + k);
    }
    // the phase-B MFMAs above have read pb / sb (operands are read at issue)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int qb = cc >> 1, r0 = (cc & 1) * 8;
      uint4 &p = pb[cc], &d = sb[cc];
      p.x = pack_bf16x2(s[qb][r0 + 0], s[qb][r0 + 1]);
      p.y = pack_bf16x2(s[qb][r0 + 2], s[qb][r0 + 3]);
      p.z = pack_bf16x2(s[qb][r0 + 4], s[qb][r0 + 5]);
      p.w = pack_bf16x2(s[qb][r0 + 6], s[qb][r0 + 7]);
      d.x = pack_bf16x2(dp[qb][r0 + 0], dp[qb][r0 + 1]);
      d.y = pack_bf16x2(dp[qb][r0 + 2], dp[qb][r0 + 3]);
      d.z = pack_bf16x2(dp[qb][r0 + 4], dp[qb][r0 + 5]);
      d.w = pack_bf16x2(dp[qb][r0 + 6], dp[qb][r0 + 7]);
    }
    wait_dma();
    __syncthreads();
    // the compiler may move accumulators at loop boundaries: only after the
    // last MFMA has finished
#pragma unroll
    for (int i = 0; i < D / 32; ++i) asm volatile("" : "+a"(dk[i]), "+a"(dv[i]));
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < D / 32; ++i) asm volatile("" : "+a"(dk[i]), "+a"(dv[i]));
  };

  // tiles [it0, ia) are cut by the causal diagonal, [ib, it1) by the window
  // or the end of the queries; the rest see every key of the work-group
  int ia = it0, ib = it1;
  if (causal) {
    const int lim = k0 + BC - 1 - off;  // first query row that sees all keys
    ia = min(it1, max(it0, (lim + BR - 1) / BR));
  }
  if (window > 0) {
    const int lim = k0 - off + window;  // rows >= lim lose the first key
    ib = max(ia, min(it1, lim / BR));
  }
  if (it1 * BR > nq) ib = max(ia, min(ib, it1 - 1));

  if (it0 < it1) load_tile(it0);
  wait_dma();
  __syncthreads();
  const std::true_type masked;
  const std::false_type whole;
  for (int it = it0; it < ia; ++it) one_tile(masked, it);
  for (int it = ia; it < ib; ++it) one_tile(whole, it);
  for (int it = ib; it < it1; ++it) one_tile(masked, it);
  // the last tile's products
  if (it0 < it1) {
    const int it = it1 - 1;
    uint4 ring[RING];
#pragma unroll
    for (int j = 0; j < RING; ++j) ring[j] = fread(it, NA + j);
    asm volatile("s_nop 1");
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint4 f = ring[j % RING];
      if (j + RING < NB) ring[j % RING] = fread(it, NA + j + RING);
      const int db = j / 8, cc = (j / 2) % 4, w = j % 2;
      if (w) mfma_a(dk[db], f, sb[cc]);
      else mfma_a(dv[db], f, pb[cc]);
    }
  }
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    mfma_drain_a(dk[i]);
    mfma_drain_a(dv[i]);
  }

  // dK = scale * (dS^T Q), dV = P^T dO; lane = key, d = db*32 + 8*rb + 4*hf + 0..3
  if (my_k < nk) {
    const float sc = a.scale;
    const int64_t kro = b * a.dk_sb + (int64_t)my_k * a.dk_st + h * a.dk_sh;
    const int64_t vro = b * a.dv_sb + (int64_t)my_k * a.dv_st + h * a.dv_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int d0 = db * 32 + 8 * rb + 4 * hf;
        store_grad4(a.dk, kro + d0, a.grad_f32, sc * dk[db][4 * rb], sc * dk[db][4 * rb + 1],
                    sc * dk[db][4 * rb + 2], sc * dk[db][4 * rb + 3]);
        store_grad4(a.dv, vro + d0, a.grad_f32, dv[db][4 * rb], dv[db][4 * rb + 1], dv[db][4 * rb + 2],
                    dv[db][4 * rb + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ: query-tile outer, key-tile inner
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BC = 64;                // keys per tile
  constexpr int BR = 32 * NW;           // queries per work-group
  constexpr int T = NW * 64;
  constexpr int DCH = D / 8;
  constexpr int KP = D + 8;
  constexpr int TP = BC + 8;
  constexpr int KS = BC * KP;
  constexpr int TS = D * TP;
  constexpr int STAGE = 2 * KS + TS;    // Ks | Vs | Kt (bf16)
  constexpr int KUNITS = (BC / 4) * DCH;
  constexpr int KU = (KUNITS + T - 1) / T;
  constexpr int VCH = (BC * DCH + T - 1) / T;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int ql = lane & 31, hf = lane >> 5;
  const int nq = a.nq, nk = a.nk, off = nk - nq;
  const int causal = a.causal, window = a.window;

  const int nqt = (nq + BR - 1) / BR;
  const int item = xcd_item(blockIdx.x, nqt * a.heads * a.batch);
  const int bh = item / nqt, t = item % nqt;
  const int qt = causal ? nqt - 1 - t : t;
  const int b = bh / a.heads, h = bh % a.heads;
  const int q0 = qt * BR;

  const uint16_t *qbase = (const uint16_t *)a.q + b * a.q_sb + h * a.q_sh;
  const uint16_t *dobase = (const uint16_t *)a.dout + b * a.do_sb + h * a.do_sh;
  const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_sb + h * a.k_sh;
  const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_sb + h * a.v_sh;
  const __amdgpu_buffer_rsrc_t qrs = slice_rsrc(qbase, slice_bytes(nq, a.q_st, D, 2));
  const __amdgpu_buffer_rsrc_t dors = slice_rsrc(dobase, slice_bytes(nq, a.do_st, D, 2));
  const __amdgpu_buffer_rsrc_t krs = slice_rsrc(kbase, slice_bytes(nk, a.k_st, D, 2));
  const __amdgpu_buffer_rsrc_t vrs = slice_rsrc(vbase, slice_bytes(nk, a.v_st, D, 2));
  const uint32_t kst2 = (uint32_t)a.k_st * 2, vst2 = (uint32_t)a.v_st * 2;

  const int p_lo = q0 + off, p_hi = min(q0 + BR, nq) - 1 + off;
  int kv_lo = 0, kv_hi = nk;
  if (causal) kv_hi = min(nk, p_hi + 1);
  if (window > 0) kv_lo = max(0, p_lo - window + 1);
  const int jt0 = kv_lo / BC;
  const int jt1 = kv_hi > kv_lo ? (kv_hi + BC - 1) / BC : jt0;

  const int wq0 = q0 + 32 * wave;
  const bool wave_rows = wq0 < nq;
  const int wp_lo = wq0 + off, wp_hi = min(wq0 + 31, nq - 1) + off;
  const int my_q = wq0 + ql;
  const int my_p = my_q + off;

  uint4 qreg[D / 16], doreg[D / 16];
  {
    const uint32_t qo = (uint32_t)my_q * (uint32_t)a.q_st * 2 + hf * 16;
    const uint32_t dqo = (uint32_t)my_q * (uint32_t)a.do_st * 2 + hf * 16;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qreg[kk] = bload16(qrs, qo + kk * 32);
      doreg[kk] = bload16(dors, dqo + kk * 32);
    }
  }
  float lse2 = INFINITY, dsum = 0.f;  // rows past the end or without visible keys: P = 0
  if (my_q < nq) {
    const float x = a.lse[(int64_t)bh * nq + my_q];
    if (x != -INFINITY) lse2 = x * kLog2e;
    dsum = a.dpsum[(int64_t)bh * nq + my_q];
  }

  uint4 ku[KU][4], vr[VCH];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + u * T;
      const int g = unit / DCH, dc = unit % DCH;
#pragma unroll
      for (int i = 0; i < 4; ++i) ku[u][i] = bload16(krs, (uint32_t)(k0 + 4 * g + i) * kst2 + dc * 16);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int cidx = tid + i * T;
      const int row = cidx / DCH, col = cidx % DCH;
      vr[i] = bload16(vrs, (uint32_t)(k0 + row) * vst2 + col * 16);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t *ks = smem + buf * STAGE;
    uint16_t *vs = ks + KS;
    uint16_t *kt = vs + KS;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + u * T;
      if (KU * T == KUNITS || unit < KUNITS) {
        const int g = unit / DCH, dc = unit % DCH;
#pragma unroll
        for (int i = 0; i < 4; ++i) *(uint4 *)(ks + (4 * g + i) * KP + dc * 8) = ku[u][i];
        store_transposed_4x8(kt, TP, dc * 8, vt_group_pos(g), ku[u]);
      }
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int cidx = tid + i * T;
      if (VCH * T == BC * DCH || cidx < BC * DCH) {
        const int row = cidx / DCH, col = cidx % DCH;
        *(uint4 *)(vs + row * KP + col * 8) = vr[i];
      }
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
  const float c = a.scale_log2;

  if (jt0 < jt1) {
    load_tile(jt0 * BC);
    store_tile(0);
  }
  __syncthreads();

  for (int jt = jt0; jt < jt1; ++jt) {
    const int buf = (jt - jt0) & 1;
    const int k0 = jt * BC;
    const bool more = jt + 1 < jt1;
    if (more) load_tile(k0 + BC);
    const uint16_t *ks = smem + buf * STAGE;
    const uint16_t *vs = ks + KS;
    const uint16_t *kt = vs + KS;

    const bool active = wave_rows && (!causal || k0 <= wp_hi) &&
                        (window <= 0 || k0 + BC - 1 > wp_lo - window);
    if (active) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = (f32x16){};
        dp[kb] = (f32x16){};
        const uint16_t *krow = ks + (kb * 32 + ql) * KP + hf * 8;
        const uint16_t *vrow = vs + (kb * 32 + ql) * KP + hf * 8;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          s[kb] = mfma_bf16(*(const uint4 *)(krow + kk * 16), qreg[kk], s[kb]);
          dp[kb] = mfma_bf16(*(const uint4 *)(vrow + kk * 16), doreg[kk], dp[kb]);
        }
      }
      const bool need_mask = (causal && k0 + BC - 1 > wp_lo) ||
                             (window > 0 && k0 <= wp_hi - window) || (k0 + BC > nk);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -lse2));
          if (need_mask) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = key < nk && (!causal || key <= my_p) && (window <= 0 || key > my_p - window);
            if (!ok) p = 0.f;
          }
          dp[kb][r] = p * (dp[kb][r] - dsum);
        }
      uint4 sb[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int kb = cc >> 1, r0 = (cc & 1) * 8;
        sb[cc].x = pack_bf16x2(dp[kb][r0 + 0], dp[kb][r0 + 1]);
        sb[cc].y = pack_bf16x2(dp[kb][r0 + 2], dp[kb][r0 + 3]);
        sb[cc].z = pack_bf16x2(dp[kb][r0 + 4], dp[kb][r0 + 5]);
        sb[cc].w = pack_bf16x2(dp[kb][r0 + 6], dp[kb][r0 + 7]);
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t *trow = kt + (db * 32 + ql) * TP + hf * 8;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) acc[db] = mfma_bf16(*(const uint4 *)(trow + cc * 16), sb[cc], acc[db]);
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // dQ = scale * dS K; lane = query, d = db*32 + 8*rb + 4*hf + 0..3
  if (my_q < nq) {
    const float sc = a.scale;
    const int64_t ro = b * a.dq_sb + (int64_t)my_q * a.dq_st + h * a.dq_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        store_grad4(a.dq, ro + db * 32 + 8 * rb + 4 * hf, a.grad_f32, sc * acc[db][4 * rb],
                    sc * acc[db][4 * rb + 1], sc * acc[db][4 * rb + 2], sc * acc[db][4 * rb + 3]);
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs &a, hipStream_t s) {
  constexpr int NW_KV = 4, NW_Q = 8;  // bwd_dkdv_kernel uses 4 waves
  const int64_t rows = (int64_t)a.batch * a.heads * a.nq;
  if (rows > 0) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_dsum_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, a);
  }
  const int64_t kv_items = (int64_t)((a.nk + 32 * NW_KV - 1) / (32 * NW_KV)) * a.heads * a.batch;
  if (kv_items > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)kv_items), dim3(NW_KV * 64), 0, s, a);
  const int64_t q_items = (int64_t)((a.nq + 32 * NW_Q - 1) / (32 * NW_Q)) * a.heads * a.batch;
  if (q_items > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW_Q>), dim3((unsigned)q_items), dim3(NW_Q * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int batch, int heads, int nq, int head_dim, int deterministic) {
  (void)head_dim;
  (void)deterministic;
  // D and LSE * log2(e), each [batch, heads, nq] fp32 rounded up to 256 bytes
  return 2 * (((size_t)batch * heads * nq * sizeof(float) + 255) / 256 * 256);
}

hipError_t launch_bwd_bf16(const BwdArgs &a, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_bwd_d<128>(a, s) : launch_bwd_d<64>(a, s);
}

}  // namespace fa
