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
// Four launches on the caller's stream:
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
//   4. bwd_start_kernel (causal only) the first kStartRows query rows of each
//      sequence, which see fewer than kStartRows keys, exactly in fp32.
// Splitting dQ from dK/dV costs the recomputation of S and dP a second time
// (7 tile products instead of 5) but needs no cross-work-group reduction, so
// the gradients are bitwise reproducible from call to call.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// Workspace of fa_bwd_noalloc, for callers that cannot allocate: D and
// LSE log2(e) of every query row (8 bytes per row of batch x heads x
// seqlen_q) live in this array, one copy per device, held until the process
// ends.  Host code must not pass `scratch` itself to a kernel (on the host
// it names a stand-in, not device memory): bwd_scratch() looks up the
// device address once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

hipError_t bwd_scratch(void **ptr) {
  static std::mutex mu;
  static void *addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

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

// Rows of a causal sequence that see fewer than this many keys (its first
// kStartRows positions) are computed by bwd_start_kernel in fp32.
constexpr int kStartRows = 64;
constexpr int kDsumRows = 4;  // rows per lane group of the D = rowsum(dO * O) kernel
constexpr int kDsumSeqs = 255;  // packed calls with up to this many sequences look them up in LDS

__device__ __forceinline__ float load_grad(const void *base, int64_t off, bool f32) {
  return f32 ? ((const float *)base)[off] : bf16_to_f32(((const uint16_t *)base)[off]);
}

// ---------------------------------------------------------------------------
// 1. D_i = sum_c dO_ic O_ic and LSE_i log2(e), laid out like the LSE
//    ([batch, heads, nq], or [heads, total_tokens] for packed sequences).
//    A row that saw no key (LSE = -inf) gets +inf, so P = 2^(s - lse2) = 0.
//    So does a row at the start of a causal sequence (fewer than
//    kStartRows visible keys): bwd_start_kernel does those rows exactly, and
//    the MFMA kernels then see P = 0 for them.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(BwdArgs a, int64_t total) {
  constexpr int LPR = D / 8;      // lanes per row, 8 bf16 each
  constexpr int GPB = 256 / LPR;  // lane groups per block
  // rows per lane group: their O and dO loads are all in flight at once
  // (one row per group left the kernel at 3.4-4.1 TB/s)
  constexpr int R = kDsumRows;
  const int tid = threadIdx.x, sub = tid % LPR;
  const int64_t row0 = ((int64_t)blockIdx.x * GPB + tid / LPR) * R;  // (b, h, q) or (h, token) order
  // packed causal calls: cu_seqlens staged in LDS (read together with the
  // rows' O and dO), so each row's sequence lookup costs no global round trip
  __shared__ int cus[kDsumSeqs + 1];
  const bool cu_lds = a.cu_seqlens && a.causal && a.batch <= kDsumSeqs;
  const int cu_mine = cu_lds && tid <= a.batch ? a.cu_seqlens[tid] : 0;
  uint4 ov[R], dv[R];
  int tok[R];  // packed calls: the row's token
  bool start_row[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
    ov[r] = dv[r] = uint4{0u, 0u, 0u, 0u};
    start_row[r] = false;
    tok[r] = -1;
    if (row < total) {
      int b = 0, h, q;  // q: token row of the tensors
      if (a.cu_seqlens) {
        const int ntok = (int)a.lse_sh;
        h = (int)(row / ntok);
        q = (int)(row % ntok);
        tok[r] = q;
      } else {
        q = (int)(row % a.nq);
        const int64_t bh = row / a.nq;
        h = (int)(bh % a.heads);
        b = (int)(bh / a.heads);
        const int pos = q + a.nk - a.nq;
        start_row[r] = a.causal && pos >= 0 && pos < kStartRows;
      }
      ov[r] = *(const uint4 *)((const uint16_t *)a.o + b * a.o_sb + (int64_t)q * a.o_st + h * a.o_sh + sub * 8);
      dv[r] = *(const uint4 *)((const uint16_t *)a.dout + b * a.do_sb + (int64_t)q * a.do_st + h * a.do_sh + sub * 8);
    }
  }
  // position of token q in its sequence s (cu[s] <= q < cu[s + 1]) below kStartRows
  auto starts = [&](const int *cu, int q) __attribute__((always_inline)) {
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= q) lo = mid;
      else hi = mid;
    }
    return q - cu[lo] < kStartRows;
  };
  if (cu_lds) {
    if (tid <= a.batch) cus[tid] = cu_mine;
    __syncthreads();  // uniform
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (tok[r] >= 0) start_row[r] = starts(cus, tok[r]);
  } else if (a.cu_seqlens && a.causal) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (tok[r] >= 0) start_row[r] = starts(a.cu_seqlens, tok[r]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc = __builtin_fmaf(bf16_to_f32(u16_at(ov[r], e)), bf16_to_f32(u16_at(dv[r], e)), acc);
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (row < total && sub == 0) {
      a.dpsum[row] = acc;
      const float x = a.lse[row];
      a.lse2[row] = (x == -INFINITY || start_row[r]) ? INFINITY : x * kLog2e;
    }
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
template <int D, bool DROP>
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
  // dropout: per wave, the keep bits of the tile's 64 query rows against the
  // wave's 32 keys (one word per row, bit = key)
  __shared__ __attribute__((aligned(16))) uint32_t drop_rec[DROP ? NW * 64 : 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hf = lane >> 5;
  const int causal = a.causal, window = a.window;

  // low key tiles (the most work under a causal mask) first
  const int nkt = (a.nk + BC - 1) / BC;
  int b, h, kt;
  fwd_item(blockIdx.x, nkt, a.heads, a.batch, a.cu_seqlens != nullptr, false, b, h, kt);
  int seq0 = 0, nq = a.nq, nk = a.nk;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    nq = nk = a.cu_seqlens[b + 1] - seq0;
  }
  const int k0 = kt * BC;
  if (k0 >= nk) return;  // uniform for the whole work-group
  const int off = nk - nq;
  const int wk0 = k0 + 32 * wave;
  const int my_k = wk0 + ql;
  // query rows (indices, not positions) that see this lane's key
  const VisRange vq = vis_range(causal ? (int64_t)my_k - off : 0,
                                min((int64_t)nq - 1, window > 0 ? (int64_t)my_k + window - 1 - off : (int64_t)INT32_MAX));

  const uint16_t *qbase = (const uint16_t *)a.q + b * a.q_sb + (int64_t)seq0 * a.q_st + h * a.q_sh;
  const uint16_t *dobase = (const uint16_t *)a.dout + b * a.do_sb + (int64_t)seq0 * a.do_st + h * a.do_sh;
  const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_sb + (int64_t)seq0 * a.k_st + h * a.k_sh;
  const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_sb + (int64_t)seq0 * a.v_st + h * a.v_sh;
  const int64_t lrow = b * a.lse_sb + h * a.lse_sh + seq0;
  const i32x4 qw = buffer_words(qbase, slice_bytes(nq, a.q_st, D, 2));
  const i32x4 dow = buffer_words(dobase, slice_bytes(nq, a.do_st, D, 2));
  const i32x4 lw = buffer_words(a.lse2 + lrow, (uint32_t)nq * 4);
  const i32x4 dw = buffer_words(a.dpsum + lrow, (uint32_t)nq * 4);
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

  // Dropout keep flags of this lane's 32 elements (bit e), for tile row q0.
  // The random bytes come in query-row order (one Philox call covers 16 keys
  // of one row), the lane needs them in key order: each lane makes the two
  // calls of row q0 + lane, packs the 32 flags into one word in LDS, and
  // reads back the words of the 32 rows it holds.
  const uint32_t dslot = (uint32_t)(b * a.heads + h);
  auto drop_mask = [&](int q0) __attribute__((always_inline)) -> uint32_t {
    const uint32_t kblk = (uint32_t)(k0 >> 5) + (uint32_t)wave, qi = (uint32_t)(q0 + lane);
    const Philox x0 = philox10(2u * kblk, qi, dslot, a.drop_offset, a.seed_lo, a.seed_hi);
    const Philox x1 = philox10(2u * kblk + 1u, qi, dslot, a.drop_offset, a.seed_lo, a.seed_hi);
    uint32_t rec = 0;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {  // key jj of the block: call (jj >> 2) & 1, element 4 (jj >> 3) + jj % 4
      const uint32_t w = ((jj >> 2) & 1) ? x1.c[jj >> 3] : x0.c[jj >> 3];
      rec |= (((w >> (8 * (jj & 3))) & 0xFFu) < a.drop_k ? 1u : 0u) << jj;
    }
    drop_rec[wave * 64 + lane] = rec;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's words are in LDS
    uint32_t em = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {  // rows 32 (g / 4) + 8 (g % 4) + 4 hf + 0..3
      const uint4 rr = *(const uint4 *)(drop_rec + wave * 64 + 32 * (g >> 2) + 8 * (g & 3) + 4 * hf);
      const int e0 = 16 * (g >> 2) + 4 * (g & 3);
      em |= ((rr.x >> ql) & 1u) << e0;
      em |= ((rr.y >> ql) & 1u) << (e0 + 1);
      em |= ((rr.z >> ql) & 1u) << (e0 + 2);
      em |= ((rr.w >> ql) & 1u) << (e0 + 3);
    }
    return em;
  };

  // P, dS of one tile (MASK: causal / window edge); element e = 16 qb + r is
  // query 32 qb + 8 (r / 4) + 4 hf + r % 4 of the tile
  auto one_tile = [&](auto mask_tag, int it) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int q0 = it * BR;
    if (it + 1 < it1) load_tile(it + 1);
    uint32_t emask = 0;
    if constexpr (DROP) emask = drop_mask(q0);
    // keep ? scale : 0 for element e (1 without dropout)
    auto kf = [&](int e) __attribute__((always_inline)) -> float {
      if constexpr (DROP) return ((emask >> e) & 1u) ? a.drop_scale : 0.f;
      else return 1.f;
    };
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
      const uint32_t vo = vis_offset(vq, q0 + 4 * hf);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!vis(vo, vq, qb * 32 + 8 * (r >> 2) + (r & 3))) s[qb][r] = -INFINITY;
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
      if constexpr (DROP)
        dp[e / 16][e % 16] =
            s[e / 16][e % 16] * __builtin_fmaf(dp[e / 16][e % 16], kf(e), -comp(d4[e / 4], e % 4));
      else
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
      if constexpr (DROP) {  // dV takes the dropped, rescaled P
#pragma unroll
        for (int r = r0; r < r0 + 8; ++r) s[qb][r] *= kf(16 * qb + r);
      }
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
    const int64_t kro = b * a.dk_sb + (int64_t)(seq0 + my_k) * a.dk_st + h * a.dk_sh;
    const int64_t vro = b * a.dv_sb + (int64_t)(seq0 + my_k) * a.dv_st + h * a.dv_sh;
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
// 3. dQ: query-tile outer, key-tile inner.  One work-group of 4 waves per
//    256 queries (64 per wave, two blocks of 32, one wave per SIMD); key
//    tiles of 64 arrive by LDS DMA one tile ahead (three buffers each for K
//    and V, unpadded, XOR-swizzled) and are processed as two sub-tiles of 32.
//    Per sub-tile u:
//      phase A: S^T = K Q^T and dP^T = V dO^T for both query blocks (each K
//               or V row fragment feeds two MFMAs; Q^T, dO^T are B operands
//               held in AGPRs; lane = query, so LSE and D are per-lane
//               scalars), with the VALU turning S, dP of sub-tile u-1 into
//               dS = 2^(s c - lse2) (dP - D) and packing it to bf16;
//      phase B: dQ^T += K^T dS^T for sub-tile u-1 (K^T read transposed from
//               the row-major K tile, in the key order of the dS^T operand).
//    dQ is written once, no atomics.
// ---------------------------------------------------------------------------
template <int D, bool DROP>
__device__ __forceinline__ void dq_item(const BwdArgs &a, int b, int h, int qt) {
  constexpr int NW = 4, T = NW * 64, QW = 64, BR = NW * QW, BC = 64;
  constexpr int DCH = D / 8, TS = BC * D;
  constexpr int PER = BC * DCH / T;  // DMA loads per lane per tile and tensor
  constexpr int NK = D / 16;         // d-steps of S and dP (fragments per sub-tile and tensor)
  constexpr int NF = (D / 32) * 2;   // phase-B K^T fragments per sub-tile
  constexpr int RING = 6;
  __shared__ __attribute__((aligned(16))) uint16_t smem[6 * TS];  // K x3, V x3

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hf = lane >> 5;
  const int causal = a.causal, window = a.window;

  int seq0 = 0, nq = a.nq, nk = a.nk;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    nq = nk = a.cu_seqlens[b + 1] - seq0;
  }
  const int q0 = qt * BR;
  if (q0 >= nq) return;  // uniform for the whole work-group
  const int off = nk - nq;

  const uint16_t *qbase = (const uint16_t *)a.q + b * a.q_sb + (int64_t)seq0 * a.q_st + h * a.q_sh;
  const uint16_t *dobase = (const uint16_t *)a.dout + b * a.do_sb + (int64_t)seq0 * a.do_st + h * a.do_sh;
  const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_sb + (int64_t)seq0 * a.k_st + h * a.k_sh;
  const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_sb + (int64_t)seq0 * a.v_st + h * a.v_sh;
  const int64_t lrow = b * a.lse_sb + h * a.lse_sh + seq0;
  const __amdgpu_buffer_rsrc_t qrs = slice_rsrc(qbase, slice_bytes(nq, a.q_st, D, 2));
  const __amdgpu_buffer_rsrc_t dors = slice_rsrc(dobase, slice_bytes(nq, a.do_st, D, 2));
  const i32x4 kw = buffer_words(kbase, slice_bytes(nk, a.k_st, D, 2));
  const i32x4 vw = buffer_words(vbase, slice_bytes(nk, a.v_st, D, 2));
  const uint32_t kst2 = (uint32_t)a.k_st * 2, vst2 = (uint32_t)a.v_st * 2;

  const int p_lo = q0 + off, p_hi = min(q0 + BR, nq) - 1 + off;
  int kv_lo = 0, kv_hi = nk;
  if (causal) kv_hi = min(nk, p_hi + 1);
  if (window > 0) kv_lo = max(0, p_lo - window + 1);
  const int jt0 = kv_lo / BC;
  const int jt1 = kv_hi > kv_lo ? (kv_hi + BC - 1) / BC : jt0;

  const int wq0 = q0 + QW * wave;
  const bool wave_rows = wq0 < nq;
  const int wp_lo = wq0 + off, wp_hi = min(wq0 + QW - 1, nq - 1) + off;
  // keys that this lane's two query rows see (no length limit: past the end
  // K loads as zero rows, so those keys add nothing to dQ)
  VisRange vk[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int my_p = wq0 + 32 * qb + ql + off;
    vk[qb] = vis_range(window > 0 ? (int64_t)my_p - window + 1 : 0, causal ? (int64_t)my_p : (int64_t)INT32_MAX);
  }
  auto active = [&](int k0) __attribute__((always_inline)) {  // 32 keys from k0
    return wave_rows && (!causal || k0 <= wp_hi) && (window <= 0 || k0 + 31 > wp_lo - window);
  };

  const uint32_t lds0 = lds_addr(smem);
  auto slot = [&](int jt) __attribute__((always_inline)) { return (jt - jt0) % 3; };
  auto kbuf = [&](int jt) __attribute__((always_inline)) { return smem + slot(jt) * TS; };
  auto vbuf = [&](int jt) __attribute__((always_inline)) { return smem + (3 + slot(jt)) * TS; };
  uint32_t kgo[PER], vgo[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int sl = i * T + tid, r = sl / DCH, lc = (sl % DCH) ^ swz<D>(r);
    kgo[i] = (uint32_t)r * kst2 + lc * 16;
    vgo[i] = (uint32_t)r * vst2 + lc * 16;
  }
  auto load_kv = [&](int jt) __attribute__((always_inline)) {
    const uint32_t gk = (uint32_t)(jt * BC) * kst2, gv = (uint32_t)(jt * BC) * vst2;
    const uint32_t lk = lds0 + (uint32_t)(slot(jt) * TS * 2 + wave * 1024);
    const uint32_t lv = lds0 + (uint32_t)((3 + slot(jt)) * TS * 2 + wave * 1024);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      dma16_at(kw, lk + i * T * 16, gk + kgo[i]);
      dma16_at(vw, lv + i * T * 16, gv + vgo[i]);
    }
  };

  // Q^T and dO^T of both query blocks: B operands for the whole loop (AGPRs)
  u32x4 qreg[2][NK], doreg[2][NK];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const uint32_t r = (uint32_t)(wq0 + 32 * qb + ql);
    const uint32_t qo = r * (uint32_t)a.q_st * 2 + hf * 16, dqo = r * (uint32_t)a.do_st * 2 + hf * 16;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      qreg[qb][kk] = vec4(bload16(qrs, qo + kk * 32));
      doreg[qb][kk] = vec4(bload16(dors, dqo + kk * 32));
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) asm volatile("s_nop 1" : "+a"(qreg[qb][kk]), "+a"(doreg[qb][kk]));
  // per-lane LSE*log2(e) and D of the lane's two query rows
  float lse2[2], dsum[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int my_q = wq0 + 32 * qb + ql;
    lse2[qb] = INFINITY;  // rows past the end: P = 0
    dsum[qb] = 0.f;
    if (my_q < nq) {
      lse2[qb] = a.lse2[lrow + my_q];
      dsum[qb] = a.dpsum[lrow + my_q];
    }
  }

  f32x16 acc[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[qb][i] = (f32x16){};
  const float c = a.scale_log2;
  f32x16 s[2], dp[2];          // [query block]: S^T then P; dP^T then dS; lane = query
  uint4 sb[2][2];              // bf16 dS^T of the pending sub-tile, [query block][16-key half]
  const uint16_t *k_p = smem;  // K rows of the pending sub-tile
  // the pending sub-tile before the first one has dS = 0
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) dp[qb] = (f32x16){};

  // dropout: the keep bytes of a sub-tile's 32 keys for the lane's two query
  // rows, one Philox call each; its 10 rounds are spread over the 2 NK
  // stages of the S and dP MFMAs, round r at stage r * 2 NK / 10
  const uint32_t dslot = (uint32_t)(b * a.heads + h);
  Philox rx[2];
  auto drop_rounds = [&](int stage) __attribute__((always_inline)) {
    if constexpr (DROP) {
#pragma unroll
      for (int r = 0; r < 10; ++r)
        if (r * 2 * NK / 10 == stage) {
          philox_round(rx[0], philox_k0(a.seed_lo, r), philox_k1(a.seed_hi, r));
          philox_round(rx[1], philox_k0(a.seed_lo, r), philox_k1(a.seed_hi, r));
        }
    }
  };
  // dS = P (dP keep scale - D) for DROP (kf = keep ? scale : 0), else P (dP - D)
  auto kfac = [&](int qb, int r) __attribute__((always_inline)) -> float {
    if constexpr (DROP) return drop_keep(rx[qb], r, a.drop_k) ? a.drop_scale : 0.f;
    else return 1.f;
  };

  const int kx = hf ^ swz<D>(ql);
  // phase-A fragment kk of sub-tile (jt, kb): K rows (S) or V rows (dP)
  auto kread = [&](int jt, int kb, int kk) __attribute__((always_inline)) -> uint4 {
    return *(const uint4 *)(kbuf(jt) + (kb * 32 + ql) * D + (((2 * kk) ^ kx) << 3));
  };
  auto vread = [&](int jt, int kb, int kk) __attribute__((always_inline)) -> uint4 {
    return *(const uint4 *)(vbuf(jt) + (kb * 32 + ql) * D + (((2 * kk) ^ kx) << 3));
  };
  // phase-B fragment f = (db = f / 2, h2 = f % 2) of K^T for the 32 K rows at ks
  auto bread = [&](const uint16_t *ks, int f) __attribute__((always_inline)) -> uint4 {
    const uint16_t *kp = ks + (f % 2) * 16 * D;
    const uint2 lo = lds_read_tr16(kp + tr_off<D>(lane, f / 2, 0));
    const uint2 hi = lds_read_tr16(kp + tr_off<D>(lane, f / 2, 1));
    return (uint4){lo.x, lo.y, hi.x, hi.y};
  };
  // element e of query block qb is key 8 (e / 4) + 4 hf + e % 4 of the sub-tile
  auto pack_ds = [&](int qb, int h2) __attribute__((always_inline)) {
    const int r0 = h2 * 8;
    uint4 &w = sb[qb][h2];
    w.x = pack_bf16x2(dp[qb][r0 + 0], dp[qb][r0 + 1]);
    w.y = pack_bf16x2(dp[qb][r0 + 2], dp[qb][r0 + 3]);
    w.z = pack_bf16x2(dp[qb][r0 + 4], dp[qb][r0 + 5]);
    w.w = pack_bf16x2(dp[qb][r0 + 6], dp[qb][r0 + 7]);
    asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));  // keep the work in its stage
  };

  auto sub = [&](auto mask_tag, int jt, int kb) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = jt * BC + kb * 32;
    const bool act = !MASK || active(k0);
    if constexpr (DROP) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        rx[qb].c[0] = 2u * (uint32_t)(k0 >> 5) + (uint32_t)hf;
        rx[qb].c[1] = (uint32_t)(wq0 + 32 * qb + ql);
        rx[qb].c[2] = dslot;
        rx[qb].c[3] = a.drop_offset;
      }
    }
    // ---- S MFMAs; meanwhile dS of the pending sub-tile is packed to bf16
    if (act) {
      uint4 ring[RING];
#pragma unroll
      for (int j = 0; j < RING; ++j) ring[j] = kread(jt, kb, j);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const uint4 f = ring[kk % RING];
        if (kk + RING < NK) ring[kk % RING] = kread(jt, kb, kk + RING);
        if (kk == 0) {
          mfma_v_first(s[0], f, qreg[0][0]);
          mfma_v_first(s[1], f, qreg[1][0]);
        } else {
          mfma_v(s[0], f, qreg[0][kk]);
          mfma_v(s[1], f, qreg[1][kk]);
        }
        constexpr int PK = NK / 4;
        if (kk % PK == PK - 1) pack_ds((kk / PK) / 2, (kk / PK) % 2);
        drop_rounds(kk);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_drain2_v(s[0], s[1]);
    } else {
#pragma unroll
      for (int part = 0; part < 4; ++part) pack_ds(part / 2, part % 2);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) drop_rounds(kk);
      // S = -inf for a sub-tile these rows do not see.  Written by volatile asm
      // so that the compiler keeps the 32 moves on this path: as plain
      // assignments it hoisted them above the branch, onto the visible path.
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x0, x1;
        asm volatile("v_mov_b32 %0, 0xff800000" : "=v"(x0));
        asm volatile("v_mov_b32 %0, 0xff800000" : "=v"(x1));
        s[0][e] = x0;
        s[1][e] = x1;
      }
    }
    if (MASK) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const uint32_t vo = vis_offset(vk[qb], k0 + 4 * hf);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (!vis(vo, vk[qb], 8 * (e >> 2) + (e & 3))) s[qb][e] = -INFINITY;
      }
    }
    // ---- dP MFMAs; meanwhile P = 2^(s c - lse2) in place
    __builtin_amdgcn_sched_barrier(0);
    {
      uint4 ring[RING];
      if (act) {
#pragma unroll
        for (int j = 0; j < RING; ++j) ring[j] = vread(jt, kb, j);
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        if (act) {
          const uint4 f = ring[kk % RING];
          if (kk + RING < NK) ring[kk % RING] = vread(jt, kb, kk + RING);
          if (kk == 0) {
            mfma_v_first(dp[0], f, doreg[0][0]);
            mfma_v_first(dp[1], f, doreg[1][0]);
          } else {
            mfma_v(dp[0], f, doreg[0][kk]);
            mfma_v(dp[1], f, doreg[1][kk]);
          }
        }
        constexpr int EPS = 32 / NK;
#pragma unroll
        for (int k = 0; k < EPS; ++k) {
          const int e = kk * EPS + k, qb = e / 16, r = e % 16;
          s[qb][r] = fast_exp2(__builtin_fmaf(s[qb][r], c, -lse2[qb]));
        }
        drop_rounds(NK + kk);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (act) mfma_drain2_v(dp[0], dp[1]);
    }
    // ---- dQ^T += K^T dS^T of the pending sub-tile; meanwhile dS = P (dP - D)
    {
      uint4 ring[RING];
#pragma unroll
      for (int j = 0; j < RING; ++j) ring[j] = bread(k_p, j);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const uint4 kf = ring[f % RING];
        if (f + RING < NF) ring[f % RING] = bread(k_p, f + RING);
        mfma_a(acc[0][f / 2], kf, sb[0][f % 2]);
        mfma_a(acc[1][f / 2], kf, sb[1][f % 2]);
        constexpr int EPS = 32 / NF;
#pragma unroll
        for (int k = 0; k < EPS; ++k) {
          const int e = f * EPS + k, qb = e / 16, r = e % 16;
          if (act) dp[qb][r] = s[qb][r] * (DROP ? __builtin_fmaf(dp[qb][r], kfac(qb, r), -dsum[qb]) : dp[qb][r] - dsum[qb]);
          else dp[qb][r] = 0.f;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    k_p = kbuf(jt) + kb * 32 * D;
  };
  auto step = [&](auto mask_tag, int jt) __attribute__((always_inline)) {
    if (jt + 1 < jt1) load_kv(jt + 1);
    sub(mask_tag, jt, 0);
    sub(mask_tag, jt, 1);
    wait_dma();
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < D / 32; ++i) asm volatile("" : "+a"(acc[qb][i]));
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < D / 32; ++i) asm volatile("" : "+a"(acc[qb][i]));
  };

  int ja = jt0, jb = jt1;
  if (window > 0) {
    const int lim = p_hi - window;
    ja = lim >= 0 ? min(jt1, max(jt0, lim / BC + 1)) : jt0;
  }
  if (causal) {
    const int lim = p_lo - (BC - 1);
    jb = lim >= 0 ? max(ja, min(jt1, lim / BC + 1)) : ja;
  }

  if (jt0 < jt1) load_kv(jt0);
  wait_dma();
  __syncthreads();
  k_p = kbuf(jt0);
  const std::true_type masked;
  const std::false_type whole;
  for (int jt = jt0; jt < ja; ++jt) step(masked, jt);
  for (int jt = ja; jt < jb; ++jt) step(whole, jt);
  for (int jt = jb; jt < jt1; ++jt) step(masked, jt);
  if (jt0 < jt1) {
    // the last sub-tile's product
#pragma unroll
    for (int part = 0; part < 4; ++part) pack_ds(part / 2, part % 2);
    asm volatile("s_nop 1");
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint4 kf = bread(k_p, f);
      mfma_a(acc[0][f / 2], kf, sb[0][f % 2]);
      mfma_a(acc[1][f / 2], kf, sb[1][f % 2]);
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < D / 32; ++i) mfma_drain_a(acc[qb][i]);

  // dQ = scale * dS K; lane = query, d = db*32 + 8*rb + 4*hf + 0..3
  const float sc = a.scale;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int my_q = wq0 + 32 * qb + ql;
    if (my_q < nq) {
      const int64_t ro = b * a.dq_sb + (int64_t)(seq0 + my_q) * a.dq_st + h * a.dq_sh;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          store_grad4(a.dq, ro + db * 32 + 8 * rb + 4 * hf, a.grad_f32, sc * acc[qb][db][4 * rb],
                      sc * acc[qb][db][4 * rb + 1], sc * acc[qb][db][4 * rb + 2], sc * acc[qb][db][4 * rb + 3]);
    }
  }
}
// dQ items: query tiles of 256, high ones carry the most work under a causal
// mask.  Dense calls with at least one unit per CU run persistently (see
// launch_units), packed calls with up to kPackedSeqs sequences on the
// schedule built from cu_seqlens (persist 2); the item body is called from one
// place, on the kernel's own by-value argument block (a reference to it would
// push it to scratch).
template <int D, bool DROP>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a) {
  __shared__ int s_key[kPackedSeqs], s_order[kPackedSeqs], s_first[kPackedSeqs + 2];
  const int nqt = (a.nq + 255) / 256;
  const bool varlen = a.cu_seqlens != nullptr;
  const bool packed = a.persist == 2;
  PackedSchedule ps{s_key, s_order, s_first, a.batch, a.heads};
  if (packed) packed_schedule_build(ps, a.cu_seqlens, 256, a.causal, a.window);
  const UnitRange r = launch_units(a.persist == 1, a.batch, a.heads, nqt, a.causal);
  for (int i = 0;; ++i) {
    int b, h, qt;
    if (packed) {
      const int st = packed_schedule_item(ps, i, a.causal, b, h, qt);
      if (st < 0) break;
      if (st == 0) continue;
    } else {
      const int u = r.lo + (i >> 1) * r.step;
      if (u >= r.hi) break;
      if (!launch_tile(a.persist == 1, r, u, i & 1, a.batch, a.heads, nqt, varlen, a.causal, false, b, h, qt))
        continue;
    }
    dq_item<D, DROP>(a, b, h, qt);
    lds_barrier();  // the next item's DMA reuses the LDS tiles
  }
}


// ---------------------------------------------------------------------------
// 4. The start of every causal sequence: query rows at positions p with
//    p + (Nk - Nq) < kStartRows, whose visible keys all lie among the first
//    kStartRows keys.  One work-group per (sequence, head) does this
//    kStartRows x kStartRows block in fp32: the softmax of each row over all
//    of its keys, D_i = sum_j P_ij dP_ij, dS = P (dP - D), then writes dQ of
//    these rows and adds their contributions to dK and dV of the first keys.
//    Runs after the MFMA kernels, which skipped these rows (lse2 = +inf).
//    With few keys, P is concentrated and |dS| large; the bf16 dS operand
//    and a D taken from the bf16 O would then cost these rows most of the
//    accuracy the gradients have elsewhere.
// ---------------------------------------------------------------------------
// work-groups per (sequence, head), each 1/4 of the head dims; one work-group
// per pair (4x the fp32 work each) measured no faster on the 11-sequence
// packed backward, which launches 308 pairs
constexpr int kStartSplit = 4;

template <int D>
__global__ __launch_bounds__(256) void bwd_start_kernel(BwdArgs a) {
  constexpr int T = kStartRows, PITCH = D + 8, DCH = D / 8;  // bf16 row pitch (16-byte multiple)
  constexpr int DS = D / kStartSplit;                         // head dims of this work-group's outputs
  constexpr int G = DS / 4, RG = 256 / G, RPT = T / RG;       // 4 dims x RPT rows per thread
  __shared__ __attribute__((aligned(16))) uint16_t qs[T * PITCH], dos[T * PITCH], ks[T * PITCH], vs[T * PITCH];
  __shared__ float ps[T][T + 1], dss[T][T + 1];  // S then P; dP then dS
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / kStartSplit, sp = blockIdx.x % kStartSplit;
  const int b = bh / a.heads, h = bh % a.heads;
  int seq0 = 0, nq = a.nq, nk = a.nk;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    nq = nk = a.cu_seqlens[b + 1] - seq0;
  }
  const int off = nk - nq;
  // local row r is query r - off: its last visible key is key r
  const int r_lo = max(0, off), r_hi = min(T, nq + off), kn = min(nk, T);
  if (r_lo >= r_hi || kn <= 0) return;  // uniform: no start rows here
  const int window = a.window;
  const float scale = a.scale;
  const uint32_t dslot = (uint32_t)(b * a.heads + h);

  const uint16_t *qg = (const uint16_t *)a.q + b * a.q_sb + h * a.q_sh;
  const uint16_t *dog = (const uint16_t *)a.dout + b * a.do_sb + h * a.do_sh;
  const uint16_t *kg = (const uint16_t *)a.k + b * a.k_sb + h * a.k_sh;
  const uint16_t *vg = (const uint16_t *)a.v + b * a.v_sb + h * a.v_sh;
  for (int idx = tid; idx < T * DCH; idx += 256) {
    const int r = idx / DCH, ch = idx % DCH;
    uint4 q4 = {0u, 0u, 0u, 0u}, o4 = q4, k4 = q4, v4 = q4;
    if (r >= r_lo && r < r_hi) {
      const int64_t t = seq0 + r - off;
      q4 = *(const uint4 *)(qg + t * a.q_st + ch * 8);
      o4 = *(const uint4 *)(dog + t * a.do_st + ch * 8);
    }
    if (r < kn) {
      const int64_t t = seq0 + r;
      k4 = *(const uint4 *)(kg + t * a.k_st + ch * 8);
      v4 = *(const uint4 *)(vg + t * a.v_st + ch * 8);
    }
    *(uint4 *)(qs + r * PITCH + ch * 8) = q4;
    *(uint4 *)(dos + r * PITCH + ch * 8) = o4;
    *(uint4 *)(ks + r * PITCH + ch * 8) = k4;
    *(uint4 *)(vs + r * PITCH + ch * 8) = v4;
  }
  __syncthreads();

  // S = Q K^T and dP = dO V^T on MFMA (exact bf16 products, fp32 sums): wave
  // w owns the 32 x 32 block of rows 32 (w / 2), keys 32 (w % 2)
  {
    const int r0 = 32 * (wave >> 1), c0 = 32 * (wave & 1), l32 = lane & 31, hf = lane >> 5;
    f32x16 sacc = {}, dacc = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int col = kk * 16 + hf * 8;
      sacc = mfma_bf16(*(const uint4 *)(qs + (r0 + l32) * PITCH + col), *(const uint4 *)(ks + (c0 + l32) * PITCH + col),
                       sacc);
      dacc = mfma_bf16(*(const uint4 *)(dos + (r0 + l32) * PITCH + col),
                       *(const uint4 *)(vs + (c0 + l32) * PITCH + col), dacc);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = r0 + 8 * (i / 4) + 4 * hf + i % 4;
      ps[r][c0 + l32] = sacc[i] * scale;
      dss[r][c0 + l32] = dacc[i];
    }
  }
  __syncthreads();

  // per row r = tid / 4 (keys c = tid % 4 + 4 j): softmax over the row's
  // visible keys, D = sum_j P dP, dS = P (dP - D); sums across the 4 lanes
  {
    const int r = tid >> 2, part = tid & 3;
    const bool row_ok = r >= r_lo && r < r_hi;
    float sv[T / 4], m = -INFINITY;
#pragma unroll
    for (int j = 0; j < T / 4; ++j) {
      const int c = part + 4 * j;
      const bool vis = row_ok && c < kn && c <= r && (window <= 0 || c > r - window);
      sv[j] = vis ? ps[r][c] : -INFINITY;
      m = fmaxf(m, sv[j]);
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < T / 4; ++j) {
      sv[j] = sv[j] == -INFINITY ? 0.f : expf(sv[j] - m);
      l += sv[j];
    }
    l += __shfl_xor(l, 1);
    l += __shfl_xor(l, 2);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // dropout: kf = keep ? scale : 0 per key (keys c < 64: blocks 0, 1)
    float kfv[T / 4];
#pragma unroll
    for (int j = 0; j < T / 4; ++j) kfv[j] = 1.f;
    if (a.drop_k) {
      const uint32_t qi = (uint32_t)(r - off);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const Philox x = philox10(2u * cb + hh, qi, dslot, a.drop_offset, a.seed_lo, a.seed_hi);
#pragma unroll
          for (int j = 0; j < T / 4; ++j) {
            const int c = part + 4 * j;  // (c >> 2) & 1 == j & 1, c >> 5 == j >> 3
            if ((j >> 3) == cb && (j & 1) == hh) {
              const uint32_t byte = (x.c[(c & 31) >> 3] >> (8 * (c & 3))) & 0xFFu;
              kfv[j] = byte < a.drop_k ? a.drop_scale : 0.f;
            }
          }
        }
    }
    float dd = 0.f;  // D = sum_j P_j kf_j dP_j
#pragma unroll
    for (int j = 0; j < T / 4; ++j) {
      sv[j] *= inv;
      dd = __builtin_fmaf(sv[j] * kfv[j], dss[r][part + 4 * j], dd);
    }
    dd += __shfl_xor(dd, 1);
    dd += __shfl_xor(dd, 2);
#pragma unroll
    for (int j = 0; j < T / 4; ++j) {
      const int c = part + 4 * j;
      dss[r][c] = sv[j] * __builtin_fmaf(kfv[j], dss[r][c], -dd);  // 0 where P = 0
      ps[r][c] = sv[j] * kfv[j];
    }
  }
  __syncthreads();

  // dQ of the start rows (written: the MFMA kernels left them zero) and their
  // share of dK, dV of the first keys (added to what those kernels wrote),
  // in fp32; dims d0..d0+3 of this work-group's slice, rows / keys tg + RG i
  const int d0 = sp * DS + 4 * (tid % G), tg = tid / G;
  auto bf4 = [](uint2 w, float (&x)[4]) __attribute__((always_inline)) {
    x[0] = bf16_to_f32(w.x & 0xffffu);
    x[1] = bf16_to_f32(w.x >> 16);
    x[2] = bf16_to_f32(w.y & 0xffffu);
    x[3] = bf16_to_f32(w.y >> 16);
  };
  {
    float acc[RPT][4] = {};
#pragma unroll 8
    for (int c = 0; c < kn; ++c) {
      float kx[4];
      bf4(*(const uint2 *)(ks + c * PITCH + d0), kx);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float ds = dss[tg + RG * i][c];
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[i][x] = __builtin_fmaf(ds, kx[x], acc[i][x]);
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = tg + RG * i;
      if (r >= r_lo && r < r_hi)
        store_grad4(a.dq, b * a.dq_sb + (int64_t)(seq0 + r - off) * a.dq_st + h * a.dq_sh + d0, a.grad_f32,
                    scale * acc[i][0], scale * acc[i][1], scale * acc[i][2], scale * acc[i][3]);
    }
  }
  {
    float gk[RPT][4] = {}, gv[RPT][4] = {};
#pragma unroll 8
    for (int r = r_lo; r < r_hi; ++r) {
      float qx[4], ox[4];
      bf4(*(const uint2 *)(qs + r * PITCH + d0), qx);
      bf4(*(const uint2 *)(dos + r * PITCH + d0), ox);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float ds = dss[r][tg + RG * i], p = ps[r][tg + RG * i];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          gk[i][x] = __builtin_fmaf(ds, qx[x], gk[i][x]);
          gv[i][x] = __builtin_fmaf(p, ox[x], gv[i][x]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = tg + RG * i;
      if (c < kn) {
        const int64_t ko = b * a.dk_sb + (int64_t)(seq0 + c) * a.dk_st + h * a.dk_sh + d0;
        const int64_t vo = b * a.dv_sb + (int64_t)(seq0 + c) * a.dv_st + h * a.dv_sh + d0;
        float k4[4], v4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          k4[x] = load_grad(a.dk, ko + x, a.grad_f32) + scale * gk[i][x];
          v4[x] = load_grad(a.dv, vo + x, a.grad_f32) + gv[i][x];
        }
        store_grad4(a.dk, ko, a.grad_f32, k4[0], k4[1], k4[2], k4[3]);
        store_grad4(a.dv, vo, a.grad_f32, v4[0], v4[1], v4[2], v4[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 5. Causal mask with a sliding window of at most kBandMax keys: every query
//    row then sees at most kBandMax keys, all among the kBandMax - 1
//    positions before it.  Such rows' probabilities can sit on a few keys,
//    where the bf16 P and dS operands of the MFMA kernels (and a D taken
//    from the bf16 O) cost most of the accuracy the gradients have elsewhere,
//    as at the causal start rows.  These calls run two exact fp32 kernels
//    instead of kernels 1-4:
//      bwd_band_dq_kernel    32 query rows against the aligned slab of 128
//                            keys (four 32-key blocks) that holds all their
//                            visible keys: each row's softmax over its keys,
//                            D_i = sum_j P_ij dP_ij, dS = P (dP - D), dQ; the
//                            row's D and log-sum-exp go to the workspace.
//      bwd_band_dkdv_kernel  32 keys against the 128 query rows from their
//                            first position on (all rows that can see them):
//                            P from that log-sum-exp, dS with that D, dK, dV.
//    S and dP come from MFMA on the bf16 operands (exact products, fp32
//    sums); everything after them is fp32, and no output is shared between
//    work-groups.
// ---------------------------------------------------------------------------
constexpr int kBandMax = 64;
constexpr int kBandRows = 32;   // query rows (dQ kernel) or keys (dK/dV kernel) per work-group
constexpr int kBandSlab = 128;  // keys (dQ kernel) or query rows (dK/dV kernel) staged against them

// bf16 x 4 (8 bytes) to fp32
__device__ __forceinline__ void band_bf4(uint2 w, float (&x)[4]) {
  x[0] = bf16_to_f32(w.x & 0xffffu);
  x[1] = bf16_to_f32(w.x >> 16);
  x[2] = bf16_to_f32(w.y & 0xffffu);
  x[3] = bf16_to_f32(w.y >> 16);
}

// S = A B^T and dP = C E^T of one 32 x 32 block on MFMA: rows 32 ra.. of the
// row-major LDS tiles a (for S) and c (for dP), columns 32 rb.. from the
// tiles b and e; results into s_out / dp_out [row][col] (pitch P floats).
template <int D, int PITCH, int P>
__device__ __forceinline__ void band_block(const uint16_t *a, const uint16_t *bt, const uint16_t *c,
                                           const uint16_t *e, int ra, int rb, float *s_out, float *dp_out,
                                           int lane) {
  const int l32 = lane & 31, hf = lane >> 5;
  f32x16 sacc = {}, dacc = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const int col = kk * 16 + hf * 8;
    sacc = mfma_bf16(*(const uint4 *)(a + (32 * ra + l32) * PITCH + col),
                     *(const uint4 *)(bt + (32 * rb + l32) * PITCH + col), sacc);
    dacc = mfma_bf16(*(const uint4 *)(c + (32 * ra + l32) * PITCH + col),
                     *(const uint4 *)(e + (32 * rb + l32) * PITCH + col), dacc);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 32 * ra + 8 * (i / 4) + 4 * hf + i % 4;
    s_out[r * P + 32 * rb + l32] = sacc[i];
    dp_out[r * P + 32 * rb + l32] = dacc[i];
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_band_dq_kernel(BwdArgs a) {
  constexpr int R = kBandRows, K = kBandSlab, PITCH = D + 8, DCH = D / 8, SP = K + 1;
  constexpr int G = D / 4, RG = 256 / G, RPT = R / RG;  // dQ: 4 dims x RPT rows per thread
  static_assert(RPT * RG == R, "row split");
  __shared__ __attribute__((aligned(16))) uint16_t qs[R * PITCH], dos[R * PITCH], ks[K * PITCH], vs[K * PITCH];
  __shared__ float ss[R * SP], dps[R * SP];  // S; dP then dS
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nqt = (a.nq + R - 1) / R;
  const int qt = blockIdx.x % nqt, bh = blockIdx.x / nqt;
  const int b = bh / a.heads, h = bh % a.heads;
  int seq0 = 0, nq = a.nq, nk = a.nk;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    nq = nk = a.cu_seqlens[b + 1] - seq0;
  }
  const int q0 = qt * R;
  if (q0 >= nq) return;  // uniform
  const int off = nk - nq, window = a.window;
  const int p0 = q0 + off;                   // key position of row q0
  const int ks0 = (p0 - (kBandMax - 1)) & ~31;  // slab [ks0, ks0 + K): 32-aligned, holds [p0 - 63, p0 + 31]
  const float scale = a.scale;

  const uint16_t *qg = (const uint16_t *)a.q + b * a.q_sb + (int64_t)seq0 * a.q_st + h * a.q_sh;
  const uint16_t *dog = (const uint16_t *)a.dout + b * a.do_sb + (int64_t)seq0 * a.do_st + h * a.do_sh;
  const uint16_t *kg = (const uint16_t *)a.k + b * a.k_sb + (int64_t)seq0 * a.k_st + h * a.k_sh;
  const uint16_t *vg = (const uint16_t *)a.v + b * a.v_sb + (int64_t)seq0 * a.v_st + h * a.v_sh;
  for (int idx = tid; idx < R * DCH; idx += 256) {
    const int r = idx / DCH, ch = idx % DCH;
    uint4 q4 = {0u, 0u, 0u, 0u}, o4 = q4;
    if (q0 + r < nq) {
      q4 = *(const uint4 *)(qg + (int64_t)(q0 + r) * a.q_st + ch * 8);
      o4 = *(const uint4 *)(dog + (int64_t)(q0 + r) * a.do_st + ch * 8);
    }
    *(uint4 *)(qs + r * PITCH + ch * 8) = q4;
    *(uint4 *)(dos + r * PITCH + ch * 8) = o4;
  }
  for (int idx = tid; idx < K * DCH; idx += 256) {
    const int c = idx / DCH, ch = idx % DCH, j = ks0 + c;
    uint4 k4 = {0u, 0u, 0u, 0u}, v4 = k4;
    if (j >= 0 && j < nk) {
      k4 = *(const uint4 *)(kg + (int64_t)j * a.k_st + ch * 8);
      v4 = *(const uint4 *)(vg + (int64_t)j * a.v_st + ch * 8);
    }
    *(uint4 *)(ks + c * PITCH + ch * 8) = k4;
    *(uint4 *)(vs + c * PITCH + ch * 8) = v4;
  }
  __syncthreads();
  // wave w: rows 0..31 against keys 32 w..32 w + 31
  band_block<D, PITCH, SP>(qs, ks, dos, vs, 0, wave, ss, dps, lane);
  __syncthreads();

  // row r, Philox call `call` of it: the 16 keys 32 kb + 8 (e / 4) + 4 hq + e % 4
  // (e < 16) of slab block kb, whose random bytes that one call gives
  {
    const int r = tid >> 3, call = tid & 7, kb = call >> 1, hq = call & 1;
    const int q = q0 + r, p = q + off;
    const bool row_ok = q < nq;
    float sv[16], dp[16], kf[16];
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 32 * kb + 8 * (e >> 2) + 4 * hq + (e & 3), j = ks0 + c;
      const bool vis = row_ok && j >= 0 && j < nk && j <= p && j > p - window;
      sv[e] = vis ? ss[r * SP + c] * scale : -INFINITY;
      dp[e] = dps[r * SP + c];
      kf[e] = 1.f;
      m = fmaxf(m, sv[e]);
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sv[e] = sv[e] == -INFINITY ? 0.f : expf(sv[e] - m);
      l += sv[e];
    }
    l += __shfl_xor(l, 1);
    l += __shfl_xor(l, 2);
    l += __shfl_xor(l, 4);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (a.drop_k && row_ok) {
      const uint32_t kbg = (uint32_t)((ks0 >> 5) + kb);  // global 32-key block (used only where keys exist)
      const Philox x = philox10(2u * kbg + (uint32_t)hq, (uint32_t)q, (uint32_t)(b * a.heads + h), a.drop_offset,
                                a.seed_lo, a.seed_hi);
#pragma unroll
      for (int e = 0; e < 16; ++e) kf[e] = drop_keep(x, e, a.drop_k) ? a.drop_scale : 0.f;
    }
    float dd = 0.f;  // D = sum_j P_j kf_j dP_j
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sv[e] *= inv;
      dd = __builtin_fmaf(sv[e] * kf[e], dp[e], dd);
    }
    dd += __shfl_xor(dd, 1);
    dd += __shfl_xor(dd, 2);
    dd += __shfl_xor(dd, 4);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 32 * kb + 8 * (e >> 2) + 4 * hq + (e & 3);
      dps[r * SP + c] = sv[e] * __builtin_fmaf(kf[e], dp[e], -dd);  // 0 where P = 0
    }
    if (row_ok && call == 0) {
      const int64_t lr = b * a.lse_sb + h * a.lse_sh + seq0 + q;
      a.dpsum[lr] = dd;
      a.lse2[lr] = l > 0.f ? m + logf(l) : INFINITY;  // natural log of the scaled scores' exponent sum
    }
  }
  __syncthreads();

  // dQ = scale dS K over the keys any of the rows can see
  const int c_lo = max(0, p0 - window + 1 - ks0), c_hi = min(K, p0 + R - ks0);
  const int d0 = 4 * (tid % G), tg = tid / G;
  float acc[RPT][4] = {};
  for (int c = c_lo; c < c_hi; ++c) {
    float kx[4];
    band_bf4(*(const uint2 *)(ks + c * PITCH + d0), kx);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float ds = dps[(tg + RG * i) * SP + c];
#pragma unroll
      for (int x = 0; x < 4; ++x) acc[i][x] = __builtin_fmaf(ds, kx[x], acc[i][x]);
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int q = q0 + tg + RG * i;
    if (q < nq)
      store_grad4(a.dq, b * a.dq_sb + (int64_t)(seq0 + q) * a.dq_st + h * a.dq_sh + d0, a.grad_f32,
                  scale * acc[i][0], scale * acc[i][1], scale * acc[i][2], scale * acc[i][3]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_band_dkdv_kernel(BwdArgs a) {
  constexpr int KB = kBandRows, RS = kBandSlab, PITCH = D + 8, DCH = D / 8, SP = KB + 1;
  constexpr int G = D / 4, KG = 256 / G, KPT = KB / KG;  // dK, dV: 4 dims x KPT keys per thread
  static_assert(KPT * KG == KB, "key split");
  __shared__ __attribute__((aligned(16))) uint16_t ks[KB * PITCH], vs[KB * PITCH], qs[RS * PITCH], dos[RS * PITCH];
  __shared__ float ss[RS * SP], dps[RS * SP];  // S then P kf; dP then dS
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nkt = (a.nk + KB - 1) / KB;
  const int kt = blockIdx.x % nkt, bh = blockIdx.x / nkt;
  const int b = bh / a.heads, h = bh % a.heads;
  int seq0 = 0, nq = a.nq, nk = a.nk;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    nq = nk = a.cu_seqlens[b + 1] - seq0;
  }
  const int k0 = kt * KB;
  if (k0 >= nk) return;  // uniform
  const int off = nk - nq, window = a.window;
  const int qr0 = k0 - off;  // query row at key position k0: slab rows qr0 .. qr0 + RS - 1
  const float scale = a.scale;

  const uint16_t *qg = (const uint16_t *)a.q + b * a.q_sb + (int64_t)seq0 * a.q_st + h * a.q_sh;
  const uint16_t *dog = (const uint16_t *)a.dout + b * a.do_sb + (int64_t)seq0 * a.do_st + h * a.do_sh;
  const uint16_t *kg = (const uint16_t *)a.k + b * a.k_sb + (int64_t)seq0 * a.k_st + h * a.k_sh;
  const uint16_t *vg = (const uint16_t *)a.v + b * a.v_sb + (int64_t)seq0 * a.v_st + h * a.v_sh;
  for (int idx = tid; idx < KB * DCH; idx += 256) {
    const int c = idx / DCH, ch = idx % DCH;
    uint4 k4 = {0u, 0u, 0u, 0u}, v4 = k4;
    if (k0 + c < nk) {
      k4 = *(const uint4 *)(kg + (int64_t)(k0 + c) * a.k_st + ch * 8);
      v4 = *(const uint4 *)(vg + (int64_t)(k0 + c) * a.v_st + ch * 8);
    }
    *(uint4 *)(ks + c * PITCH + ch * 8) = k4;
    *(uint4 *)(vs + c * PITCH + ch * 8) = v4;
  }
  for (int idx = tid; idx < RS * DCH; idx += 256) {
    const int r = idx / DCH, ch = idx % DCH, q = qr0 + r;
    uint4 q4 = {0u, 0u, 0u, 0u}, o4 = q4;
    if (q >= 0 && q < nq) {
      q4 = *(const uint4 *)(qg + (int64_t)q * a.q_st + ch * 8);
      o4 = *(const uint4 *)(dog + (int64_t)q * a.do_st + ch * 8);
    }
    *(uint4 *)(qs + r * PITCH + ch * 8) = q4;
    *(uint4 *)(dos + r * PITCH + ch * 8) = o4;
  }
  __syncthreads();
  // wave w: slab rows 32 w..32 w + 31 against the 32 keys
  band_block<D, PITCH, SP>(qs, ks, dos, vs, wave, 0, ss, dps, lane);
  __syncthreads();

  // slab row r, Philox call hq of it: keys 8 (e / 4) + 4 hq + e % 4 (e < 16)
  {
    const int r = tid >> 1, hq = tid & 1;
    const int q = qr0 + r, p = k0 + r;
    const bool row_ok = q >= 0 && q < nq;
    const int64_t lr = b * a.lse_sb + h * a.lse_sh + seq0 + q;
    const float lse = row_ok ? a.lse2[lr] : INFINITY, dd = row_ok ? a.dpsum[lr] : 0.f;
    Philox x = {{0u, 0u, 0u, 0u}};
    if (a.drop_k && row_ok)
      x = philox10(2u * (uint32_t)kt + (uint32_t)hq, (uint32_t)q, (uint32_t)(b * a.heads + h), a.drop_offset,
                   a.seed_lo, a.seed_hi);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 8 * (e >> 2) + 4 * hq + (e & 3), j = k0 + c;
      const bool vis = row_ok && j < nk && j <= p && j > p - window;
      const float pr = vis ? expf(ss[r * SP + c] * scale - lse) : 0.f;
      const float kf = a.drop_k ? (drop_keep(x, e, a.drop_k) ? a.drop_scale : 0.f) : 1.f;
      const float dp = dps[r * SP + c];
      ss[r * SP + c] = pr * kf;
      dps[r * SP + c] = pr * __builtin_fmaf(kf, dp, -dd);
    }
  }
  __syncthreads();

  // dV = (P kf)^T dO and dK = scale dS^T Q over the rows that can see a key here
  const int r_lo = max(0, -qr0), r_hi = min(min(RS, KB - 1 + window), nq - qr0);
  const int d0 = 4 * (tid % G), kgp = tid / G;
  float gk[KPT][4] = {}, gv[KPT][4] = {};
  for (int r = r_lo; r < r_hi; ++r) {
    float qx[4], ox[4];
    band_bf4(*(const uint2 *)(qs + r * PITCH + d0), qx);
    band_bf4(*(const uint2 *)(dos + r * PITCH + d0), ox);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = kgp + KG * i;
      const float ds = dps[r * SP + c], pk = ss[r * SP + c];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        gk[i][x] = __builtin_fmaf(ds, qx[x], gk[i][x]);
        gv[i][x] = __builtin_fmaf(pk, ox[x], gv[i][x]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = k0 + kgp + KG * i;
    if (j < nk) {
      store_grad4(a.dk, b * a.dk_sb + (int64_t)(seq0 + j) * a.dk_st + h * a.dk_sh + d0, a.grad_f32,
                  scale * gk[i][0], scale * gk[i][1], scale * gk[i][2], scale * gk[i][3]);
      store_grad4(a.dv, b * a.dv_sb + (int64_t)(seq0 + j) * a.dv_st + h * a.dv_sh + d0, a.grad_f32, gv[i][0],
                  gv[i][1], gv[i][2], gv[i][3]);
    }
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs &a, hipStream_t s) {
  constexpr int NW_KV = 4;
  if (bwd_band(a.causal, a.window)) {
    const int64_t bh = (int64_t)a.batch * a.heads;
    const int64_t q_items = bh * ((a.nq + kBandRows - 1) / kBandRows);
    const int64_t k_items = bh * ((a.nk + kBandRows - 1) / kBandRows);
    if (q_items > 0) hipLaunchKernelGGL((bwd_band_dq_kernel<D>), dim3((unsigned)q_items), dim3(256), 0, s, a);
    if (k_items > 0) hipLaunchKernelGGL((bwd_band_dkdv_kernel<D>), dim3((unsigned)k_items), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // D and lse2 of every row: [batch, heads, nq], or heads x total_tokens
  // rows for a packed call (its lse layout)
  const int64_t rows = a.cu_seqlens ? (int64_t)a.heads * a.lse_sh : (int64_t)a.batch * a.heads * a.nq;
  if (rows > 0) {
    constexpr int RPB = 256 / (D / 8) * kDsumRows;
    hipLaunchKernelGGL((bwd_dsum_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, a, rows);
  }
  const int cus = persistent_groups();
  // grid and flag of a launch over `tiles` tiles per (batch, head)
  auto plan = [&](int64_t tiles, BwdArgs &p) {
    const int64_t items = tiles * a.heads * a.batch;
    const int64_t units = (a.causal ? (tiles + 1) / 2 : tiles) * a.heads * a.batch;
    p = a;
    p.persist = !a.cu_seqlens && cus >= 8 && units >= cus;
    return p.persist ? (int64_t)cus : items;
  };
  // dK/dV keeps one work-group per key tile: its items end in 128 KB of
  // fp32 gradient stores that the next item's DMA wait would drain, and a
  // persistent schedule measured 9% slower there (dQ: 7-8% faster)
  const int64_t kv_items = (int64_t)((a.nk + 32 * NW_KV - 1) / (32 * NW_KV)) * a.heads * a.batch;
  if (kv_items > 0) {
    if (a.drop_k) hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3((unsigned)kv_items), dim3(NW_KV * 64), 0, s, a);
    else hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3((unsigned)kv_items), dim3(NW_KV * 64), 0, s, a);
  }
  BwdArgs pq;
  int64_t q_grid = plan((a.nq + 256 - 1) / 256, pq);
  if (a.cu_seqlens && cus >= 8 && a.batch <= kPackedSeqs && q_grid > 0) {  // packed: schedule from cu_seqlens
    pq.persist = 2;
    q_grid = cus;
  }
  if (q_grid > 0) {
    if (a.drop_k) hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3((unsigned)q_grid), dim3(256), 0, s, pq);
    else hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3((unsigned)q_grid), dim3(256), 0, s, pq);
  }
  const int64_t start_items = (int64_t)a.batch * a.heads * kStartSplit;
  if (a.causal && start_items > 0 && a.nq > 0 && a.nk > 0)
    hipLaunchKernelGGL((bwd_start_kernel<D>), dim3((unsigned)start_items), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool bwd_band(int causal, int window) { return causal && window > 0 && window <= kBandMax; }

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
