// FP8 (OCP e4m3) forward: the same tiled online-softmax attention as the bf16
// kernel, with Q, K, V stored as e4m3 codes plus one fp32 descale per tensor
// (the FP8 paragraph of the FA-3 section of "Flash-Attention 2/3在ms-swift中的
// 集成与性能提升"; the value a code stands for is code * descale).
//
//   S^T = (s_q s_k scale) * K8 Q8^T   on v_mfma_f32_32x32x64_f8f6f4 (fp8 x fp8)
//   online softmax in fp32 registers (per-row max m, sum l), as in bf16
//   P~ -> e4m3 (RNE, values in [0, 1]);  O^T += V8^T P~8^T on the same MFMA
//   O = s_v * O / l -> bf16,  LSE in natural log
//
// gfx950 specifics: the fp8 MFMA takes 32 codes per lane and operand; the
// accumulator has the same 32x32 layout as the bf16 one, so each lane again
// owns one query (lane % 32) and 16 keys of each 32-key block, and its 32
// P~ values of a 64-key tile form the B operand of one K=64 product.  The V
// tile is stored row-major; its V^T operand comes from 8-bit transposed LDS
// reads whose source rows follow exactly that key order.  As in the bf16
// kernel, the product of tile j-1 is issued between the softmax stages of
// tile j.
// P~ is quantised without a scale: it is <= 2^8 (the running max lags the
// true one by at most 8 in log2 units) and e4m3 keeps 3 mantissa bits from
// 2^-6 up to 448 (subnormals to 2^-9).

#include <hip/hip_runtime.h>

#include <cfloat>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_fp8(const uint4 &a0, const uint4 &a1, const uint4 &b0, const uint4 &b1,
                                           f32x16 c) {
  const i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  // format codes 0/0: both operands OCP fp8 e4m3; no block scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// four fp32 values -> four e4m3 codes in one dword (RNE).  The first
// conversion writes the low half and keeps the high half of its `old`
// operand, which the second one overwrites; `dead` is a dword whose last use
// has passed (the previous tile's packed P~ word that this one replaces), so
// the compiler converts in that register instead of first zeroing or copying
// into one.
__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3, uint32_t dead) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, (int)dead, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}

// 8-byte transposed LDS read (ds_read_b64_tr_b8): within each 16-lane group,
// output lane l receives byte (l % 8) of the 8-byte chunks addressed by the
// source lanes (l % 16) / 8 + 2 j, j = 0..7, in that order.
__device__ __forceinline__ uint2 lds_read_tr8(const uint8_t *p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)(p));
  return (uint2){(uint32_t)r.x, (uint32_t)r.y};
}

// V tiles (64 keys x D bytes) are stored row-major with their 32-byte chunks
// XOR-swizzled per row: chunk c of row r sits at c ^ vswz<D>(r).  With it,
// the eight rows of one transposed read (keys {0..3, 8..11} + 4 hf, shifted
// by 16 for the upper k-slots) hit eight different 32-byte bank groups.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (D == 128)
    return ((r >> 1) & 1) + 2 * ((r >> 3) & 1);
  else
    return (r >> 3) & 1;
}

// B-operand byte e (0..31) of lane half hf is P~ of key 32 (e / 16) +
// 8 ((e % 16) / 4) + 4 hf + e % 4 of the 64-key tile (the accumulator order).
__device__ __forceinline__ int pkey(int e, int hf) {
  return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * hf + (e & 3);
}

// ---------------------------------------------------------------------------
// FP8 forward, 8 waves of 32 query rows, two waves per SIMD, with the P.V
// product of tile j-1 issued next to the softmax stages of tile j.
// ---------------------------------------------------------------------------
// row pitch (elements) of the bf16 O tile staged in LDS by the epilogue
template <int D>
constexpr int kFp8OP = D + 8;

template <int D, int NW>
__device__ __forceinline__ void fp8_item(const FwdArgs &a, int b, int h, int qt) {
  constexpr int BC = 64, BR = 32 * NW, T = NW * 64;
  constexpr int KPB = D + 16;          // K tile row pitch (bytes): 16 rows of a b128 read hit distinct banks
  constexpr int KSB = BC * KPB, VSB = BC * D;
  constexpr int DCH = D / 16;          // 16-byte chunks per row
  constexpr int NCH = (BC * DCH + T - 1) / T;
  constexpr int OSB = BR * kFp8OP<D> * 2;  // staged O tile (bytes)
  // K and V rings; the epilogue reuses the space for the O tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[(2 * KSB + 2 * VSB > OSB) ? 2 * KSB + 2 * VSB : OSB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int ql = lane & 31, hf = lane >> 5;

  int seq0 = 0, nq = a.nq, nk = a.nk;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    nq = nk = a.cu_seqlens[b + 1] - seq0;
  }
  const int q0 = qt * BR;
  if (q0 >= nq) return;
  const int off = nk - nq;
  const int causal = a.causal, window = a.window;

  const uint8_t *qbase = (const uint8_t *)a.q + b * a.q_sb + (int64_t)seq0 * a.q_st + h * a.q_sh;
  const uint8_t *kbase = (const uint8_t *)a.k + b * a.k_sb + (int64_t)seq0 * a.k_st + h * a.k_sh;
  const uint8_t *vbase = (const uint8_t *)a.v + b * a.v_sb + (int64_t)seq0 * a.v_st + h * a.v_sh;
  const __amdgpu_buffer_rsrc_t qrs = slice_rsrc(qbase, slice_bytes(nq, a.q_st, D, 1));
  const __amdgpu_buffer_rsrc_t krs = slice_rsrc(kbase, slice_bytes(nk, a.k_st, D, 1));
  const __amdgpu_buffer_rsrc_t vrs = slice_rsrc(vbase, slice_bytes(nk, a.v_st, D, 1));
  const uint32_t kst = (uint32_t)a.k_st, vst = (uint32_t)a.v_st;

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
  // keys this lane's query row may see
  const VisRange vr = vis_range(window > 0 ? (int64_t)my_p - window + 1 : 0, causal ? min(nk - 1, my_p) : nk - 1);
  auto active = [&](int jt) __attribute__((always_inline)) {
    const int k0 = jt * BC;
    return wave_rows && (!causal || k0 <= wp_hi) && (window <= 0 || k0 + BC - 1 > wp_lo - window);
  };
  auto kbuf = [&](int jt) __attribute__((always_inline)) { return smem + ((jt - jt0) & 1) * KSB; };
  auto vbuf = [&](int jt) __attribute__((always_inline)) { return smem + 2 * KSB + ((jt - jt0) & 1) * VSB; };

  // Q^T B operands: per 64-dim step, lane half hf holds dims [64 ks + 32 hf, +32)
  uint4 qreg[D / 64][2];
  {
    const uint32_t qo = (uint32_t)my_q * (uint32_t)a.q_st + hf * 32;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      qreg[ks][0] = bload16(qrs, qo + ks * 64);
      qreg[ks][1] = bload16(qrs, qo + ks * 64 + 16);
    }
  }

  // per-lane V^T operand offsets: read t (0..3) of 32-dim block db gives
  // k-slots 8t..8t+7; this lane serves as source lane s of the transposed read
  int voff[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) {
    const int key = pkey(8 * t4 + (lane & 15) / 2, hf);
    const int col = 8 * (lane & 1) + 16 * ((lane >> 4) & 1);  // byte within the 32-byte chunk
    voff[t4] = key * D + col;
  }

  uint4 kreg[NCH], vreg[NCH];
  auto load_k = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int cidx = tid + i * T;
      kreg[i] = bload16(krs, (uint32_t)(k0 + cidx / DCH) * kst + (cidx % DCH) * 16);
    }
  };
  auto load_v = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int cidx = tid + i * T;
      vreg[i] = bload16(vrs, (uint32_t)(k0 + cidx / DCH) * vst + (cidx % DCH) * 16);
    }
  };
  auto store_k = [&](uint8_t *ks) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int cidx = tid + i * T;
      if (NCH * T == BC * DCH || cidx < BC * DCH) *(uint4 *)(ks + (cidx / DCH) * KPB + (cidx % DCH) * 16) = kreg[i];
    }
  };
  auto store_v = [&](uint8_t *vs) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int cidx = tid + i * T;
      if (NCH * T == BC * DCH || cidx < BC * DCH) {
        const int r = cidx / DCH, c16 = cidx % DCH;
        const int c32 = (c16 >> 1) ^ vswz<D>(r);
        *(uint4 *)(vs + r * D + c32 * 32 + (c16 & 1) * 16) = vreg[i];
      }
    }
  };
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
  // the running max starts at -FLT_MAX, not -inf: the first finite score of
  // a row replaces it, and a row whose scores are all masked keeps it and
  // gets p = 2^(-inf) = 0, so the exponent's offset needs no -inf guard
  float m = -FLT_MAX, l = 0.f;
  const float c = a.scale_log2;  // includes the q and k descales
  f32x16 s[2];
  uint4 pb0_prev = {0u, 0u, 0u, 0u}, pb1_prev = {0u, 0u, 0u, 0u};
  float alpha_prev = 1.f;

  // per-lane swizzled V offsets for the two lane halves' keys are fixed:
  // source lane s reads row pkey(8 t + (s % 16) / 2, s / 32)
  int vrow_sw[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) vrow_sw[t4] = vswz<D>(pkey(8 * t4 + (lane & 15) / 2, hf));

  auto vfrag = [&](const uint8_t *vs, int db, uint4 &lo, uint4 &hi) __attribute__((always_inline)) {
    uint2 r[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) r[t4] = lds_read_tr8(vs + voff[t4] + ((db ^ vrow_sw[t4]) << 5));
    lo = (uint4){r[0].x, r[0].y, r[1].x, r[1].y};
    hi = (uint4){r[2].x, r[2].y, r[3].x, r[3].y};
  };
  auto qk = [&](const uint8_t *ks) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (f32x16){};
      const uint8_t *krow = ks + (kb * 32 + ql) * KPB + hf * 32;
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk)
        s[kb] = mfma_fp8(*(const uint4 *)(krow + kk * 64), *(const uint4 *)(krow + kk * 64 + 16), qreg[kk][0],
                         qreg[kk][1], s[kb]);
    }
  };
  auto rescale_prev = [&]() __attribute__((always_inline)) {
    if (__ballot(alpha_prev != 1.f)) {
      float a_r = alpha_prev;
      asm volatile("" : "+v"(a_r));  // keep the multiplies inside this branch
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= a_r;
    }
  };

  // one key tile: K(jt+1) and V(jt) are fetched into registers meanwhile;
  // the previous tile's D/32 product MFMAs are issued between the softmax
  // stages of this tile
  auto step = [&](auto mask_tag, int jt) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = jt * BC;
    const bool more_k = jt + 1 < jt1;
    if (!MASK || more_k) load_k(k0 + BC);
    load_v(k0);
    float alpha = 1.f;
    uint4 pb0 = {0u, 0u, 0u, 0u}, pb1 = {0u, 0u, 0u, 0u};
    const bool act = !MASK || active(jt);
    if (act) {
      qk(kbuf(jt));
      if (MASK) {
        const uint32_t vo = vis_offset(vr, k0 + 4 * hf);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!vis(vo, vr, kb * 32 + 8 * (r >> 2) + (r & 3))) s[kb][r] = -INFINITY;
      }
    }
    rescale_prev();
    const uint8_t *vs = vbuf(jt - 1);
    uint4 vlo, vhi;
    vfrag(vs, 0, vlo, vhi);
    float mx = 0.f, mx1 = 0.f, rs[2] = {0.f, 0.f};
    __builtin_amdgcn_sched_barrier(0);
    // stages: 0 max, 1 max + new m, 2..5 exponentials (8 each), 6 pack;
    // the product MFMA of block db is issued at stage 2 db (its operand
    // read one stage before)
    constexpr int NDB = D / 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 nlo, nhi;
      const bool mf = (i % 2 == 0) && (i / 2) < NDB;
      if (mf && i / 2 + 1 < NDB) vfrag(vs, i / 2 + 1, nlo, nhi);
      if (mf) acc[i / 2] = mfma_fp8(vlo, vhi, pb0_prev, pb1_prev, acc[i / 2]);
      if (mf && i / 2 + 1 < NDB) {
        vlo = nlo;
        vhi = nhi;
      }
      if (act) {
        if (i == 0) {
          // row max as two chains of v_max3 over the 32 scores
          mx = max3f(s[0][0], s[0][1], s[0][2]);
          mx1 = max3f(s[0][3], s[0][4], s[0][5]);
#pragma unroll
          for (int r = 6; r < 14; r += 4) {
            mx = max3f(mx, s[0][r], s[0][r + 1]);
            mx1 = max3f(mx1, s[0][r + 2], s[0][r + 3]);
          }
          mx = max3f(mx, s[0][14], s[0][15]);
        } else if (i == 1) {
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            mx = max3f(mx, s[1][r], s[1][r + 1]);
            mx1 = max3f(mx1, s[1][r + 2], s[1][r + 3]);
          }
          mx = max3f(mx, mx1, mx1);
          {  // with lane l ^ 32, which holds the rest of the row
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = max3f(__uint_as_float(sw[0]), __uint_as_float(sw[1]), __uint_as_float(sw[1])) * c;
          }
          // the running max moves only when a row max jumps by more than
          // a.lazy <= 8 (P~ <= 256 stays inside e4m3's range of 448)
          const bool up = mx > m + a.lazy;
          alpha = up ? fast_exp2(m - mx) : 1.f;
          m = up ? mx : m;
        } else if (i < 6) {
          const int kb = (i - 2) >> 1, r0 = ((i - 2) & 1) * 8;
#pragma unroll
          for (int r = r0; r < r0 + 8; ++r) {
            const float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -m));
            s[kb][r] = p;
            // two partial sums, each started from its first term
            rs[r & 1] = (i == 2 && r < 2) ? p : rs[r & 1] + p;
          }
          if (i == 5) l = l * alpha + (rs[0] + rs[1]);
        } else if (i == 6) {
          // B operand bytes b = 0..31 <- (kb, r) = (b / 16, b % 16)
          pb0.x = pack_fp8x4(s[0][0], s[0][1], s[0][2], s[0][3], pb0_prev.x);
          pb0.y = pack_fp8x4(s[0][4], s[0][5], s[0][6], s[0][7], pb0_prev.y);
          pb0.z = pack_fp8x4(s[0][8], s[0][9], s[0][10], s[0][11], pb0_prev.z);
          pb0.w = pack_fp8x4(s[0][12], s[0][13], s[0][14], s[0][15], pb0_prev.w);
          pb1.x = pack_fp8x4(s[1][0], s[1][1], s[1][2], s[1][3], pb1_prev.x);
          pb1.y = pack_fp8x4(s[1][4], s[1][5], s[1][6], s[1][7], pb1_prev.y);
          pb1.z = pack_fp8x4(s[1][8], s[1][9], s[1][10], s[1][11], pb1_prev.z);
          pb1.w = pack_fp8x4(s[1][12], s[1][13], s[1][14], s[1][15], pb1_prev.w);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!MASK || more_k) store_k(kbuf(jt + 1));
    store_v(vbuf(jt));
    __syncthreads();
    pb0_prev = pb0;
    pb1_prev = pb1;
    alpha_prev = alpha;
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
  jb = max(min(jb, jt1 - 1), ja);  // the last tile is masked: it has no next K tile

  if (jt0 < jt1) {
    load_k(jt0 * BC);
    store_k(kbuf(jt0));
  }
  {  // the V buffer the first tile's (empty) product reads
    uint4 *vz = (uint4 *)vbuf(jt0 - 1);
    for (int i = tid; i < VSB / 16; i += T) vz[i] = (uint4){0u, 0u, 0u, 0u};
  }
  __syncthreads();
  const std::true_type masked;
  const std::false_type whole;
  for (int jt = jt0; jt < ja; ++jt) step(masked, jt);
  for (int jt = ja; jt < jb; ++jt) step(whole, jt);
  for (int jt = jb; jt < jt1; ++jt) step(masked, jt);
  if (jt0 < jt1) {
    rescale_prev();
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      uint4 lo, hi;
      vfrag(vbuf(jt1 - 1), db, lo, hi);
      acc[db] = mfma_fp8(lo, hi, pb0_prev, pb1_prev, acc[db]);
    }
  }

  // note: l sums the fp32 P~ (before quantisation), as the softmax denominator.
  // O goes through LDS (free once every wave is past its last product) so
  // that it leaves as whole 16-byte-per-lane rows.
  const float lt = half_swap_sum(l);
  const float inv = lt > 0.f ? a.v_descale / lt : 0.f;
  lds_barrier();
  {
    uint16_t *ot = (uint16_t *)smem + (32 * wave + ql) * kFp8OP<D>;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        uint2 w;
        w.x = pack_bf16x2(acc[db][4 * rb + 0] * inv, acc[db][4 * rb + 1] * inv);
        w.y = pack_bf16x2(acc[db][4 * rb + 2] * inv, acc[db][4 * rb + 3] * inv);
        *(uint2 *)(ot + db * 32 + 8 * rb + 4 * hf) = w;
      }
  }
  if (my_q < nq && hf == 0 && a.lse)
    a.lse[b * a.lse_sb + h * a.lse_sh + seq0 + my_q] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  lds_barrier();
  uint16_t *obase = (uint16_t *)a.o + b * a.o_sb + (int64_t)(seq0 + q0) * a.o_st + h * a.o_sh;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < BR * CPR / T; ++i) {
    const int idx = tid + i * T, row = idx / CPR, ch = idx % CPR;
    const uint4 v = *(const uint4 *)((const uint16_t *)smem + row * kFp8OP<D> + ch * 8);
    if (q0 + row < nq) *(uint4 *)(obase + (int64_t)row * a.o_st + ch * 8) = v;
  }
}

// Dense calls with at least one unit per CU run persistently (launch_units);
// the item body is called from one place, on the kernel's by-value arguments.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fwd_fp8_kernel(FwdArgs a) {
  const UnitRange r = launch_units(a.persist, a.batch, a.heads, a.nqt, a.causal);
  for (int u = r.lo; u < r.hi; u += r.step)
    for (int j = 0; j < 2; ++j) {
      int b, h, qt;
      if (!launch_tile(a.persist, r, u, j, a.batch, a.heads, a.nqt, a.cu_seqlens != nullptr, a.causal, false, b, h,
                       qt))
        break;
      fp8_item<D, NW>(a, b, h, qt);
      lds_barrier();  // the next item stages its tiles into the same LDS
    }
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdArgs &a, int head_dim, hipStream_t s) {
  FwdArgs p = a;
  dim3 grid((unsigned)(a.nqt * a.heads * a.batch));
  const int cus = persistent_groups();
  const int64_t units = (int64_t)a.batch * a.heads * (a.causal ? (a.nqt + 1) / 2 : a.nqt);
  p.persist = !a.cu_seqlens && cus >= 8 && units >= cus;
  if (p.persist) grid = dim3((unsigned)cus);
  if (head_dim == 128)
    hipLaunchKernelGGL((fwd_fp8_kernel<128, 8>), grid, dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<64, 8>), grid, dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
