// Forward kernels: exact attention by tiling with an online softmax.
//
// What is computed (per query row i of one (batch, head)):
//   O_i = sum_j softmax_j(scale * q_i . k_j + mask_ij) v_j,   LSE_i = ln sum_j e^{...}
// Definition: the attention formula of "Flash-Attention 2/3在ms-swift中的集成与性能提升"
// and section 2.1 of "FlashAttention优化Transformer显存与计算效率" (jsqmd.com).
// Method: Q/K/V are split into tiles held on chip (jsqmd.com 2.2.1), each key
// tile updates a running row max m and exponent sum l (jsqmd.com 2.2.2), and
// QK^T, mask, softmax and the P.V product run in one kernel (jsqmd.com 2.2.3),
// so S never reaches HBM.  bf16 operands with fp32 softmax accumulation and a
// conversion only at the output follow jsqmd.com 3.2.  Causal / sliding-window
// tiles that the mask hides entirely are skipped (FA-3 paragraph of the
// ms-swift integration page).
//
// gfx950 mapping of the bf16 kernel (one work-group = NW waves, 32 query rows
// per wave, key tiles of 64):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims read as
//     16-byte rows of the K tile in LDS, B = Q^T held in VGPRs for the whole
//     loop.  The 32x32 accumulator then gives every lane ONE query (lane % 32)
//     and 16 keys, so the row max / row sum need only in-lane work plus one
//     exchange with lane ^ 32.
//   * O^T += V^T P^T on the same MFMA: B = P^T comes straight from the S^T
//     accumulator registers (converted to bf16), A = V^T read from a
//     transposed copy of the V tile in LDS whose key order inside each group
//     of 16 keys matches the accumulator's layout, so no register shuffles are
//     needed.  O^T again gives each lane one query, so the rescale by
//     alpha = 2^(m_old - m_new) is a per-lane scalar.
//   * K/V tiles stream global -> VGPR -> LDS with 16-byte coalesced loads,
//     issued one tile ahead and double-buffered in LDS (one barrier per tile).
//   * Work-group ids are renumbered so each XCD (own L2) processes a
//     contiguous range of (head, query-tile) items, keeping a head's K/V in one
//     L2; causal items run heaviest first.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

// Split the (XCD-renumbered) block id into (batch, head, query tile),
// heaviest causal tiles first.
__device__ __forceinline__ void decode_item(const FwdArgs &a, int &b, int &h, int &qt) {
  const int item = xcd_item(blockIdx.x, a.nqt * a.heads * a.batch);
  const int bh = item / a.nqt, t = item % a.nqt;
  qt = a.causal ? a.nqt - 1 - t : t;
  b = bh / a.heads;
  h = bh % a.heads;
}

// K/V tile staging for the bf16 kernel: global -> VGPR (buffer loads, rows
// past the slice come back as zeros) -> LDS, both tiles row-major.
template <int D, int T>
struct KvStage {
  static constexpr int BC = 64;
  static constexpr int DCH = D / 8;                  // 16-byte chunks per row
  static constexpr int NCH = (BC * DCH + T - 1) / T; // chunks per thread and tile
  static constexpr int KP = D + 8;   // K row pitch (bf16): 16-lane b128 reads of 16 rows hit distinct banks
  static constexpr int VP = D + 32;  // V row pitch (bf16): the 4 rows of a 32-lane transposed read start
                                     // 16 banks apart
  static constexpr int KS = BC * KP;
  static constexpr int VS = BC * VP;
  static constexpr int STAGE = KS + VS;

  uint4 kreg[NCH], vreg[NCH];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, int k0,
                                       int tid, uint32_t kst2, uint32_t vst2) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * T;
      const int row = c / DCH, col = (c % DCH) * 8;
      kreg[i] = bload16(krs, (uint32_t)(k0 + row) * kst2 + col * 2);
      vreg[i] = bload16(vrs, (uint32_t)(k0 + row) * vst2 + col * 2);
    }
  }

  __device__ __forceinline__ void store(uint16_t *ks, int tid) const {
    uint16_t *vs = ks + KS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * T;
      if (NCH * T == BC * DCH || c < BC * DCH) {
        const int row = c / DCH, col = (c % DCH) * 8;
        *(uint4 *)(ks + row * KP + col) = kreg[i];
        *(uint4 *)(vs + row * VP + col) = vreg[i];
      }
    }
  }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(FwdArgs a) {
  using St = KvStage<D, NW * 64>;
  constexpr int BC = St::BC;        // keys per tile
  constexpr int BR = 32 * NW;       // query rows per work-group
  constexpr int T = NW * 64;        // threads
  constexpr int KP = St::KP, VP = St::VP, KS = St::KS, STAGE = St::STAGE;
  static_assert(VP % 4 == 0, "8-byte aligned transposed reads");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int ql = lane & 31, hf = lane >> 5;
  // this lane's source address (in V-tile elements) for the transposed reads
  const int vtr_off = (4 * hf + (lane & 15) / 4) * St::VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int b, h, qt;
  decode_item(a, b, h, qt);
  int seq0 = 0, nq = a.nq, nk = a.nk;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    nq = nk = a.cu_seqlens[b + 1] - seq0;
  }
  const int q0 = qt * BR;
  if (q0 >= nq) return;  // uniform for the whole work-group
  const int off = nk - nq;
  const int causal = a.causal, window = a.window;

  const uint16_t *qbase = (const uint16_t *)a.q + b * a.q_sb + (int64_t)seq0 * a.q_st + h * a.q_sh;
  const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_sb + (int64_t)seq0 * a.k_st + h * a.k_sh;
  const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_sb + (int64_t)seq0 * a.v_st + h * a.v_sh;
  const __amdgpu_buffer_rsrc_t qrs = slice_rsrc(qbase, slice_bytes(nq, a.q_st, D, 2));
  const __amdgpu_buffer_rsrc_t krs = slice_rsrc(kbase, slice_bytes(nk, a.k_st, D, 2));
  const __amdgpu_buffer_rsrc_t vrs = slice_rsrc(vbase, slice_bytes(nk, a.v_st, D, 2));
  const uint32_t kst2 = (uint32_t)a.k_st * 2, vst2 = (uint32_t)a.v_st * 2;

  // key range the whole work-group needs
  const int p_lo = q0 + off, p_hi = min(q0 + BR, nq) - 1 + off;
  int kv_lo = 0, kv_hi = nk;
  if (causal) kv_hi = min(nk, p_hi + 1);
  if (window > 0) kv_lo = max(0, p_lo - window + 1);
  const int jt0 = kv_lo / BC;
  const int jt1 = kv_hi > kv_lo ? (kv_hi + BC - 1) / BC : jt0;

  // this wave's rows
  const int wq0 = q0 + 32 * wave;
  const bool wave_rows = wq0 < nq;
  const int wp_lo = wq0 + off, wp_hi = min(wq0 + 31, nq - 1) + off;
  const int my_q = wq0 + ql;
  const int my_p = my_q + off;

  uint4 qreg[D / 16];
  {
    const uint32_t qoff = (uint32_t)my_q * (uint32_t)a.q_st * 2 + hf * 16;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = bload16(qrs, qoff + kk * 32);
  }

  St st;
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
  float m = -INFINITY, l = 0.f;
  const float c = a.scale_log2;

  // One key tile: S^T = K Q^T, (mask), online softmax, O^T += V^T P^T.
  // MASK = false is only used for tiles that no row of the work-group sees
  // partially, so that path carries no compare or select at all.
  auto tile = [&](auto mask_tag, int jt) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = (jt - jt0) & 1;
    const int k0 = jt * BC;
    const bool more = jt + 1 < jt1;
    if (more) st.load(krs, vrs, k0 + BC, tid, kst2, vst2);
    const uint16_t *ks = smem + buf * STAGE;
    const uint16_t *vt = ks + KS;
    const bool active = !MASK || (wave_rows && (!causal || k0 <= wp_hi) &&
                                  (window <= 0 || k0 + BC - 1 > wp_lo - window));
    if (active) {
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = (f32x16){};
        const uint16_t *krow = ks + (kb * 32 + ql) * KP + hf * 8;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          s[kb] = mfma_bf16(*(const uint4 *)(krow + kk * 16), qreg[kk], s[kb]);
      }
      if (MASK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = key < nk && (!causal || key <= my_p) &&
                            (window <= 0 || key > my_p - window);
            if (!ok) s[kb][r] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m, mx * c);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      m = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
          s[kb][r] = p;
          rs += p;
        }
      l = l * alpha + rs;
      // the running max of most rows stops changing after a few tiles: skip
      // the accumulator rescale when it is 1 for every row of the wave.
      // Passing alpha through an empty asm inside the branch stops the
      // compiler from hoisting the 64 multiplies out of it.
      if (__ballot(alpha != 1.f)) {
        float a_r = alpha;
        asm volatile("" : "+v"(a_r));
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= a_r;
      }
      uint4 pb[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int kb = cc >> 1, r0 = (cc & 1) * 8;
        pb[cc].x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
        pb[cc].y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
        pb[cc].z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
        pb[cc].w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
      }
      // A = V^T (32 dims x 16 keys) straight from the row-major V tile:
      // two transposed reads give lane (d = lane % 32, half hf) the keys
      // 16 cc + 4 hf + 0..3 and 16 cc + 8 + 4 hf + 0..3, the order in which
      // the accumulator lists P~ for that lane half.
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const uint16_t *vp = vt + vtr_off + cc * 16 * VP + db * 32;
          const uint2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 8 * VP);
          const uint4 va = {lo.x, lo.y, hi.x, hi.y};
          acc[db] = mfma_bf16(va, pb[cc], acc[db]);
        }
      }
    }
    if (more) st.store(smem + (buf ^ 1) * STAGE, tid);
    __syncthreads();
  };

  // Tiles [jt0, ja) may be cut by the window, [jb, jt1) by the diagonal or
  // the end of the keys; [ja, jb) is seen whole by every row.
  int ja = jt0, jb = jt1;
  if (window > 0) {
    // tile jt needs the mask while its first key is <= p_hi - window
    const int lim = p_hi - window;
    ja = lim >= 0 ? min(jt1, max(jt0, lim / BC + 1)) : jt0;
  }
  if (causal) {
    // tile jt needs the mask once its last key exceeds p_lo
    const int lim = p_lo - (BC - 1);
    jb = lim >= 0 ? max(ja, min(jt1, lim / BC + 1)) : ja;
  }
  if (jt1 > jt0 && jt1 * BC > nk) jb = max(ja, min(jb, jt1 - 1));

  if (jt0 < jt1) {
    st.load(krs, vrs, jt0 * BC, tid, kst2, vst2);
    st.store(smem, tid);
  }
  __syncthreads();
  const std::true_type masked;
  const std::false_type whole;
  for (int jt = jt0; jt < ja; ++jt) tile(masked, jt);
  for (int jt = ja; jt < jb; ++jt) tile(whole, jt);
  for (int jt = jb; jt < jt1; ++jt) tile(masked, jt);

  // epilogue: O = acc / l (bf16, round to nearest even), LSE = (m + log2 l) ln 2
  const float lt = half_swap_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (my_q < nq) {
    uint16_t *orow = (uint16_t *)a.o + b * a.o_sb + (int64_t)(seq0 + my_q) * a.o_st + h * a.o_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        uint2 w;
        w.x = pack_bf16x2(acc[db][4 * rb + 0] * inv, acc[db][4 * rb + 1] * inv);
        w.y = pack_bf16x2(acc[db][4 * rb + 2] * inv, acc[db][4 * rb + 3] * inv);
        *(uint2 *)(orow + db * 32 + 8 * rb + 4 * hf) = w;
      }
    if (hf == 0 && a.lse)
      a.lse[b * a.lse_sb + h * a.lse_sh + seq0 + my_q] =
          lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

// fp32 forward (small workloads): 4 waves x 16 query rows; a query's dot
// product is split over 4 lanes (one quarter of the head dim each) and
// combined with two lane exchanges.  Key tiles of 32 in LDS, the same online
// softmax as the bf16 kernel, all arithmetic in fp32 FMA.
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BC = 32, BR = 64, DQ = D / 4, KP = D + 4;
  __shared__ float ks[BC * KP];
  __shared__ float vs[BC * KP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int qr = lane & 15, quarter = lane >> 4;

  int b, h, qt;
  decode_item(a, b, h, qt);
  int seq0 = 0, nq = a.nq, nk = a.nk;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    nq = nk = a.cu_seqlens[b + 1] - seq0;
  }
  const int q0 = qt * BR;
  if (q0 >= nq) return;
  const int off = nk - nq;
  const int causal = a.causal, window = a.window;
  const float *qbase = (const float *)a.q + b * a.q_sb + (int64_t)seq0 * a.q_st + h * a.q_sh;
  const float *kbase = (const float *)a.k + b * a.k_sb + (int64_t)seq0 * a.k_st + h * a.k_sh;
  const float *vbase = (const float *)a.v + b * a.v_sb + (int64_t)seq0 * a.v_st + h * a.v_sh;

  const int p_lo = q0 + off, p_hi = min(q0 + BR, nq) - 1 + off;
  int kv_lo = 0, kv_hi = nk;
  if (causal) kv_hi = min(nk, p_hi + 1);
  if (window > 0) kv_lo = max(0, p_lo - window + 1);

  const int my_q = q0 + wave * 16 + qr;
  const int my_p = my_q + off;
  float qv[DQ], acc[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    qv[e] = my_q < nq ? qbase[(int64_t)my_q * a.q_st + quarter * DQ + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float c = a.scale_log2;

  for (int k0 = (kv_lo / BC) * BC; k0 < kv_hi; k0 += BC) {
    __syncthreads();
    for (int i = tid; i < BC * D; i += 256) {
      const int row = i / D, col = i % D, key = k0 + row;
      ks[row * KP + col] = key < nk ? kbase[(int64_t)key * a.k_st + col] : 0.f;
      vs[row * KP + col] = key < nk ? vbase[(int64_t)key * a.v_st + col] : 0.f;
    }
    __syncthreads();
    float s[BC];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) part = __builtin_fmaf(qv[e], ks[j * KP + quarter * DQ + e], part);
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      const int key = k0 + j;
      const bool ok = key < nk && (!causal || key <= my_p) && (window <= 0 || key > my_p - window);
      s[j] = ok ? part : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx * c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      s[j] = exp2f(__builtin_fmaf(s[j], c, -m_use));
      rs += s[j];
    }
    l = l * alpha + rs;
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      float t = acc[e] * alpha;
#pragma unroll
      for (int j = 0; j < BC; ++j) t = __builtin_fmaf(s[j], vs[j * KP + quarter * DQ + e], t);
      acc[e] = t;
    }
  }
  if (my_q < nq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *orow = (float *)a.o + b * a.o_sb + (int64_t)(seq0 + my_q) * a.o_st + h * a.o_sh;
#pragma unroll
    for (int e = 0; e < DQ; ++e) orow[quarter * DQ + e] = acc[e] * inv;
    if (quarter == 0 && a.lse)
      a.lse[b * a.lse_sb + h * a.lse_sh + seq0 + my_q] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

// Waves per work-group of the bf16 forward (32 query rows each).  8 by
// default; FA_FWD_WAVES=4 selects the 4-wave variant (for tuning runs).
static int bf16_waves() {
  static const int w = [] {
    const char *e = getenv("FA_FWD_WAVES");
    return (e && atoi(e) == 4) ? 4 : 8;
  }();
  return w;
}

int fwd_block_rows(int qkv_dtype, int head_dim) {
  (void)head_dim;
  if (qkv_dtype == 0) return 64;   // fp32 kernel
  if (qkv_dtype == 2) return 256;  // fp8 kernel: 8 waves
  return 32 * bf16_waves();
}

hipError_t launch_fwd_bf16(const FwdArgs &a, int head_dim, hipStream_t s) {
  const dim3 grid((unsigned)(a.nqt * a.heads * a.batch));
  const int nw = bf16_waves();
  if (head_dim == 128) {
    if (nw == 8)
      hipLaunchKernelGGL((fwd_bf16_kernel<128, 8>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<128, 4>), grid, dim3(256), 0, s, a);
  } else {
    if (nw == 8)
      hipLaunchKernelGGL((fwd_bf16_kernel<64, 8>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<64, 4>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs &a, int head_dim, hipStream_t s) {
  const dim3 grid((unsigned)(a.nqt * a.heads * a.batch));
  if (head_dim == 128)
    hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
