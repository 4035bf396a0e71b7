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
// tile is stored transposed in LDS with its keys in exactly that order.
// P~ is quantised without a scale: it is <= 2^8 (the running max lags the
// true one by at most 8 in log2 units) and e4m3 keeps 3 mantissa bits from
// 2^-6 up to 448 (subnormals to 2^-9).

#include <hip/hip_runtime.h>
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

// four fp32 values -> four e4m3 codes in one dword (RNE)
__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t u8_at(const uint4 &v, int e) {
  const uint32_t w = e < 4 ? v.x : e < 8 ? v.y : e < 12 ? v.z : v.w;
  return (w >> (8 * (e & 3))) & 0xffu;
}

// Position of key group g (keys 4g..4g+3 of a 64-key tile) in a transposed V
// row: lane half hf's 32 B-operand bytes are the accumulator entries
// (kb, r) = (b / 16, b % 16), i.e. key 32 kb + 8 (r / 4) + 4 hf + r % 4.
__device__ __forceinline__ int vt8_group_pos(int g) {
  return 32 * (g & 1) + 16 * (g >> 3) + 4 * ((g & 7) >> 1);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fwd_fp8_kernel(FwdArgs a) {
  constexpr int BC = 64, BR = 32 * NW, T = NW * 64;
  constexpr int KPB = D + 16;          // K tile row pitch (bytes)
  constexpr int VPB = BC + 16;         // V^T tile row pitch (bytes)
  constexpr int KSB = BC * KPB, VSB = D * VPB, STAGE = KSB + VSB;
  constexpr int DCH = D / 16;          // 16-byte chunks per row
  constexpr int KCH = (BC * DCH + T - 1) / T;
  constexpr int VUNITS = (BC / 4) * DCH;  // 4 keys x 16 dims
  constexpr int VCH = (VUNITS + T - 1) / T;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int ql = lane & 31, hf = lane >> 5;

  const int item = xcd_item(blockIdx.x, a.nqt * a.heads * a.batch);
  const int bh = item / a.nqt, t = item % a.nqt;
  const int qt = a.causal ? a.nqt - 1 - t : t;
  const int b = bh / a.heads, h = bh % a.heads;
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

  uint4 kreg[KCH], vreg[VCH][4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + i * T;
      const int row = cidx / DCH, col = cidx % DCH;
      kreg[i] = bload16(krs, (uint32_t)(k0 + row) * kst + col * 16);
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int unit = tid + u * T;
      const int g = unit / DCH, dc = unit % DCH;
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[u][i] = bload16(vrs, (uint32_t)(k0 + 4 * g + i) * vst + dc * 16);
    }
  };
  auto store_tile = [&](int buf) {
    uint8_t *ks = smem + buf * STAGE;
    uint8_t *vt = ks + KSB;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + i * T;
      if (KCH * T == BC * DCH || cidx < BC * DCH) {
        const int row = cidx / DCH, col = cidx % DCH;
        *(uint4 *)(ks + row * KPB + col * 16) = kreg[i];
      }
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int unit = tid + u * T;
      if (VCH * T == VUNITS || unit < VUNITS) {
        const int g = unit / DCH, dc = unit % DCH;
        const int pos = vt8_group_pos(g);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t w = u8_at(vreg[u][0], e) | (u8_at(vreg[u][1], e) << 8) |
                             (u8_at(vreg[u][2], e) << 16) | (u8_at(vreg[u][3], e) << 24);
          *(uint32_t *)(vt + (dc * 16 + e) * VPB + pos) = w;
        }
      }
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
  float m = -INFINITY, l = 0.f;
  const float c = a.scale_log2;  // includes the q and k descales

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
    const uint8_t *ks = smem + buf * STAGE;
    const uint8_t *vt = ks + KSB;

    const bool active = wave_rows && (!causal || k0 <= wp_hi) &&
                        (window <= 0 || k0 + BC - 1 > wp_lo - window);
    if (active) {
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = (f32x16){};
        const uint8_t *krow = ks + (kb * 32 + ql) * KPB + hf * 32;
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk)
          s[kb] = mfma_fp8(*(const uint4 *)(krow + kk * 64), *(const uint4 *)(krow + kk * 64 + 16),
                           qreg[kk][0], qreg[kk][1], s[kb]);
      }
      const bool need_mask = (causal && k0 + BC - 1 > wp_lo) ||
                             (window > 0 && k0 <= wp_hi - window) || (k0 + BC > nk);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = key < nk && (!causal || key <= my_p) && (window <= 0 || key > my_p - window);
            if (!ok) s[kb][r] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = half_swap_max(mx) * c;
      // the running max moves only when a row max jumps by more than 2^8
      // (P~ <= 256 stays inside e4m3's range of 448), so the accumulators
      // are rescaled only then
      const bool up = mx > m + 8.f;
      const float alpha = up ? fast_exp2(m - mx) : 1.f;
      m = up ? mx : m;
      const float m_use = m == -INFINITY ? 0.f : m;
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
      if (__ballot(alpha != 1.f)) {
        float a_r = alpha;
        asm volatile("" : "+v"(a_r));  // keep the multiplies inside this branch
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= a_r;
      }
      // B operand bytes b = 0..31 <- (kb, r) = (b / 16, b % 16)
      uint4 pb0, pb1;
      pb0.x = pack_fp8x4(s[0][0], s[0][1], s[0][2], s[0][3]);
      pb0.y = pack_fp8x4(s[0][4], s[0][5], s[0][6], s[0][7]);
      pb0.z = pack_fp8x4(s[0][8], s[0][9], s[0][10], s[0][11]);
      pb0.w = pack_fp8x4(s[0][12], s[0][13], s[0][14], s[0][15]);
      pb1.x = pack_fp8x4(s[1][0], s[1][1], s[1][2], s[1][3]);
      pb1.y = pack_fp8x4(s[1][4], s[1][5], s[1][6], s[1][7]);
      pb1.z = pack_fp8x4(s[1][8], s[1][9], s[1][10], s[1][11]);
      pb1.w = pack_fp8x4(s[1][12], s[1][13], s[1][14], s[1][15]);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint8_t *vrow = vt + (db * 32 + ql) * VPB + hf * 32;
        acc[db] = mfma_fp8(*(const uint4 *)vrow, *(const uint4 *)(vrow + 16), pb0, pb1, acc[db]);
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // note: l sums the fp32 P~ (before quantisation), as the softmax denominator
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? a.v_descale / lt : 0.f;
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
      a.lse[b * a.lse_sb + h * a.lse_sh + seq0 + my_q] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdArgs &a, int head_dim, hipStream_t s) {
  const dim3 grid((unsigned)(a.nqt * a.heads * a.batch));
  if (head_dim == 128)
    hipLaunchKernelGGL((fwd_fp8_kernel<128, 8>), grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<64, 8>), grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
