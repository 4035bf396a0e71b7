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
// gfx950 mapping of the bf16 kernels (work-group = 8 waves x 32 query rows,
// key tiles of 64, two waves per SIMD), common to both:
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims read as
//     16-byte rows of the K tile in LDS, B = Q^T held in VGPRs for the whole
//     loop.  The 32x32 accumulator gives every lane ONE query (lane % 32) and
//     16 keys, so the row max / row sum need only in-lane work plus one
//     v_permlane32_swap with the other half of the wave.
//   * O^T += V^T P~^T on the same MFMA: B = P~^T straight from the S^T
//     accumulator (converted to bf16), A = V^T read with ds_read_b64_tr_b16
//     from the row-major V tile, addressed so that its key order matches the
//     accumulator's; O^T again gives each lane one query, so the rescale by
//     alpha = 2^(m_old - m_new) is a per-lane scalar (and is skipped when no
//     row max of the wave changed).
//   * Key tiles that no row sees partially run without any mask code; the
//     edge tiles of the causal diagonal, the window and the key tail take a
//     masked path.
//   * Work-group ids are renumbered so each XCD (own L2) processes a
//     contiguous range of (head, query-tile) items, keeping a head's K/V in one
//     L2; causal items run heaviest first.
// fwd_bf16_pp_kernel (no dropout): the two waves of a SIMD take turns, one
// issuing the MFMAs of a key tile while the other runs its softmax, with
// K/V staged by LDS DMA into XOR-swizzled tiles.  fwd_bf16_kernel (dropout):
// each wave issues the softmax of tile j between the P.V MFMAs of tile j-1,
// with K/V staged through registers into padded tiles.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

// Split the (XCD-renumbered) block id into (batch, head, query tile),
// heaviest causal tiles first.
__device__ __forceinline__ void decode_item(const FwdArgs &a, int &b, int &h, int &qt) {
  fwd_item(blockIdx.x, a.nqt, a.heads, a.batch, a.cu_seqlens != nullptr, a.causal, b, h, qt);
}

// K/V staging with K and V of different tiles (K runs one tile ahead).
template <int D, int T>
struct KvStage {
  static constexpr int BC = 64;
  static constexpr int DCH = D / 8;
  static constexpr int NCH = (BC * DCH + T - 1) / T;
  static constexpr int KP = D + 8;   // K row pitch (bf16): 16-lane b128 reads of 16 rows hit distinct banks
  static constexpr int VP = D + 32;  // V row pitch (bf16): the 4 rows of a 32-lane transposed read start
                                     // 16 banks apart
  static constexpr int KS = BC * KP;
  static constexpr int VS = BC * VP;

  uint4 kreg[NCH], vreg[NCH];

  __device__ __forceinline__ void load_k(__amdgpu_buffer_rsrc_t krs, int k0, int tid, uint32_t kst2) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * T;
      kreg[i] = bload16(krs, (uint32_t)(k0 + c / DCH) * kst2 + (c % DCH) * 16);
    }
  }
  __device__ __forceinline__ void load_v(__amdgpu_buffer_rsrc_t vrs, int k0, int tid, uint32_t vst2) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * T;
      vreg[i] = bload16(vrs, (uint32_t)(k0 + c / DCH) * vst2 + (c % DCH) * 16);
    }
  }
  __device__ __forceinline__ void store_k(uint16_t *ks, int tid) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * T;
      if (NCH * T == BC * DCH || c < BC * DCH) *(uint4 *)(ks + (c / DCH) * KP + (c % DCH) * 8) = kreg[i];
    }
  }
  __device__ __forceinline__ void store_v(uint16_t *vs, int tid) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * T;
      if (NCH * T == BC * DCH || c < BC * DCH) *(uint4 *)(vs + (c / DCH) * VP + (c % DCH) * 8) = vreg[i];
    }
  }
};

// The running row max only moves when a tile's row max exceeds it by more
// than a.lazy (log2 units): P~ = 2^(s - m) then stays <= 2^a.lazy, far inside
// fp32 and bf16 range, and the accumulators are rescaled only when a row max
// jumps that far (with inputs of unit scale, only on the first tile).  The
// result is exact either way: O and LSE are formed with the same m.  The
// launcher sets a.lazy = 8, or 0 (an exact running max) where every row sees
// at most 64 keys: those rows' weights can sit on a few keys, and with an
// exact max the largest P~ is 1, which bf16 holds without rounding.

// ---------------------------------------------------------------------------
// bf16 forward with the P.V product deferred by one key tile.  8 waves of 32
// query rows (256 rows per work-group), two waves per SIMD.  For key tile j
// each wave computes S(j) = K(j) Q^T, then runs the online softmax of S(j)
// on the VALU while the matrix cores accumulate O += V(j-1)^T P~(j-1)^T of
// the previous tile: the softmax overlaps matrix work inside every wave,
// and both waves of a SIMD keep feeding the matrix cores from LDS.  K is
// staged one tile ahead of V (LDS rings of two for each).
// ---------------------------------------------------------------------------
template <int D, int NW, bool DROP>
__device__ __forceinline__ void drop_item(const FwdArgs &a, int b, int h, int qt) {
  constexpr int T = NW * 64, BR = NW * 32;
  using St = KvStage<D, T>;
  constexpr int BC = St::BC, KP = St::KP, VP = St::VP, KS = St::KS, VS = St::VS;
  static_assert(VP % 4 == 0, "8-byte aligned transposed reads");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KS + 2 * VS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int ql = lane & 31, hf = lane >> 5;
  const int vtr_off = (4 * hf + (lane & 15) / 4) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

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
  const uint32_t slot = (uint32_t)(b * a.heads + h);  // dropout counter word 2
  // dropout randomness of key block (2 jt + kb) for this lane's query
  auto drop_init = [&](Philox &x, int jt, int kb) __attribute__((always_inline)) {
    x.c[0] = 2u * (uint32_t)(2 * jt + kb) + (uint32_t)hf;
    x.c[1] = (uint32_t)my_q;
    x.c[2] = slot;
    x.c[3] = a.drop_offset;
  };
  auto drop_apply = [&](const Philox &x, f32x16 &sv, int r0, int r1) __attribute__((always_inline)) {
#pragma unroll
    for (int e = r0; e < r1; ++e)
      if (!drop_keep(x, e, a.drop_k)) sv[e] = 0.f;
  };
  auto active = [&](int jt) __attribute__((always_inline)) {
    const int k0 = jt * BC;
    return wave_rows && (!causal || k0 <= wp_hi) && (window <= 0 || k0 + BC - 1 > wp_lo - window);
  };
  auto kbuf = [&](int jt) __attribute__((always_inline)) { return smem + ((jt - jt0) & 1) * KS; };
  auto vbuf = [&](int jt) __attribute__((always_inline)) { return smem + 2 * KS + ((jt - jt0) & 1) * VS; };

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
  // the running max starts at -FLT_MAX, not -inf: the first finite score of
  // a row replaces it, and a row whose scores are all masked keeps it and
  // gets p = 2^(-inf) = 0, so the exponent's offset needs no -inf guard
  float m = -FLT_MAX, l = 0.f;
  const float c = a.scale_log2;
  f32x16 s[2];
  uint4 pb_prev[4] = {};   // P~ of the previous tile (B operands)
  float alpha_prev = 1.f;  // accumulator rescale that goes with it
  bool has_prev = false;

  auto qk = [&](const uint16_t *ks) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (f32x16){};
      const uint16_t *krow = ks + (kb * 32 + ql) * KP + hf * 8;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) s[kb] = mfma_bf16(*(const uint4 *)(krow + kk * 16), qreg[kk], s[kb]);
    }
  };
  auto rescale_prev = [&]() __attribute__((always_inline)) {
    if (__ballot(alpha_prev != 1.f)) {  // rarely taken once the row maxima settle
      float a_r = alpha_prev;
      asm volatile("" : "+v"(a_r));  // keep the multiplies inside this branch
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= a_r;
    }
  };
  auto pv_prev = [&](const uint16_t *vs) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const uint16_t *vp = vs + vtr_off + cc * 16 * VP + db * 32;
        const uint2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 8 * VP);
        const uint4 va = {lo.x, lo.y, hi.x, hi.y};
        acc[db] = mfma_bf16(va, pb_prev[cc], acc[db]);
      }
    }
  };
  auto softmax = [&](auto mask_tag, int k0, uint4 (&pb)[4]) __attribute__((always_inline)) -> float {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (MASK) {
      const uint32_t vo = vis_offset(vr, k0 + 4 * hf);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (!vis(vo, vr, kb * 32 + 8 * (e >> 2) + (e & 3))) s[kb][e] = -INFINITY;
    }
    // row max: two chains of v_max3 over the lane's 32 scores
    float mx = max3f(s[0][0], s[0][1], s[0][2]), mx1 = max3f(s[0][3], s[0][4], s[0][5]);
#pragma unroll
    for (int i = 6; i < 30; i += 4) {
      mx = max3f(mx, s[i >> 4][i & 15], s[(i + 1) >> 4][(i + 1) & 15]);
      mx1 = max3f(mx1, s[(i + 2) >> 4][(i + 2) & 15], s[(i + 3) >> 4][(i + 3) & 15]);
    }
    mx = max3f(mx, s[1][14], s[1][15]);
    mx = swap_max3(max3f(mx, mx1, mx1)) * c;
    const bool up = mx > m + a.lazy;
    const float alpha = up ? fast_exp2(m - mx) : 1.f;
    m = up ? mx : m;
    float rs[2];  // two partial row sums, each started from its first term
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][e], c, -m));
        s[kb][e] = p;
        rs[e & 1] = (kb == 0 && e < 2) ? p : rs[e & 1] + p;
      }
    l = l * alpha + (rs[0] + rs[1]);
    if constexpr (DROP) {  // the row sum above is of the undropped P~
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Philox x;
        drop_init(x, k0 / BC, kb);
        x = philox10(x.c[0], x.c[1], x.c[2], x.c[3], a.seed_lo, a.seed_hi);
        drop_apply(x, s[kb], 0, 16);
      }
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int kb = cc >> 1, r0 = (cc & 1) * 8;
      pb[cc].x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
      pb[cc].y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
      pb[cc].z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
      pb[cc].w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
    }
    return alpha;
  };

  // one key tile: K(jt+1) and V(jt) are fetched into registers meanwhile
  auto step = [&](auto mask_tag, int jt) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = jt * BC;
    const bool more_k = jt + 1 < jt1;
    if (!MASK || more_k) st.load_k(krs, k0 + BC, tid, kst2);
    st.load_v(vrs, k0, tid, vst2);
    // zero unless this wave's softmax writes it: a wave that sits out a
    // masked tile hands P~ = 0 to the next interior tile's product, which
    // runs without a has_prev check
    uint4 pb[4] = {};
    float alpha = 1.f;
    if (!MASK) {
      // interior tile: the wave sees the whole tile and the previous one.
      // The softmax of S(jt) is cut into 16 stages, each issued next to one
      // MFMA of the previous tile's O += V^T P~^T (whose transposed operand
      // reads run two MFMAs ahead); the scheduling fences keep the compiler
      // from regrouping them, so the VALU and the matrix cores work at once.
      qk(kbuf(jt));
      rescale_prev();
      const uint16_t *vs = vbuf(jt - 1) + vtr_off;
      auto vread = [&](int i) __attribute__((always_inline)) {
        const uint16_t *vp = vs + (i % 4) * 16 * VP + (i / 4) * 32;
        const uint2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 8 * VP);
        return (uint4){lo.x, lo.y, hi.x, hi.y};
      };
      constexpr int NOP = (D / 32) * 4;  // MFMAs of the product
      uint4 va[NOP];
      va[0] = vread(0);
      va[1] = vread(1);
      float mx = 0.f, mx1 = 0.f, rs[2] = {0.f, 0.f};
      Philox rx[2];
      if constexpr (DROP) {
        drop_init(rx[0], jt, 0);
        drop_init(rx[1], jt, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + 2 < NOP) va[i + 2] = vread(i + 2);
        if (i < NOP) acc[i / 4] = mfma_bf16(va[i], pb_prev[i % 4], acc[i / 4]);
        if constexpr (DROP) {  // one Philox round of each key block per stage
          if (i < 10) {
            philox_round(rx[0], philox_k0(a.seed_lo, i), philox_k1(a.seed_hi, i));
            philox_round(rx[1], philox_k0(a.seed_lo, i), philox_k1(a.seed_hi, i));
          }
        }
        // softmax stage i
        if (i == 0) {  // row max: two chains of v_max3
          mx = max3f(s[0][0], s[0][1], s[0][2]);
          mx1 = max3f(s[0][3], s[0][4], s[0][5]);
#pragma unroll
          for (int e = 6; e < 14; e += 4) {
            mx = max3f(mx, s[0][e], s[0][e + 1]);
            mx1 = max3f(mx1, s[0][e + 2], s[0][e + 3]);
          }
          mx = max3f(mx, s[0][14], s[0][15]);
        } else if (i == 1) {
#pragma unroll
          for (int e = 0; e < 16; e += 4) {
            mx = max3f(mx, s[1][e], s[1][e + 1]);
            mx1 = max3f(mx1, s[1][e + 2], s[1][e + 3]);
          }
          mx = swap_max3(max3f(mx, mx1, mx1)) * c;
          const bool up = mx > m + a.lazy;
          alpha = up ? fast_exp2(m - mx) : 1.f;
          m = up ? mx : m;
        } else if (i < 10) {
          const int kb = (i - 2) >> 2, e0 = ((i - 2) & 3) * 4;
#pragma unroll
          for (int e = e0; e < e0 + 4; ++e) {
            const float p = fast_exp2(__builtin_fmaf(s[kb][e], c, -m));
            s[kb][e] = p;
            // two partial row sums, each started from its first term
            rs[e & 1] = (i == 2 && e < 2) ? p : rs[e & 1] + p;
          }
          if (i == 9) l = l * alpha + (rs[0] + rs[1]);
        } else if (i < 14) {
          const int cc = i - 10, kb = cc >> 1, r0 = (cc & 1) * 8;
          if constexpr (DROP) drop_apply(rx[kb], s[kb], r0, r0 + 8);  // after the row sum
          pb[cc].x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
          pb[cc].y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
          pb[cc].z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
          pb[cc].w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      has_prev = true;
    } else {
      const bool act = active(jt);
      if (act) qk(kbuf(jt));
      if (has_prev) {
        rescale_prev();
        pv_prev(vbuf(jt - 1));
      }
      if (act) alpha = softmax(std::true_type(), k0, pb);
      has_prev = act;
    }
    // interior tiles always have a next tile (the last tile takes the masked
    // path), so their K store is unconditional and no branch splits the
    // scheduled region above
    if (!MASK || more_k) st.store_k(kbuf(jt + 1), tid);
    st.store_v(vbuf(jt), tid);
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pb_prev[cc] = pb[cc];
    alpha_prev = alpha;
  };

  // tiles [jt0, ja) may be cut by the window, [jb, jt1) by the diagonal or
  // the end of the keys; the first tile always takes the masked path (no
  // previous product yet)
  int ja = jt0, jb = jt1;
  if (window > 0) {
    const int lim = p_hi - window;
    ja = lim >= 0 ? min(jt1, max(jt0, lim / BC + 1)) : jt0;
  }
  if (causal) {
    const int lim = p_lo - (BC - 1);
    jb = lim >= 0 ? max(ja, min(jt1, lim / BC + 1)) : ja;
  }
  if (jt1 > jt0 && jt1 * BC > nk) jb = max(ja, min(jb, jt1 - 1));
  ja = min(max(ja, jt0 + 1), jt1);
  jb = max(min(jb, jt1 - 1), ja);

  if (jt0 < jt1) {
    st.load_k(krs, jt0 * BC, tid, kst2);
    st.store_k(kbuf(jt0), tid);
  }
  __syncthreads();
  const std::true_type masked;
  const std::false_type whole;
  for (int jt = jt0; jt < ja; ++jt) step(masked, jt);
  for (int jt = ja; jt < jb; ++jt) step(whole, jt);
  for (int jt = jb; jt < jt1; ++jt) step(masked, jt);
  if (has_prev) {
    rescale_prev();
    pv_prev(vbuf(jt1 - 1));
  }

  // epilogue: O = acc / l (bf16, round to nearest even), LSE = (m + log2 l) ln 2,
  // O through LDS (free once every wave is past its last product) as whole rows
  const float lt = half_swap_sum(l);
  const float inv = lt > 0.f ? (DROP ? a.drop_scale : 1.f) / lt : 0.f;
  constexpr int OP = D + 8;
  static_assert(BR * OP <= 2 * KS + 2 * VS, "the O tile fits the K/V buffers");
  lds_barrier();
  {
    uint16_t *ot = smem + (32 * wave + ql) * OP;
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
    const uint4 v = *(const uint4 *)(smem + row * OP + ch * 8);
    if (q0 + row < nq) *(uint4 *)(obase + (int64_t)row * a.o_st + ch * 8) = v;
  }
}

// Calls with dropout; dense ones with at least one unit per CU run
// persistently on the schedule of launch_units.
template <int D, int NW, bool DROP>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(FwdArgs a) {
  const UnitRange r = launch_units(a.persist, a.batch, a.heads, a.nqt, a.causal);
  for (int u = r.lo; u < r.hi; u += r.step)
    for (int j = 0; j < 2; ++j) {
      int b, h, qt;
      if (!launch_tile(a.persist, r, u, j, a.batch, a.heads, a.nqt, a.cu_seqlens != nullptr, a.causal, false, b, h,
                       qt))
        break;
      drop_item<D, NW, DROP>(a, b, h, qt);
      lds_barrier();  // the next item stages its tiles into the same LDS
    }
}

// ---------------------------------------------------------------------------
// bf16 forward, ping-pong between the two waves of each SIMD (no dropout).
// A wave alternates two clusters:
//   M(u): O = alpha O + V(u)^T P~(u)^T, then S(u+1) = K(u+1) Q^T: 32 MFMAs
//         per 64 keys (d = 128) fed only by their LDS operand reads (P~(u)
//         dies before S(u+1) is born, which leaves room for 128-key tiles);
//   V(u): the online softmax of S(u) into P~(u) (row max, rescale factor,
//         exponentials, row sum, bf16 packing), and the issue of this wave
//         group's half of the next K/V tiles as LDS DMA.
// Waves 0-3 (one per SIMD) run half a step ahead of waves 4-7, and one
// barrier per half step keeps them there: on every SIMD one wave issues
// MFMAs back to back while the other works through its VALU cluster.
// K/V tiles (64 or 128 keys) travel HBM -> LDS by buffer_load ... lds, so staging
// takes neither registers nor LDS store instructions from the softmax wave;
// the tiles are stored unpadded with 16-byte chunks XOR-swizzled per row,
// which keeps the row-wise K reads and the transposed V reads conflict free.
// ---------------------------------------------------------------------------
constexpr int kRA = 3;  // MFMA operands read this many MFMAs ahead
// row pitch (elements) of the O tile staged in LDS by the epilogue: 16-byte
// aligned rows for the row-wise read-back
template <int D>
constexpr int kOP = D + 8;
// LDS of the ping-pong kernel: the K and V rings, or the staged O tile
template <int D, int BC>
constexpr int kPPLds = (4 * BC * D > 256 * kOP<D>) ? 4 * BC * D : 256 * kOP<D>;
// one (batch or sequence b, head h, query tile qt) work item.  RANGE: edge
// tiles test each key against the row's visible range with one compare
// (packed calls, where short sequences make most tiles edge tiles); else
// against each limit in turn, which holds fewer registers through the loop
// (measured 1-2% faster on dense calls, whose edge tiles are few).
// With CHAIN (dense persistent launches, no window) the item's Q fragments
// and its first K tile were fetched by the previous item (pre) into qreg and
// K slot 0, and this item fetches those of the next one (nb, nh, nqt when
// has_next) right after its loop, so that their latency passes under its own
// epilogue; the epilogue then stages O in the top of the LDS, clear of K slot 0.
template <int D, bool RANGE, int BC, bool CHAIN = false>
__device__ __forceinline__ void pp_item(const FwdArgs &a, int b, int h, int qt, uint16_t *smem, uint4 (&qreg)[D / 16],
                                        bool pre = false, bool has_next = false, int nb = 0, int nh = 0, int nqt = 0) {
  constexpr int BR = 256;
  constexpr int NKB = BC / 32, NKS = BC / 16;  // 32-key blocks of S, 16-key steps of P.V
  constexpr int TS = BC * D;                  // tile elements
  constexpr int NKK = D / 16, NDB = D / 32;
  constexpr int NBLK = TS * 2 / 1024;         // 1 KB DMA blocks per tile
  constexpr int RPB = 512 / D;                // rows per block
  constexpr int BPW = NBLK / 8;               // blocks per wave per tile (a group stages half a tile)
  static_assert(BPW >= 1 && BPW * 8 == NBLK, "block split");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int ql = lane & 31, hf = lane >> 5;

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
  const i32x4 kw = buffer_words(kbase, slice_bytes(nk, a.k_st, D, 2));
  const i32x4 vw = buffer_words(vbase, slice_bytes(nk, a.v_st, D, 2));
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
  auto active = [&](int jt) __attribute__((always_inline)) {
    const int k0 = jt * BC;
    return wave_rows && (!causal || k0 <= wp_hi) && (window <= 0 || k0 + BC - 1 > wp_lo - window);
  };
  // tiles a mask may cut for this wave: the window edge, the diagonal, the key tail
  auto edge = [&](int jt) __attribute__((always_inline)) {
    const int k0 = jt * BC;
    return k0 + BC > nk || (causal && k0 + BC - 1 > wp_lo) || (window > 0 && k0 <= wp_hi - window);
  };
  const uint32_t lds0 = lds_addr(smem);
  auto kslot = [&](int jt) __attribute__((always_inline)) { return ((jt - jt0) & 1) * TS; };
  auto vslot = [&](int jt) __attribute__((always_inline)) { return 2 * TS + ((jt - jt0) & 1) * TS; };

  if (!CHAIN || !pre) {
    const uint32_t qoff = (uint32_t)my_q * (uint32_t)a.q_st * 2 + hf * 16;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qreg[kk] = bload16(qrs, qoff + kk * 32);
  }

  // DMA: lane l of block q of a tile fills physical chunk l % (D / 8) of row
  // RPB q + l / (D / 8), i.e. logical chunk (that) ^ swz(row)
  auto dma_goff = [&](int q, uint32_t st2) __attribute__((always_inline)) {
    const int r = RPB * q + lane / (D / 8), lc = (lane % (D / 8)) ^ swz<D>(r);
    return (uint32_t)r * st2 + lc * 16;
  };
  uint32_t kgo[BPW], vgo[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int q = (wave & 3) * BPW + i + grp * (NBLK / 2);
    kgo[i] = dma_goff(q, kst2);
    vgo[i] = dma_goff(q, vst2);
  }
  // this wave's blocks of K(ts + 1) and V(ts)
  auto dma_half = [&](int ts) __attribute__((always_inline)) {
    if (ts + 1 < jt1) {
      const uint32_t gk = (uint32_t)((ts + 1) * BC) * kst2;
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int q = (wave & 3) * BPW + i + grp * (NBLK / 2);
        dma16_at(kw, lds0 + (uint32_t)(kslot(ts + 1) * 2 + q * 1024), gk + kgo[i]);
      }
    }
    if (ts < jt1) {
      const uint32_t gv = (uint32_t)(ts * BC) * vst2;
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int q = (wave & 3) * BPW + i + grp * (NBLK / 2);
        dma16_at(vw, lds0 + (uint32_t)(vslot(ts) * 2 + q * 1024), gv + vgo[i]);
      }
    }
  };

  // per-lane LDS offsets of the MFMA operands in a swizzled tile:
  // K fragment (kb, kk) at (kbase_off ^ 16 kk) + 32 kb D; V^T fragment
  // (cc, db, half) at (vt_off[half] ^ 32 db) + 16 cc D
  const int ksw = swz<D>(ql) ^ hf;
  const int kbase_off = ql * D + 8 * ksw;
  const int vt_off0 = tr_off<D>(lane, 0, 0), vt_off1 = tr_off<D>(lane, 0, 1);

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = (f32x16){};
  f32x16 s[NKB];
#pragma unroll
  for (int i = 0; i < NKB; ++i) s[i] = (f32x16){};
  uint4 pb[NKS];
#pragma unroll
  for (int i = 0; i < NKS; ++i) pb[i] = (uint4){0u, 0u, 0u, 0u};
  // The running max starts at -FLT_MAX, not -inf: the first finite score
  // of a row replaces it (alpha = 2^(-FLT_MAX - mx) = 0 then, on an O and l
  // that are still 0), and a row whose scores are all masked keeps it and
  // gets p = 2^(-inf) = 0, so the exponent's offset needs no -inf guard.
  float m = -FLT_MAX, l = 0.f, alpha = 1.f;
  const float c = a.scale_log2;

  // MFMA cluster: O = alpha O + V(u)^T P~(u)^T (four independent
  // accumulators in turn) and S(u+1) = K(u+1) Q^T (kb chains interleaved).
  // With 128-key tiles P.V runs first, so that P~(u) dies before S(u+1) is
  // born (the registers of both would not fit); with 64-key tiles Q.K^T
  // first measured 1% faster.
  auto pv_part = [&](int u) __attribute__((always_inline)) {
    if (u >= jt0 && active(u)) {
      if (__ballot(alpha != 1.f)) {  // rarely taken once the row maxima settle
        float a_r = alpha;
        asm volatile("" : "+v"(a_r));
#pragma unroll
        for (int i = 0; i < NDB; ++i) acc[i] *= a_r;
      }
      const uint16_t *vs = smem + vslot(u);
      auto vread = [&](int i) __attribute__((always_inline)) {
        const int cc = i / NDB, db = i % NDB;
        const uint2 lo = lds_read_tr16(vs + ((vt_off0 ^ (32 * db)) + cc * 16 * D));
        const uint2 hi = lds_read_tr16(vs + ((vt_off1 ^ (32 * db)) + cc * 16 * D));
        return (uint4){lo.x, lo.y, hi.x, hi.y};
      };
      constexpr int NPV = NKS * NDB;
      uint4 vf[NPV];
#pragma unroll
      for (int i = 0; i < kRA; ++i) vf[i] = vread(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        if (i + kRA < NPV) vf[i + kRA] = vread(i + kRA);
        const int cc = i / NDB, db = i % NDB;
        acc[db] = mfma_bf16(vf[i], pb[cc], acc[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto qk_part = [&](int u) __attribute__((always_inline)) {
    if (u + 1 < jt1 && active(u + 1)) {
      const uint16_t *ks = smem + kslot(u + 1);
      auto kread = [&](int i) __attribute__((always_inline)) {
        const int kb = i % NKB, kk = i / NKB;
        return *(const uint4 *)(ks + ((kbase_off ^ (16 * kk)) + kb * 32 * D));
      };
      uint4 kf[NKB * NKK];
#pragma unroll
      for (int i = 0; i < kRA; ++i) kf[i] = kread(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NKB * NKK; ++i) {
        const int kb = i % NKB, kk = i / NKB;
        if (i + kRA < NKB * NKK) kf[i + kRA] = kread(i + kRA);
        s[kb] = mfma_bf16(kf[i], qreg[kk], kk == 0 ? (f32x16){} : s[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto m_cluster = [&](int u) __attribute__((always_inline)) {
    // the MFMA wave issues ahead of its softmax partner on the SIMD (the
    // arbiter otherwise favours the older wave, i.e. always group 0)
    __builtin_amdgcn_s_setprio(3);
    if constexpr (BC == 128) {
      pv_part(u);
      qk_part(u);
    } else {
      qk_part(u);
      pv_part(u);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // softmax cluster for tile v: P~(v) into pb, the rescale alpha of O, l
  auto softmax = [&](auto mask_tag, int v) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = v * BC;
    if constexpr (MASK && RANGE) {
      // keys this lane's query row may see (formed here, on edge tiles only,
      // so that it holds no registers through the loop)
      const VisRange vr = vis_range(window > 0 ? (int64_t)my_p - window + 1 : 0, causal ? min(nk - 1, my_p) : nk - 1);
      const uint32_t vo = vis_offset(vr, k0 + 4 * hf);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (!vis(vo, vr, kb * 32 + 8 * (e >> 2) + (e & 3))) s[kb][e] = -INFINITY;
    } else if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
          const bool ok = key < nk && (!causal || key <= my_p) && (window <= 0 || key > my_p - window);
          if (!ok) s[kb][e] = -INFINITY;
        }
    }
    // row max over the lane's 16 NKB scores: four chains of v_max3
    constexpr int NV = 16 * NKB;
    auto sv = [&](int i) __attribute__((always_inline)) { return s[i >> 4][i & 15]; };
    float mp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mp[j] = max3f(sv(3 * j), sv(3 * j + 1), sv(3 * j + 2));
#pragma unroll
    for (int i = 12; i < NV; i += 2) mp[(i / 2) & 3] = max3f(mp[(i / 2) & 3], sv(i), sv(i + 1));
    float mx = max3f(max3f(mp[0], mp[1], mp[2]), mp[3], mp[3]);
    {  // with lane l ^ 32, which holds the rest of the row
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1])) * c;
    }
    const bool up = mx > m + a.lazy;
    alpha = up ? fast_exp2(m - mx) : 1.f;
    m = up ? mx : m;
    float rp[4];  // four partial row sums, each started from its first term
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][e], c, -m));
        s[kb][e] = p;
        const int i = kb * 16 + e;
        rp[i & 3] = i < 4 ? p : rp[i & 3] + p;
      }
    l = l * alpha + ((rp[0] + rp[1]) + (rp[2] + rp[3]));
#pragma unroll
    for (int cc = 0; cc < NKS; ++cc) {
      const int kb = cc >> 1, r0 = (cc & 1) * 8;
      pb[cc].x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
      pb[cc].y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
      pb[cc].z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
      pb[cc].w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
    }
  };
  // softmax cluster at half step hs: issue this wave's DMA blocks of
  // K(t + 1), V(t) with t = jt0 + hs / 2, then the softmax of S(v)
  auto v_cluster = [&](int hs, int v) __attribute__((always_inline)) {
    dma_half(jt0 + (hs >> 1));
    if (v >= jt0 && v < jt1 && active(v)) {
      if (edge(v)) softmax(std::true_type(), v);
      else softmax(std::false_type(), v);
    }
  };

  if (jt0 < jt1) {
    // K(jt0) whole (every wave BPW blocks of each group's half)
    if (!CHAIN || !pre) {
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const uint32_t gk = (uint32_t)(jt0 * BC) * kst2;
        const int q = (wave & 3) * BPW + i + grp * (NBLK / 2);
        dma16_at(kw, lds0 + (uint32_t)(kslot(jt0) * 2 + q * 1024), gk + kgo[i]);
      }
    }
    wait_dma();
    __syncthreads();
    // half step 2 i: group 0 runs M(jt0 + i - 1), group 1 the softmax of
    // tile jt0 + i - 1; half step 2 i + 1: group 0 the softmax of tile
    // jt0 + i, group 1 M(jt0 + i - 1).  The DMA blocks issued in half steps
    // 2 i and 2 i + 1 are read from half step 2 i + 2 on: group 0 waits for
    // its own at the end of its softmax, group 1 at the end of its M.
    const int n = jt1 - jt0;
    if (grp == 0) {
      for (int i = 0; i <= n; ++i) {
        m_cluster(jt0 + i - 1);
        __syncthreads();
        v_cluster(2 * i + 1, jt0 + i);
        wait_dma();
        __syncthreads();
      }
    } else {
      for (int i = 0; i <= n; ++i) {
        v_cluster(2 * i, jt0 + i - 1);
        __syncthreads();
        m_cluster(jt0 + i - 1);
        wait_dma();
        __syncthreads();
      }
    }
  }

  // O staging base: the top of the LDS when the next item's first K tile is
  // already on its way into K slot 0
  constexpr int OST = CHAIN ? kPPLds<D, BC> - 256 * kOP<D> : 0;
  static_assert(!CHAIN || OST >= TS, "staged O must clear K slot 0");
  if constexpr (CHAIN) {
    if (has_next) {
      // the next item's Q fragments and K tile 0 (every K/V slot is free
      // once the loop's last barrier has passed); dense calls only, so the
      // next item shares nq, nk and the strides
      const int q0n = nqt * BR;
      const uint16_t *qbn = (const uint16_t *)a.q + nb * a.q_sb + nh * a.q_sh;
      const __amdgpu_buffer_rsrc_t qrsn = slice_rsrc(qbn, slice_bytes(nq, a.q_st, D, 2));
      const uint32_t qoff = (uint32_t)(q0n + 32 * wave + ql) * (uint32_t)a.q_st * 2 + hf * 16;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) qreg[kk] = bload16(qrsn, qoff + kk * 32);
      const int kv_hin = causal ? min(nk, min(q0n + BR, nq) - 1 + off + 1) : nk;
      if (kv_hin > 0) {
        const uint16_t *kbn = (const uint16_t *)a.k + nb * a.k_sb + nh * a.k_sh;
        const i32x4 kwn = buffer_words(kbn, slice_bytes(nk, a.k_st, D, 2));
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
          const int q = (wave & 3) * BPW + i + grp * (NBLK / 2);
          dma16_at(kwn, lds0 + (uint32_t)(q * 1024), kgo[i]);
        }
      }
    }
  }

  // epilogue: O = acc / l (bf16, round to nearest even), LSE = (m + log2 l) ln 2.
  // O goes through LDS (the K/V tiles are free once the loop's last barrier
  // has passed) so that it leaves as whole 16-byte-per-lane rows: scattered
  // 8-byte pieces of 32 rows per store take several times longer to retire.
  const float lt = half_swap_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  {
    uint16_t *ot = smem + OST + (32 * wave + ql) * kOP<D>;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
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
  for (int i = 0; i < BR * CPR / 512; ++i) {
    const int idx = tid + i * 512, row = idx / CPR, ch = idx % CPR;
    const uint4 v = *(const uint4 *)(smem + OST + row * kOP<D> + ch * 8);
    if (q0 + row < nq) *(uint4 *)(obase + (int64_t)row * a.o_st + ch * 8) = v;
  }
}

// Dense calls with at least one unit per CU run persistently on the static
// schedule of launch_units (paired causal query tiles, XCD-contiguous heads);
// the item body is called from one place, on the kernel's by-value arguments.
// Packed varlen calls with up to kPackedSeqs sequences run persistently too,
// on the schedule that every work-group derives from cu_seqlens
// (packed_schedule_build: units of equal work per sequence, sequences longest
// first, dealt in a snake over XCD-major slots).
template <int D>
__device__ __forceinline__ void pp_varlen_persistent(const FwdArgs &a, uint16_t *smem) {
  __shared__ int s_key[kPackedSeqs], s_order[kPackedSeqs], s_first[kPackedSeqs + 2];
  PackedSchedule ps{s_key, s_order, s_first, a.batch, a.heads};
  packed_schedule_build(ps, a.cu_seqlens, 256, a.causal, a.window);
  for (int i = 0;; ++i) {
    int sq, h, qt;
    const int st = packed_schedule_item(ps, i, a.causal, sq, h, qt);
    if (st < 0) break;
    if (st == 0) continue;
    uint4 qreg[D / 16];
    pp_item<D, true, 64>(a, sq, h, qt, smem, qreg);
    lds_barrier();  // the next item's DMA reuses the LDS that the epilogue read
  }
}

// BC keys per tile: 128 for dense calls without a window (twice the work per
// step over the same fixed costs of each cluster: barrier, first-operand
// latency, DMA issue), 64 for packed and windowed calls, whose edge tiles a
// wider tile would make costlier.
template <int D, int BC>
__global__ __launch_bounds__(512, 2) void fwd_bf16_pp_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kPPLds<D, BC>];  // K ring, V ring / staged O
  if (a.persist == 2) {
    if constexpr (BC == 64) pp_varlen_persistent<D>(a, smem);
    return;
  }
  const UnitRange r = launch_units(a.persist, a.batch, a.heads, a.nqt, a.causal);
  uint4 qreg[D / 16];
  if constexpr (BC == 128) {
    if (a.persist == 1) {
      // the work-group's items in order, each fetching the next one's Q and
      // first K tile under its epilogue
      int u = r.lo, j = 0, b = 0, h = 0, qt = 0;
      auto next = [&](int &nu, int &nj, int &nb, int &nh, int &nqt) __attribute__((always_inline)) {
        for (; nu < r.hi; nu += r.step, nj = 0)
          if (nj < 2 && launch_tile(1, r, nu, nj, a.batch, a.heads, a.nqt, false, a.causal, false, nb, nh, nqt))
            return true;
        return false;
      };
      bool have = next(u, j, b, h, qt), pre = false;
      while (have) {
        int nu = u, nj = j + 1, nb = 0, nh = 0, nqt = 0;
        const bool more = next(nu, nj, nb, nh, nqt);
        pp_item<D, false, BC, true>(a, b, h, qt, smem, qreg, pre, more, nb, nh, nqt);
        lds_barrier();  // the next item's DMA reuses the LDS that the epilogue read
        u = nu, j = nj, b = nb, h = nh, qt = nqt, have = more, pre = more;
      }
      return;
    }
  }
  for (int u = r.lo; u < r.hi; u += r.step)
    for (int j = 0; j < 2; ++j) {
      int b, h, qt;
      if (!launch_tile(a.persist, r, u, j, a.batch, a.heads, a.nqt, a.cu_seqlens != nullptr, a.causal, false, b, h,
                       qt))
        break;
      pp_item<D, false, BC>(a, b, h, qt, smem, qreg);
      lds_barrier();  // the next item's DMA reuses the LDS that the epilogue read
    }
}

// fp32 forward (small workloads): 16 query rows per work-group, and its 4
// waves split the keys: wave w takes key tiles w, w + 4, ..., each with its
// own online softmax state (m, l, O rows), staged through its own LDS slice
// with no work-group barrier, and the four states are merged at the end the
// way partial results over disjoint key sets combine (the merge recurrence of
// "FlashAttention优化Transformer显存与计算效率" section 2.2.2).  A query's dot
// product is split over 4 lanes (one quarter of the head dim each) and
// combined with two lane exchanges.  Key tiles of 32, all arithmetic in fp32
// FMA.  Splitting the keys cuts the serial chain of tiles each wave walks
// (latency-bound at these sizes) by 4.
// x summed over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four quarters of a
// query's dot product) by two lane-half swaps on the VALU; each pair sum is
// formed in the same order on both lanes of the pair.
__device__ __forceinline__ float quarter_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BC = 32, BR = 16, DQ = D / 4, KP = D + 4, NWV = 4;
  __shared__ __attribute__((aligned(16))) float tiles[NWV][2][BC * KP];  // per wave: K, V tile
  __shared__ float s_m[NWV][BR], s_l[NWV][BR];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int qr = lane & 15, quarter = lane >> 4;
  float *ks = tiles[wave][0], *vs = tiles[wave][1];

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
  const float *qbase = (const float *)a.q + b * a.q_sb + (int64_t)seq0 * a.q_st + h * a.q_sh;
  const float *kbase = (const float *)a.k + b * a.k_sb + (int64_t)seq0 * a.k_st + h * a.k_sh;
  const float *vbase = (const float *)a.v + b * a.v_sb + (int64_t)seq0 * a.v_st + h * a.v_sh;

  const int p_lo = q0 + off, p_hi = min(q0 + BR, nq) - 1 + off;
  int kv_lo = 0, kv_hi = nk;
  if (causal) kv_hi = min(nk, p_hi + 1);
  if (window > 0) kv_lo = max(0, p_lo - window + 1);

  const int my_q = q0 + qr;
  const int my_p = my_q + off;
  float qv[DQ], acc[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    qv[e] = my_q < nq ? qbase[(int64_t)my_q * a.q_st + quarter * DQ + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float c = a.scale_log2;

  for (int k0 = (kv_lo / BC + wave) * BC; k0 < kv_hi; k0 += NWV * BC) {
    // this wave's tile: the wave's LDS operations run in order, so its reads
    // of the previous tile come before these stores
    for (int i = lane; i < BC * D / 4; i += 64) {
      const int row = i / (D / 4), col = 4 * (i % (D / 4)), key = k0 + row;
      const float4 z = {0.f, 0.f, 0.f, 0.f};
      *(float4 *)(ks + row * KP + col) = key < nk ? *(const float4 *)(kbase + (int64_t)key * a.k_st + col) : z;
      *(float4 *)(vs + row * KP + col) = key < nk ? *(const float4 *)(vbase + (int64_t)key * a.v_st + col) : z;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the stores are done before the reads below
    __builtin_amdgcn_wave_barrier();
    float sc[BC];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) part = __builtin_fmaf(qv[e], ks[j * KP + quarter * DQ + e], part);
      part = quarter_sum(part);
      const int key = k0 + j;
      const bool ok = key < nk && (!causal || key <= my_p) && (window <= 0 || key > my_p - window);
      sc[j] = ok ? part : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m, mx * c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      sc[j] = exp2f(__builtin_fmaf(sc[j], c, -m_use));
      rs += sc[j];
    }
    l = l * alpha + rs;
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      float t = acc[e] * alpha;
#pragma unroll
      for (int j = 0; j < BC; ++j) t = __builtin_fmaf(sc[j], vs[j * KP + quarter * DQ + e], t);
      acc[e] = t;
    }
    __builtin_amdgcn_wave_barrier();
  }

  // merge the waves' states: M = max m_w, L = sum l_w 2^(m_w - M),
  // O = sum O_w 2^(m_w - M) / L (m in log2 units)
  __syncthreads();  // every wave is done with its tile slice
  float *ost = &tiles[0][0][0];  // [wave][row][D] partial O rows
#pragma unroll
  for (int e = 0; e < DQ; ++e) ost[(wave * BR + qr) * D + quarter * DQ + e] = acc[e];
  if (quarter == 0) {
    s_m[wave][qr] = m;
    s_l[wave][qr] = l;
  }
  __syncthreads();
  // thread t: row t / 16, head dims (t % 16) * D / 16 ...
  constexpr int DT = D / 16;
  const int row = tid / 16, d0 = (tid % 16) * DT;
  const int q = q0 + row;
  if (q < nq) {
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) mm = fmaxf(mm, s_m[w][row]);
    float wgt[NWV], lt = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      wgt[w] = s_m[w][row] == -INFINITY ? 0.f : exp2f(s_m[w][row] - mm);
      lt += s_l[w][row] * wgt[w];
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float *orow = (float *)a.o + b * a.o_sb + (int64_t)(seq0 + q) * a.o_st + h * a.o_sh;
#pragma unroll
    for (int e = 0; e < DT; ++e) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) o = __builtin_fmaf(wgt[w], ost[(w * BR + row) * D + d0 + e], o);
      orow[d0 + e] = o * inv;
    }
    if (tid % 16 == 0 && a.lse)
      a.lse[b * a.lse_sb + h * a.lse_sh + seq0 + q] = lt > 0.f ? (mm + log2f(lt)) * kLn2 : -INFINITY;
  }
}

}  // namespace

// Work-groups of a persistent launch: the current device's CU count, rounded
// down to a multiple of the 8 XCDs (one 512-thread work-group fits per CU);
// 0 if the count cannot be read.
int persistent_groups() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = (n / 8) * 8;
  }
  return cached[dev];
}

int fwd_block_rows(int qkv_dtype, int head_dim, int64_t batch_heads, int64_t nq, bool causal, bool varlen,
                   int cus) {
  (void)head_dim;
  if (qkv_dtype == 0) return 16;  // fp32 kernel: 16 rows, the keys split over 4 waves
  if (qkv_dtype != 1) return 256;  // fp8 kernel
  const int64_t want = cus > 0 ? cus : 256;
  // 256 rows where that launch runs persistently (dense causal calls pair
  // their tiles, so they need twice the tiles): below that, CUs idle behind
  // the longest work-groups, and 128-row tiles measured faster
  const int64_t t256 = (nq + 255) / 256;
  if (batch_heads * (causal && !varlen ? (t256 + 1) / 2 : t256) >= want) return 256;
  if (batch_heads * ((nq + 127) / 128) >= want) return 128;
  return 64;
}

template <int D, int NW>
void launch_drop_kernel(const FwdArgs &p, dim3 g, hipStream_t s) {
  if (p.drop_k) hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, true>), g, dim3(NW * 64), 0, s, p);
  else hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, false>), g, dim3(NW * 64), 0, s, p);
}

hipError_t launch_fwd_bf16(const FwdArgs &a, int head_dim, hipStream_t s) {
  FwdArgs p = a;
  dim3 g((unsigned)(a.nqt * a.heads * a.batch));
  const int cus = persistent_groups();
  const int64_t units = (int64_t)a.batch * a.heads * (a.causal ? (a.nqt + 1) / 2 : a.nqt);
  p.persist = !a.cu_seqlens && cus >= 8 && units >= cus;
  if (p.persist) g = dim3((unsigned)cus);
  if (a.br < 256) {
    // short sequences: 4 or 2 waves of 32 rows per work-group, one work item each
    if (a.br == 128) {
      if (head_dim == 128) launch_drop_kernel<128, 4>(p, g, s);
      else launch_drop_kernel<64, 4>(p, g, s);
    } else {
      if (head_dim == 128) launch_drop_kernel<128, 2>(p, g, s);
      else launch_drop_kernel<64, 2>(p, g, s);
    }
  } else if (a.drop_k) {
    if (head_dim == 128) hipLaunchKernelGGL((fwd_bf16_kernel<128, 8, true>), g, dim3(512), 0, s, p);
    else hipLaunchKernelGGL((fwd_bf16_kernel<64, 8, true>), g, dim3(512), 0, s, p);
  } else {
    // packed calls: persistent with a schedule derived on the device
    if (a.cu_seqlens && cus >= 8 && a.batch <= kPackedSeqs) {
      p.persist = 2;
      g = dim3((unsigned)cus);
    }
    const bool wide = !a.cu_seqlens && a.window <= 0;
    if (head_dim == 128) {
      if (wide) hipLaunchKernelGGL((fwd_bf16_pp_kernel<128, 128>), g, dim3(512), 0, s, p);
      else hipLaunchKernelGGL((fwd_bf16_pp_kernel<128, 64>), g, dim3(512), 0, s, p);
    } else {
      if (wide) hipLaunchKernelGGL((fwd_bf16_pp_kernel<64, 128>), g, dim3(512), 0, s, p);
      else hipLaunchKernelGGL((fwd_bf16_pp_kernel<64, 64>), g, dim3(512), 0, s, p);
    }
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
