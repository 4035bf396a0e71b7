// Device-side helpers shared by the forward and backward kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_bf16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over one (batch, head) slice.  Loads whose byte offset
// lies at or beyond `bytes` return zeros, which is how rows past the end of a
// sequence are zero-filled without any predication.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Bytes spanned by rows 0..n-1 of width w elements at row stride st.
__device__ __forceinline__ uint32_t slice_bytes(int n, int64_t st, int w, int elem) {
  return n > 0 ? (uint32_t)(((int64_t)(n - 1) * st + w) * elem) : 0u;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t u16_at(const uint4 &v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Combine a per-lane value with the one in lane l ^ 32 (the other half of a
// 32x32 accumulator column): v_permlane32_swap exchanges the halves, and the
// pair {own, other} comes back in some order, which max and + ignore.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, the four 16-bit values
// lane l receives are element (l % 4) of the 8-byte chunks addressed by
// lanes (l % 16) / 4 + 4 j of its group, j = 0..3 (measured on gfx950).
// Used to read MFMA operands "down the columns" of a row-major LDS tile.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
  return __builtin_bit_cast(uint2, r);
}

// Row-major bf16 tiles of 64 rows x D elements that are read both along rows
// (ds_read_b128, 16 rows per pass) and down columns (ds_read_b64_tr_b16) are
// stored without padding, their 16-byte chunks XOR-swizzled per row:
// physical chunk = chunk ^ swz(row).  These swizzles make both read patterns
// and the staging writes bank-conflict free (checked exhaustively on a CPU
// model of the 64 LDS banks).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128)
    return 4 * (row & 3) + ((row >> 2) & 3);
  else
    return 4 * ((row >> 1) & 1) + ((row >> 2) & 1) + 2 * ((row >> 3) & 1);
}
// element offset of 16-byte chunk `chunk` of row `row`
template <int D>
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * D + ((chunk ^ swz<D>(row)) << 3);
}
// Per-lane element offsets of the transposed operand reads from a swizzled
// tile: lane s reads rows 16 cc + 8 half + 4 (s / 32) + (s % 16) / 4 at
// column 32 db + 16 ((s / 16) % 2) + 4 (s % 4); the swizzle of those rows
// does not depend on cc, so the offset for (db, half) is a per-lane constant
// and cc adds 16 cc D.
template <int D>
__device__ __forceinline__ int tr_off(int lane, int db, int half) {
  const int row = 8 * half + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  return swz_off<D>(row, chunk) + 4 * (lane & 1);
}

// Buffer resource words for LDS DMA: `bytes` bytes from `base`, raw
// (stride 0), so offsets at or past `bytes` read as zeros.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_words(const void *base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return (i32x4){(int)(uint32_t)p, (int)((p >> 32) & 0xffff), (int)bytes, 0x00020000};
}
// Wait for this wave's LDS DMA.  The builtin (not inline asm) lets the
// compiler's own load tracking see every vector load complete here: with an
// asm wait, register loads issued before it (the Q fragments) stayed
// "pending" in that tracking across the main loop, and the compiler waited
// for them inside the loop, which at run time also waited for the DMA of the
// next tiles in flight.  The empty asm keeps LDS reads from moving above it.
__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0; expcnt, lgkmcnt unchanged (7, 15)
  asm volatile("" ::: "memory");
}
// LDS DMA of 16 bytes per lane: the 16 bytes at byte offset `off` of the
// buffer described by `r` land at LDS byte address lds_byte + 16 * lane
// (lds_byte must be wave-uniform); offsets past the end of the buffer
// deliver zeros.  Issued from inline assembly so the compiler does not wait
// for its completion before unrelated LDS reads; callers wait with
// wait_dma() and a barrier before anything reads the destination.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_at(i32x4 r, uint32_t lds_byte, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_byte), "v"(off), "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// MFMA issued from inline assembly with the register file of every operand
// pinned (accumulators of O in AGPRs, S in VGPRs, persistent B operands in
// AGPRs), so the compiler never shuttles them between files.  The compiler
// does not see these as MFMAs, so the waits the hardware does not enforce
// are the caller's: an MFMA result is read by any other instruction only
// after mfma_drain*() (the hardware needs >= 11 wait states after an 8-pass
// XDL op such as v_mfma_f32_32x32x16_bf16; the drains give 16), and a VALU
// write of an operand precedes its MFMA read by >= 2 wait states.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 vec4(const uint4 &x) { return (u32x4){x.x, x.y, x.z, x.w}; }
__device__ __forceinline__ void mfma_a(f32x16 &acc, const uint4 &a, const uint4 &b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(vec4(a)), "v"(vec4(b)));
}
__device__ __forceinline__ void mfma_v_first(f32x16 &d, const uint4 &a, const u32x4 &b_agpr) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(vec4(a)), "a"(b_agpr));
}
__device__ __forceinline__ void mfma_v(f32x16 &d, const uint4 &a, const u32x4 &b_agpr) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(vec4(a)), "a"(b_agpr));
}
__device__ __forceinline__ void mfma_drain2_v(f32x16 &x, f32x16 &y) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void mfma_drain_a(f32x16 &x) { asm volatile("s_nop 7\n\ts_nop 7" : "+a"(x)); }

// XCD-aware renumbering of the linear block id: the hardware hands
// consecutive block ids to the 8 XCDs in turn, so XCD x sees ids x, x+8, ...;
// map them to one contiguous range of logical items per XCD so that items
// sharing data (the query tiles of one head) share that XCD's L2.
__device__ __forceinline__ int xcd_item(int bid, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
}

// Work item of forward work-group bid: (batch or sequence b, head h, query
// tile qt).  Each XCD processes a contiguous range of items.  Dense calls
// are (b, h)-major, so an XCD holds whole heads and their K/V stay in its
// L2.  Packed varlen calls are head-major: every XCD then gets the same mix
// of sequence lengths (sequence-major ranges would hand one XCD the longest
// sequences).  Causal items run heaviest (last) query tile first.
__device__ __forceinline__ void fwd_item(int bid, int nqt, int heads, int batch, bool varlen, bool causal, int &b,
                                         int &h, int &qt) {
  const int item = xcd_item(bid, nqt * heads * batch);
  const int t = item % nqt;
  if (varlen) {
    const int hb = item / nqt;
    h = hb / batch;
    b = hb % batch;
  } else {
    const int bh = item / nqt;
    b = bh / heads;
    h = bh % heads;
  }
  qt = causal ? nqt - 1 - t : t;
}

// ---------------------------------------------------------------------------
// Static schedule of a persistent launch (one work-group per CU, the grid a
// multiple of the 8 XCDs).  Work is cut into units of one (batch, head) and
// either one tile or, under a causal mask, the pair of tiles i and n - 1 - i,
// which together carry as much work as any other pair.  XCD x = blockIdx % 8
// owns the contiguous unit range [x U / 8, (x + 1) U / 8) (a few heads, so
// their K/V stay in its L2) and its work-groups take every (G / 8)-th unit.
// A static schedule has no dispatch gaps: the hardware hands out work-groups
// in block order over the XCDs, so with one work-group per item a CU that
// frees up early can idle until the next block's XCD has room.
// Without `persist` the same loop runs the one item of fwd_item(blockIdx).
// ---------------------------------------------------------------------------
struct UnitRange {
  int lo, hi, step, per;  // units [lo, hi) by step; units per (batch, head)
};
__device__ __forceinline__ UnitRange launch_units(bool persist, int batch, int heads, int ntiles, bool pair) {
  if (!persist) return {0, 1, 1, 1};
  const int per = pair ? (ntiles + 1) / 2 : ntiles;
  const int units = batch * heads * per;
  const int xcd = blockIdx.x % 8;
  return {(int)((int64_t)units * xcd / 8) + (int)(blockIdx.x / 8), (int)((int64_t)units * (xcd + 1) / 8),
          (int)(gridDim.x / 8), per};
}
// tile j (0, 1) of unit u, the heavier one first; false if there is none.
// heavy_low: low tile indices carry the most work (key tiles under a causal
// mask) rather than high ones (query tiles).
__device__ __forceinline__ bool launch_tile(bool persist, const UnitRange &r, int u, int j, int batch, int heads,
                                            int ntiles, bool varlen, bool causal, bool heavy_low, int &b, int &h,
                                            int &t) {
  if (!persist) {
    fwd_item(blockIdx.x, ntiles, heads, batch, varlen, causal && !heavy_low, b, h, t);
    return j == 0;
  }
  const int bh = u / r.per, i = u % r.per;
  b = bh / heads;
  h = bh % heads;
  if (!causal) {
    t = i;
    return j == 0;
  }
  const int heavy = heavy_low ? i : ntiles - 1 - i, light = ntiles - 1 - heavy;
  t = j == 0 ? heavy : light;
  return j == 0 || heavy != light;
}

// ---------------------------------------------------------------------------
// Persistent schedule of a packed (cu_seqlens) call over query tiles, derived
// on the device.  The host does not know the sequence lengths, so every
// work-group builds the same tables in LDS: tiles of `rows` rows per
// sequence, sequences ranked longest first, and the first unit of each ranked
// sequence.  A unit is one query tile, or two tiles whose work adds up to that
// of one full tile:
//   - under a causal mask, tile qt sees qt + 1 tiles' worth of keys until the
//     window (if any) caps it; with F the first tile the window caps (F = all
//     tiles without a window), tiles qt >= F are single units of the full
//     window, and the tiles below F pair up as (f - 1 - i, i), f = min(F, n),
//     which together see f + 1 tiles' worth, as much as one full tile (the
//     plain causal case pairs n - 1 - i with i);
//   - without a causal mask every tile is a unit.
// So the units of one sequence carry equal work, and ranked longest first the
// list decreases.  Unit k goes to slot k mod 2G, or 2G - 1 - (k mod 2G) on the
// way back (a snake over decreasing unit sizes, close to longest-processing-
// time first); slots are numbered XCD-major (slot = (block % 8) G / 8 +
// block / 8), so consecutive units, those of one (sequence, head), share an
// XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kPackedSeqs = 512;  // packed calls with more sequences take one work-group per item
struct PackedSchedule {
  int *key;    // [kPackedSeqs] tiles of sequence i
  int *order;  // [kPackedSeqs] sequences, longest first
  int *first;  // [kPackedSeqs + 2] first unit of each ranked sequence; then F
  int nseq, heads;
  int units = 0, fcap = 0;  // fcap: tiles below it pair up (0: none)
};
// Units of a sequence of nt tiles: full single tiles, then pairs.
__device__ __forceinline__ int packed_units(int nt, int fcap) {
  const int f = min(fcap, nt);
  return nt - f + (f + 1) / 2;
}
// All threads of the work-group; ends with a barrier.
__device__ __forceinline__ void packed_schedule_build(PackedSchedule &ps, const int32_t *cu, int rows, bool causal,
                                                      int window) {
  const int tid = threadIdx.x, nseq = ps.nseq;
  for (int i = tid; i < nseq; i += blockDim.x) ps.key[i] = max(0, cu[i + 1] - cu[i] + rows - 1) / rows;
  __syncthreads();
  for (int i = tid; i < nseq; i += blockDim.x) {
    const int ki = ps.key[i];
    int rank = 0;
    for (int j = 0; j < nseq; ++j) {
      const int kj = ps.key[j];
      rank += kj > ki || (kj == ki && j < i);
    }
    ps.order[rank] = i;
  }
  __syncthreads();
  if (tid == 0) {
    // tile qt sees the whole window iff qt rows >= window - 1
    int fcap = 0;
    if (causal) fcap = window > 0 ? (int)min((int64_t)0x7FFFFFFF, ((int64_t)window - 1 + rows - 1) / rows) : 0x7FFFFFFF;
    int acc = 0;
    for (int r = 0; r < nseq; ++r) {
      ps.first[r] = acc;
      acc += ps.heads * packed_units(ps.key[ps.order[r]], fcap);
    }
    ps.first[nseq] = acc;
    ps.first[nseq + 1] = fcap;
  }
  __syncthreads();
  ps.units = ps.first[nseq];
  ps.fcap = ps.first[nseq + 1];
}
// Item i (0, 1, ...) of this work-group: 1 and (seq, head, tile) for an
// item, 0 for a slot with nothing to do, -1 when the work-group is done.
// The full tiles of a sequence come highest first, then the pairs, the
// higher tile of each first.
__device__ __forceinline__ int packed_schedule_item(const PackedSchedule &ps, int i, bool causal, int &seq, int &h,
                                                    int &tile) {
  const int G = gridDim.x, slot = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
  const int lap = i >> 2, e = i & 3;  // e / 2: outward or return slot of the lap; e % 2: tile of a pair
  const int k0 = lap * 2 * G;
  if (k0 >= ps.units) return -1;
  const int k = k0 + ((e >> 1) == 0 ? slot : 2 * G - 1 - slot);
  if (k >= ps.units) return 0;
  int lo = 0, hi = ps.nseq;  // the ranked sequence r with first[r] <= k < first[r + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ps.first[mid] <= k) lo = mid;
    else hi = mid;
  }
  seq = ps.order[lo];
  const int nt = ps.key[seq], f = min(ps.fcap, nt), per = nt - f + (f + 1) / 2;
  const int local = k - ps.first[lo], u = local % per;
  h = local / per;
  if (u < nt - f) {  // a full tile
    if (e & 1) return 0;
    tile = causal ? nt - 1 - u : u;
    return 1;
  }
  const int j = u - (nt - f), hi_t = f - 1 - j;
  if (e & 1) {
    if (hi_t == j) return 0;  // the middle tile stands alone
    tile = j;
  } else {
    tile = hi_t;
  }
  return 1;
}

// Work-group barrier for LDS reuse only: waits for this wave's LDS accesses,
// not for its global stores to retire (__syncthreads would wait for both).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// max of three floats in one v_max3_f32.  fmaxf compiles to v_max3_f32 too,
// but first quiets a possible signalling NaN in every operand it cannot prove
// canonical (MFMA results among them) with an extra v_max_f32 x, x; no input
// here is a signalling NaN, so those are skipped.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// half_swap_max through max3f: the row max with lane l ^ 32, without the
// NaN-quieting instructions that fmaxf adds
__device__ __forceinline__ float swap_max3(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------------------
// Masks as index ranges.  The causal, window and length limits leave each row
// (or column) an inclusive range [lo, hi] of visible partner positions.  With
// lo >= 0 and hi < 2^31, position base + c lies in it iff the unsigned 32-bit
// value c - (lo - base) is at most hi - lo: per element one subtract from a
// constant and one compare, where testing the limits one by one costs three
// compares and their combination.  An empty range is lo = 2^31, span 0, which
// no position below 2^31 passes.
// ---------------------------------------------------------------------------
struct VisRange {
  uint32_t lo, span;
};
__device__ __forceinline__ VisRange vis_range(int64_t lo, int64_t hi) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > 0x7FFFFFFF ? 0x7FFFFFFF : hi;
  if (hi < lo) return {0x80000000u, 0u};
  return {(uint32_t)lo, (uint32_t)(hi - lo)};
}
// lo - base, computed once per tile
__device__ __forceinline__ uint32_t vis_offset(const VisRange &v, int base) { return v.lo - (uint32_t)base; }
__device__ __forceinline__ bool vis(uint32_t offset, const VisRange &v, int c) {
  return (uint32_t)c - offset <= v.span;
}

// ---------------------------------------------------------------------------
// Dropout randomness: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011).  Each round multiplies words
// 0 and 2 by 0xD2511F53 / 0xCD9E8D57 into 64-bit products and forms
// (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is bumped by the Weyl
// constants 0x9E3779B9 / 0xBB67AE85 between rounds.
//
// The attention element (query row i, key j) of head slot b * heads + h
// draws byte (j & 3) of word ((j & 31) >> 3) of the call with counter
// (2 (j >> 5) + ((j >> 2) & 1), i, slot, offset): one call covers the 16
// elements that one lane half holds of a 32-key block in the MFMA
// accumulator layout (keys 8 (r / 4) + 4 hf + r % 4, r = 0..15), so lane
// half hf of key block kb makes exactly one call.  The element is kept iff
// its byte < drop_k.
// ---------------------------------------------------------------------------
struct Philox {
  uint32_t c[4];
};

// Each product is formed as one 64-bit multiply of zero-extended words, which
// compiles to a single v_mad_u64_u32 (both halves at once) instead of a low
// and a high 32-bit multiply: 28% more calls per second on gfx950.
__device__ __forceinline__ void philox_round(Philox &x, uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * x.c[0], p1 = (uint64_t)0xCD9E8D57u * x.c[2];
  x.c[0] = (uint32_t)(p1 >> 32) ^ x.c[1] ^ k0;
  x.c[1] = (uint32_t)p1;
  x.c[2] = (uint32_t)(p0 >> 32) ^ x.c[3] ^ k1;
  x.c[3] = (uint32_t)p0;
}

// Key of round r (0-based).
__device__ __forceinline__ uint32_t philox_k0(uint32_t seed_lo, int r) { return seed_lo + 0x9E3779B9u * (uint32_t)r; }
__device__ __forceinline__ uint32_t philox_k1(uint32_t seed_hi, int r) { return seed_hi + 0xBB67AE85u * (uint32_t)r; }

__device__ __forceinline__ Philox philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t seed_lo,
                                           uint32_t seed_hi) {
  Philox x{{c0, c1, c2, c3}};
#pragma unroll
  for (int r = 0; r < 10; ++r) philox_round(x, philox_k0(seed_lo, r), philox_k1(seed_hi, r));
  return x;
}

// Keep flag of accumulator element r (0..15) from its call's output.
__device__ __forceinline__ bool drop_keep(const Philox &x, int r, uint32_t drop_k) {
  return ((x.c[r >> 2] >> (8 * (r & 3))) & 0xFFu) < drop_k;
}

}  // namespace dev
}  // namespace fa
