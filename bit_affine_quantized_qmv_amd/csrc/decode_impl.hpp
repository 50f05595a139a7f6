// Decode family (up to 32 activation rows): y = x . dequant(W)^T, per output element
//     y[m,n] = sum_g ( s[n,g] * sum_{k in g} x[m,k] q[n,k]  +  b[n,g] * sum_{k in g} x[m,k] )
// (MLX pull request 4516, first commit: the bias term multiplies a sum of the inputs, and
// every input is widened to float before it is added).
//
// Arithmetic of one output element, identical in every kernel of this family and for any
// number of activation rows (so a batched call is bitwise equal to single-row calls, the
// property transformers issue 47331 asks for under "Expected behavior"):
//   * sum_{k in g} x q   : chain of 16x16x32 MFMAs over the group's 32-k steps, codes given
//                          as exact bf16/fp16 integers, fresh accumulator per group;
//   * acc = fma(s, sum xq, acc), group by group in k order;
//   * sum_{k in g} x     : the same MFMA chain against an all-ones operand (each x widened
//                          by the matrix core, accumulated in float32), once per call;
//   * after the scale updates of one weight slot (1, 2 or 4 groups), the slot's bias terms
//     b * sum x in one float32 16x16x4 MFMA whose k index is the group (unused k lanes
//     carry b = 0), accumulated into acc;
//   * one round-to-nearest-even to the output dtype.
// Activation rows past the call's row count are zero in LDS; weight rows past N are read
// as row N-1 (or as zeros, through a range-checked buffer descriptor) and never stored
// (MLX pull request 4516: affine_qmv_fast_rows keeps the reduction loop free of per-row
// checks).
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace qmm {
namespace decode {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

// v_permlane32_swap: the upper 32 lanes of the first operand trade places with the lower
// 32 lanes of the second.  v_permlane16_swap: odd 16-lane rows of the first operand trade
// places with even rows of the second.
__device__ inline u32x4 swap_halves(u32x4 u) {
  auto r0 = __builtin_amdgcn_permlane32_swap(u.x, u.z, false, false);
  auto r1 = __builtin_amdgcn_permlane32_swap(u.y, u.w, false, false);
  u32x4 o = {r0[0], r1[0], r0[1], r1[1]};
  return o;
}
// Lane group g holds words 4g .. 4g+3 of a 16-word slice; afterwards register c of lane
// group g holds word 4c + g (a 4x4 transpose across the four 16-lane groups).
__device__ inline u32x4 transpose_lane_groups(u32x4 u) {
  u = swap_halves(u);
  auto r0 = __builtin_amdgcn_permlane16_swap(u.x, u.y, false, false);
  auto r1 = __builtin_amdgcn_permlane16_swap(u.z, u.w, false, false);
  u32x4 o = {r0[0], r0[1], r1[0], r1[1]};
  return o;
}

// Lane group (16 lanes) feeding sub-block `sub` (8 consecutive k) of a 32-k MFMA step.
// 8-bit words arrive through swap_halves, which puts sub-blocks 1 and 2 on groups 2 and 1.
template <int BITS>
__device__ inline int lane_group_of_sub(int sub) {
  if (BITS == 8) return sub == 1 ? 2 : (sub == 2 ? 1 : sub);
  return sub;
}

// Compile-time shape of one "slot": the k span covered by one round of weight loads.
template <int BITS, int GS>
struct Slot {
  // 4-bit: one 16-byte load per lane = 128 k of a row across the 4 lane groups.
  // 8-bit: one 16-byte load per lane = 64 k; groups of 32 and 128 take two (128 k), groups
  // of 64 one (the finer parts of 64-k slots measured faster for short rows there).
  // other widths: two words per lane per 32-k step, 128 k per slot at every group size.
  // A slot then carries up to four groups, whose bias terms share one bias MFMA, and the
  // per-slot loop overhead is paid once per 128 codes.
  static constexpr int kSpan = BITS == 8 && GS == 64 ? 64 : 128;
  static constexpr int kSteps = kSpan / 32;
  static constexpr int kGroups = kSpan / GS;                       // groups ending in a slot
  static constexpr int kVec = BITS == 4 ? 1 : (BITS == 8 ? kSpan / 64 : 0);   // u32x4 loads
  static constexpr int kWords = BITS == 4 || BITS == 8 ? 4 * kVec : 2 * kSteps;  // regs of codes
  static constexpr int kRowWordsPerSlot = kSpan * BITS / 32;
};

// Whether a slot's KG scale (or bias) halfwords of a row can be read as one load: every
// row's, every expert's and both arrays' starts aligned to 2 * KG bytes.  Otherwise the
// kernels read them one halfword at a time.
template <int KG>
__device__ inline bool sb_rows_aligned(const MatArgs& a) {
  if constexpr (KG == 1) {
    return true;
  } else {
    constexpr uint64_t w = 2 * KG;
    return (((uintptr_t)a.scales | (uintptr_t)a.biases) % w) == 0 && (uint64_t)(a.sb_row_stride * 2) % w == 0 &&
           (uint64_t)(a.sb_expert_stride * 2) % w == 0;
  }
}

// Scale or bias values (raw 16-bit patterns) of NH consecutive groups of one weight row,
// two per register.  get(h): halfword h (compile-time h).  lane_half<KG>(base, lg): the
// value a lane feeds as k index lg of a bias MFMA covering the KG groups starting at
// halfword `base`; 0 for lg >= KG.
template <int NH>
struct SbRegs {
  uint32_t v[(NH + 1) / 2];
  __device__ uint32_t get(int h) const { return (v[h >> 1] >> (16 * (h & 1))) & 0xFFFFu; }
  template <int KG>
  __device__ uint32_t lane_half(int base, int lg) const {
    if constexpr (KG == 1) {
      return lg == 0 ? get(base) : 0u;
    } else if constexpr (KG == 2) {   // base is even
      return lg < 2 ? (v[base >> 1] >> (16 * lg)) & 0xFFFFu : 0u;
    } else {                          // KG == 4, base a multiple of 4
      // an arithmetic select: a conditional one can become a dynamically indexed (scratch) array
      const uint32_t lo = v[base >> 1], hi = v[(base >> 1) + 1];
      const uint32_t w = lo ^ ((lo ^ hi) & (0u - (uint32_t)((lg >> 1) & 1)));
      return (w >> (16 * (lg & 1))) & 0xFFFFu;
    }
  }
};

// N halfwords of a row's scales or biases; with `valid` < N (the row's last slot when K is
// not a multiple of the slot span) only the first `valid` are read, the rest are zero.
template <int N>
__device__ inline SbRegs<N> load_sb_part(const uint16_t* p, int valid) {
  SbRegs<N> r;
#pragma unroll
  for (int i = 0; i < (N + 1) / 2; ++i) {
    const uint32_t lo = 2 * i < valid ? p[2 * i] : 0u;
    const uint32_t hi = 2 * i + 1 < N && 2 * i + 1 < valid ? p[2 * i + 1] : 0u;
    r.v[i] = lo | (hi << 16);
  }
  return r;
}

template <int N>
__device__ inline SbRegs<N> load_sb(const uint16_t* p) {
  SbRegs<N> r;
  if constexpr (N == 1) {
    r.v[0] = *p;
  } else if constexpr (N == 2) {
    r.v[0] = *(const uint32_t*)p;
  } else {
    const uint2 u = *(const uint2*)p;
    r.v[0] = u.x;
    r.v[1] = u.y;
  }
  return r;
}

// NH halfwords at byte offset voff + soff of a buffer, NH * 2 in {2, 4, 8} bytes or a
// multiple of 16 (the offset is aligned to the load width).
template <int NH>
__device__ inline void load_sb_buf(SbRegs<NH>& r, __amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  if constexpr (NH == 1) {
    r.v[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0);
  } else if constexpr (NH == 2) {
    r.v[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
  } else if constexpr (NH == 4) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
    r.v[0] = u[0];
    r.v[1] = u[1];
  } else {
    static_assert(NH % 8 == 0, "scale/bias block loads are 2, 4, 8 or 16*k bytes");
#pragma unroll
    for (int i = 0; i < NH / 8; ++i) {
      const auto u = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * i, soff, 0);
      r.v[4 * i + 0] = u[0];
      r.v[4 * i + 1] = u[1];
      r.v[4 * i + 2] = u[2];
      r.v[4 * i + 3] = u[3];
    }
  }
}

template <int BITS, int GS>
struct SlotData {
  static constexpr bool kVecCodes = BITS == 4 || BITS == 8;
  u32x4 v[kVecCodes ? Slot<BITS, GS>::kVec : 1];          // 4/8-bit codes, 16-byte loads as issued
  uint32_t w[kVecCodes ? 1 : Slot<BITS, GS>::kWords];     // other widths
  SbRegs<Slot<BITS, GS>::kGroups> s, b;
};

// Issue the loads of one slot: weight row `wrow` (already offset to the slot's first word),
// scales/biases at `srow`/`brow` (offset to the slot's first group).  `lg` = lane group.
template <int BITS, int GS>
__device__ inline void load_slot(SlotData<BITS, GS>& d, const uint32_t* wrow, const uint16_t* srow,
                                 const uint16_t* brow, int lg, int generic_word, int row_words_left,
                                 int codes_left, bool sb_narrow) {
  using S = Slot<BITS, GS>;
  if constexpr (BITS == 4 || BITS == 8) {
    // a lane's 16 bytes hold 32 (4-bit) or 16 (8-bit) consecutive codes; past the row's end
    // (the last slot when K is not a multiple of the span) they are zero and nothing is read
    constexpr int kLaneCodes = BITS == 4 ? 32 : 16;
#pragma unroll
    for (int v = 0; v < S::kVec; ++v) {
      const int c0 = (4 * v + lg) * kLaneCodes;
      d.v[v] = c0 < codes_left ? *(const u32x4*)(wrow + 16 * v + 4 * lg) : u32x4{0u, 0u, 0u, 0u};
    }
  } else {
#pragma unroll
    for (int c = 0; c < S::kSteps; ++c) {
      const int idx = c * BITS + generic_word;
      d.w[2 * c] = wrow[idx];
      // the high word is only needed when the 8 codes straddle it; never read past the row
      d.w[2 * c + 1] = wrow[min(idx + 1, row_words_left - 1)];
    }
  }
  // halfword loads when the scale rows are not a whole number of the slot's groups (the
  // vector loads would be misaligned) or the slot ends past K (neither can happen with one
  // group per slot: the slot is then the group)
  if (S::kGroups == 1 || (!sb_narrow && codes_left >= S::kSpan)) {
    d.s = load_sb<S::kGroups>(srow);
    d.b = load_sb<S::kGroups>(brow);
  } else {
    const int valid = codes_left / GS < S::kGroups ? codes_left / GS : S::kGroups;
    d.s = load_sb_part<S::kGroups>(srow, valid);
    d.b = load_sb_part<S::kGroups>(brow, valid);
  }
}

// Buffer-descriptor variant of load_slot: `w_rs`, `s_rs`, `b_rs` describe the rows of a
// tile pair (rows outside the range read as zero); the lane's row offset is in `w_voff` /
// `sb_voff` (bytes), the slot's offset inside the row in `w_soff` / `sb_soff`.  With
// WITH_SB false the scales and biases are loaded per block elsewhere.
// With `sb_narrow` (scale rows not a whole number of the slot's groups, or a last slot that
// ends past K) the scales and biases are read one halfword at a time: every halfword is then
// aligned and range-checked on its own, so one past the described rows cannot zero a valid
// neighbour in the same dword.
template <int NH>
__device__ inline void load_sb_buf_narrow(SbRegs<NH>& r, __amdgpu_buffer_rsrc_t rs, int voff, int soff) {
#pragma unroll
  for (int i = 0; i < (NH + 1) / 2; ++i) {
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, voff + 4 * i, soff, 0);
    const uint32_t hi = 2 * i + 1 < NH ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, voff + 4 * i + 2, soff, 0)
                                       : 0u;
    r.v[i] = lo | (hi << 16);
  }
}

template <int BITS, int GS, bool WITH_SB>
__device__ inline void load_slot_buf(SlotData<BITS, GS>& d, __amdgpu_buffer_rsrc_t w_rs,
                                     __amdgpu_buffer_rsrc_t s_rs, __amdgpu_buffer_rsrc_t b_rs, int w_voff,
                                     int w_soff, int sb_voff, int sb_soff, bool sb_narrow = false) {
  using S = Slot<BITS, GS>;
  static_assert(BITS == 4 || BITS == 8, "buffer path is for 4- and 8-bit codes");
#pragma unroll
  for (int v = 0; v < S::kVec; ++v) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b128(w_rs, w_voff + 64 * v, w_soff, 0);
    d.v[v] = u32x4{u[0], u[1], u[2], u[3]};
  }
  if constexpr (WITH_SB) {
    if (sb_narrow) {
      load_sb_buf_narrow<S::kGroups>(d.s, s_rs, sb_voff, sb_soff);
      load_sb_buf_narrow<S::kGroups>(d.b, b_rs, sb_voff, sb_soff);
    } else {
      load_sb_buf<S::kGroups>(d.s, s_rs, sb_voff, sb_soff);
      load_sb_buf<S::kGroups>(d.b, b_rs, sb_voff, sb_soff);
    }
  }
}

// Raw buffer descriptor (gfx9 family word 3) over [base, base + bytes).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Codes of one slot after the cross-lane reordering that follows the loads: 4-bit words
// transposed across lane groups, 8-bit halves swapped; other widths unchanged.  The ring
// registers themselves are never rewritten, so a refill can target them directly.
template <int BITS, int GS>
struct SlotCodes {
  u32x4 v[SlotData<BITS, GS>::kVecCodes ? Slot<BITS, GS>::kVec : 1];
};

template <int BITS, int GS>
__device__ inline SlotCodes<BITS, GS> slot_reorder(const SlotData<BITS, GS>& d) {
  SlotCodes<BITS, GS> r;
  if constexpr (BITS == 4) {
    r.v[0] = transpose_lane_groups(d.v[0]);
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int v = 0; v < Slot<BITS, GS>::kVec; ++v) r.v[v] = swap_halves(d.v[v]);
  }
  return r;
}

// Exact code values of MFMA step c of a slot, in operand order.
template <class T, int BITS, int GS>
__device__ inline u32x4 slot_codes(const SlotData<BITS, GS>& d, const SlotCodes<BITS, GS>& r, int c,
                                   uint32_t generic_shift) {
  if constexpr (BITS == 4) {
    return codes4_to_v8<T>(r.v[0][c]);
  } else if constexpr (BITS == 8) {
    const int v = c >> 1;
    return (c & 1) ? codes8_to_v8<T>(r.v[v].z, r.v[v].w) : codes8_to_v8<T>(r.v[v].x, r.v[v].y);
  } else {
    return codesN_to_v8<T, BITS>(d.w[2 * c], d.w[2 * c + 1], generic_shift);
  }
}

// Per-lane constants of the generic (2/3/5/6-bit) unpacker: word offset and bit shift of
// lane group lg's 8 codes inside a 32-k step.
template <int BITS>
__device__ inline void generic_lane_offsets(int lg, int& word, uint32_t& shift) {
  const int bit0 = 8 * lg * BITS;
  word = bit0 >> 5;
  shift = (uint32_t)(bit0 & 31);
}

// Staging of activation rows [0, XR) x k in [k_begin, k_begin + k_len) into LDS in MFMA
// operand order: entry ((step * 4 + lane_group) * XR + m) holds 8 values.  XR = 2^xrl LDS
// rows (x_lds_rows_log2): all 16 * MT rows of the tiles, or the call's single row; operand
// reads for tile row r use LDS row r mod XR, so rows of the tile past XR repeat earlier
// rows, and their results are never stored.
//
// Thread t always handles activation row m = t % XR (the thread count is a multiple of
// XR) and 8-k chunks j8 = t / XR, t / XR + nthreads / XR, ...  Loads are issued
// in batches of kStageBatch with clamped (always valid) addresses and no branches, so a
// caller can issue a batch, then other loads, and only then wait for the batch: the memory
// counter retires loads in issue order, and a load issued after the weight prefetch would
// make the activation staging wait for the whole prefetch.
constexpr int kStageBatch = 8;

template <int MROWS>
struct XStage {
  u32x4 v[kStageBatch];
};

// log2 of the activation rows staged in LDS for a call of `rows` rows (see above): two tiles
// stage all 32 rows, one tile all 16 rows or, for a single activation row, that row alone
// (so single-row calls fit in LDS up to K of about 64K); the launcher also stages 8 rows
// for 2-8 rows whose 16-row staging does not fit.  A template parameter of the kernels, so
// the operand addresses stay compile-time offsets.
template <int MT>
__host__ __device__ constexpr int x_lds_rows_log2(int rows) {
  return MT != 1 ? 5 : (rows == 1 ? 0 : 4);
}

template <class T, int BITS, int MROWS>
__device__ inline const uint16_t* stage_row(const MatArgs& a, const uint16_t* xb, int rows, int tid, int xrl) {
  const int m = tid & ((1 << xrl) - 1);
  const int mr = m < rows ? m : 0;   // rows past the call's rows read row 0, stored as zero
  // decode calls have at most 32 rows, so the segment arithmetic fits 32-bit integers
  const uint32_t sr = a.seg_rows < MROWS ? (uint32_t)a.seg_rows : (uint32_t)MROWS;
  const uint32_t seg = (uint32_t)mr / sr;
  return xb + (int64_t)seg * a.seg_stride + (int64_t)((uint32_t)mr - seg * sr) * a.row_stride;
}

template <class T, int BITS, int MROWS>
__device__ inline void stage_x_issue(XStage<MROWS>& st, const uint16_t* xr, int k_begin, int k_len, int batch,
                                     int tid, int nthreads, int rows, int xrl) {
  const int c8 = k_len >> 3;
  const int per = nthreads >> xrl;        // chunks advanced per pass
  const int j0 = (tid >> xrl) + batch * kStageBatch * per;
  const bool live = (tid & ((1 << xrl) - 1)) < rows;   // padding rows are stored as zero without a load
#pragma unroll
  for (int b = 0; b < kStageBatch; ++b) {
    int j8 = j0 + b * per;
    j8 = j8 < c8 ? j8 : 0;
    st.v[b] = live ? *(const u32x4*)(xr + k_begin + 8 * j8) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <class T, int BITS, int MROWS>
__device__ inline void stage_x_commit(const XStage<MROWS>& st, u32x4* xs, int rows, int k_len, int batch, int tid,
                                      int nthreads, int xrl) {
  const int c8 = k_len >> 3;
  const int per = nthreads >> xrl;
  const int m = tid & ((1 << xrl) - 1);
  const int j0 = (tid >> xrl) + batch * kStageBatch * per;
#pragma unroll
  for (int b = 0; b < kStageBatch; ++b) {
    const int j8 = j0 + b * per;
    if (j8 < c8) {
      u32x4 u = m < rows ? st.v[b] : u32x4{0u, 0u, 0u, 0u};
      if (BITS == 4) u = interleave_even_odd(u);
      xs[(((j8 >> 2) * 4 + lane_group_of_sub<BITS>(j8 & 3)) << xrl) + m] = u;
    }
  }
}

// Zero the staged activations between k_len and k_pad (the last slot's k past K when K is
// not a multiple of the slot span), so their products with whatever codes are loaded there
// vanish.
template <int BITS>
__device__ inline void zero_x_pad(u32x4* xs, int k_len, int k_pad, int tid, int nthreads, int xrl) {
  const int per = nthreads >> xrl;
  const int m = tid & ((1 << xrl) - 1);
  for (int j8 = (k_len >> 3) + (tid >> xrl); j8 < (k_pad >> 3); j8 += per)
    xs[(((j8 >> 2) * 4 + lane_group_of_sub<BITS>(j8 & 3)) << xrl) + m] = u32x4{0u, 0u, 0u, 0u};
}

// Number of staging batches for a chunk of k_len.
__device__ inline int stage_batches(int k_len, int nthreads, int xrl) {
  const int per = nthreads >> xrl;
  const int c8 = k_len >> 3;
  return (c8 + kStageBatch * per - 1) / (kStageBatch * per);
}

// Whole staging in one call (used where nothing is in flight that must not be waited for).
template <class T, int BITS, int MROWS>
__device__ inline void stage_x(u32x4* xs, const MatArgs& a, const uint16_t* xb, int rows, int k_begin,
                               int k_len, int tid, int nthreads, int xrl) {
  const uint16_t* xr = stage_row<T, BITS, MROWS>(a, xb, rows, tid, xrl);
  const int nb = stage_batches(k_len, nthreads, xrl);
  for (int batch = 0; batch < nb; ++batch) {
    XStage<MROWS> st;
    stage_x_issue<T, BITS, MROWS>(st, xr, k_begin, k_len, batch, tid, nthreads, rows, xrl);
    stage_x_commit<T, BITS, MROWS>(st, xs, rows, k_len, batch, tid, nthreads, xrl);
  }
}

// Per (row, group) sums of the staged activations: MFMA against an all-ones operand, one
// chain per (16-row tile, group), shared out over the workgroup's waves.  Layout
// sxs[g * XR + m] for the XR staged rows; callers keep kSxPad zero groups after the last one,
// which the bias MFMA of the final slot reads on its unused k lanes.
constexpr int kSxPad = 3;

// Floats of the Σx area for ng groups and 2^xrl staged rows (with the padding groups), rounded
// up to whole 16-byte units so that the 8-byte argmax keys (updated with 64-bit LDS atomics)
// and the 16-byte hand-off entries placed after it are aligned.
__host__ __device__ inline int sx_floats(int ng, int xrl) { return (((ng + kSxPad) << xrl) + 3) & ~3; }

__device__ inline void zero_sx_pad(float* sxs, int ng, int tid, int xrl) {
  if (tid < (kSxPad << xrl)) sxs[(ng << xrl) + tid] = 0.f;
}

template <class T, int GS, int MT>
__device__ inline void sum_x(const u32x4* xs, float* sxs, int k_len, int wave, int nwaves, int lane, int xrl) {
  constexpr int SPG = GS / 32;
  const int xmask = (1 << xrl) - 1;
  const int lg = lane >> 4, col = lane & 15;
  const int ng = k_len / GS;
  const uint32_t one2 = T::pack2(1.0f, 1.0f);
  const u32x4 ones = {one2, one2, one2, one2};
#pragma unroll 4
  for (int p = wave; p < MT * ng; p += nwaves) {
    const int mt = p / ng, g = p - mt * ng;
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < SPG; ++c)
      d = T::mfma(as_v8<T>(xs[(((g * SPG + c) * 4 + lg) << xrl) + ((mt * 16 + col) & xmask)]), as_v8<T>(ones), d);
    if (col == 0) {
      if (mt * 16 + 4 * lg + 3 <= xmask) {
        *(f32x4*)&sxs[(g << xrl) + mt * 16 + 4 * lg] = d;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mt * 16 + 4 * lg + r <= xmask) sxs[(g << xrl) + mt * 16 + 4 * lg + r] = d[r];
      }
    }
  }
}

// Consume one slot of TN 16-row weight tiles: MFMAs of its steps (each activation operand
// read from LDS once and used for every tile), the scale update at each group end, then the
// slot's bias terms on the float32 matrix core.  k_local = k offset of the slot inside the
// staged activation chunk.
// Scales and biases come from `sc` / `bi` (NH halfwords per tile), the slot's groups
// starting at halfword `hbase`.
// Bias terms of up to four consecutive groups starting at group g0, one fp32 MFMA per
// (tile, 16-row block): A[m][k] = sum x of row m in group g0 + k, B[k][n] = b[n][g0 + k], with
// bh[t] the bias halfword lane group lg feeds for tile t (zero on the k lanes past the groups
// covered; their A values are the next groups' sums or the zero padding, finite either way).
template <class T, int MT, int TN>
__device__ inline void bias_mfma(const uint32_t (&bh)[TN], const float* sxs, int g0, f32x4 (&acc)[TN][MT], int lg,
                                 int col, int xrl) {
  float sxa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) sxa[mt] = sxs[((g0 + lg) << xrl) + ((mt * 16 + col) & ((1 << xrl) - 1))];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const float bv = T::to_f32(bh[t]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sxa[mt], bv, acc[t][mt], 0, 0, 0);
  }
}

// The bias halfword lane group lg feeds when one bias MFMA covers two consecutive slots of
// KG groups each (2*KG <= 4): the first slot's groups on lanes 0..KG-1, the second's next.
template <int KG>
__device__ inline uint32_t pair_lane_half(const SbRegs<KG>& first, const SbRegs<KG>& second, int lg) {
  const int h = lg < KG ? lg : lg - KG;
  const uint32_t v = lg < KG ? first.get(h & (KG - 1)) : second.get(h & (KG - 1));
  return lg < 2 * KG ? v : 0u;
}

// Slots per bias MFMA, the same in every decode kernel so that they agree bit for bit: two
// when the groups are 64 or 128 codes (two or one per 128-code slot) and the slots per
// row are even, else one.
template <int GS>
__device__ inline int bias_span(int slots_per_row) {
  return (GS >= 64 && slots_per_row % 2 == 0) ? 2 : 1;
}

// Rows of the weight a call reads from: N, or N per expert times the experts of a stack.
__host__ __device__ inline int64_t weight_rows(const MatArgs& a) {
  return a.w_index ? a.N * a.num_experts : a.N;
}

// Sub-block size (slots) the decode kernels use for a row of nit slots.
__host__ __device__ inline int block_slots(int nit) { return nit % 2 == 0 ? 2 : 1; }

// Parts per row, a function of K, the weight's row count (N, times the experts of a gathered
// stack), the code width and the group size only, so every decode kernel sums a row the same
// way (part sums in k order, then added part by part) for every row count and plan of a call
// on that weight.  P is the power of two <= 8 (parts of at least one sub-block) that
// minimises a cost model of the launch: tile pairs are spread over at most 256 workgroups
// of 8 waves, G = 8 / P pairs per workgroup and round, and a round costs a fixed overhead
// (the parts' hand-off, 4 slot-equivalents) plus the slots one wave walks; ties go to more
// parts.  P = 1 is the streaming kernel (whole rows per wave).  Few rows and long K get
// many parts, many rows get whole rows per wave (the lm_head shape), e.g. one 16-row tile of
// a K = 1024, 4-bit weight: 4 parts of 2 slots; N = 14336, K = 4096: 4 parts of 8 slots,
// 224 workgroups of two pairs in one round (8 parts needed 1.75 rounds over 256).
template <int BITS, int GS>
__host__ __device__ inline int row_parts(int64_t K, int64_t N) {
  const int nit = (int)((K + Slot<BITS, GS>::kSpan - 1) / Slot<BITS, GS>::kSpan);
  const int d = block_slots(nit);
  const int64_t n_pairs = ((N + 15) / 16 + 1) / 2;
  int best_p = 1;
  int64_t best_t = -1;
  for (int p = 1; p <= 8; p *= 2) {
    if (p > 1 && p * d > nit) break;
    const int spp = p == 1 ? nit : (nit + p * d - 1) / (p * d) * d;
    const int64_t g = 8 / p;
    const int64_t wgs = (n_pairs + g - 1) / g < 256 ? (n_pairs + g - 1) / g : 256;
    const int64_t rounds = (n_pairs + g * wgs - 1) / (g * wgs);
    const int64_t t = rounds * (4 + spp);
    if (best_t < 0 || t <= best_t) {
      best_t = t;
      best_p = p;
    }
  }
  return best_p;
}

template <int BITS, int GS>
__host__ __device__ inline int part_slots(int64_t K, int64_t N) {
  const int nit = (int)((K + Slot<BITS, GS>::kSpan - 1) / Slot<BITS, GS>::kSpan);
  const int p = row_parts<BITS, GS>(K, N), d = block_slots(nit);
  return (nit + p * d - 1) / (p * d) * d;
}


template <class T, int BITS, int GS, int MT, int TN, int NH, bool BIAS = true>
__device__ inline void consume_slot(const SlotData<BITS, GS> (&d)[TN], const SbRegs<NH> (&sc)[TN],
                                    const SbRegs<NH> (&bi)[TN], int hbase, const u32x4* xs, const float* sxs,
                                    int k_local, int k_valid, f32x4 (&acc)[TN][MT], f32x4 (&part)[TN][MT], int lg,
                                    int col, uint32_t generic_shift, int xrl) {
  using S = Slot<BITS, GS>;
  constexpr int SPG = GS / 32;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  SlotCodes<BITS, GS> rc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) rc[t] = slot_reorder<BITS, GS>(d[t]);
  const int step0 = k_local >> 5;
#pragma unroll
  for (int c = 0; c < S::kSteps; ++c) {
    typename T::v8 bq[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) bq[t] = as_v8<T>(slot_codes<T, BITS, GS>(d[t], rc[t], c, generic_shift));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const typename T::v8 av = as_v8<T>(xs[(((step0 + c) * 4 + lg) << xrl) + ((mt * 16 + col) & ((1 << xrl) - 1))]);
#pragma unroll
      for (int t = 0; t < TN; ++t) part[t][mt] = T::mfma(av, bq[t], (c % SPG) == 0 ? zero4 : part[t][mt]);
    }
    if ((c + 1) % SPG == 0) {
      const int gi = c / SPG;
      // groups past K (the last slot when K is not a multiple of the span) scale by zero:
      // their products are zero and their loaded scales need not be finite
      const bool g_ok = k_local + gi * GS < k_valid;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const float sv = g_ok ? T::to_f32(sc[t].get(hbase + gi)) : 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][mt][r] = __builtin_fmaf(sv, part[t][mt][r], acc[t][mt][r]);
      }
    }
  }
  if constexpr (BIAS) {
    const bool g_ok = (k_local / GS + lg) * GS < k_valid;
    uint32_t bh[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) bh[t] = g_ok ? bi[t].template lane_half<S::kGroups>(hbase, lg) : 0u;
    bias_mfma<T, MT, TN>(bh, sxs, k_local / GS, acc, lg, col, xrl);
  }
}

// Weight, scale and bias bases of grid batch z: the call's own, or those of the expert the
// batch's index selects (index out of range -> expert 0 is read, and *bad is set so the
// caller stores NaN).
struct WeightBase {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  bool bad;
};

__device__ inline WeightBase weight_base(const MatArgs& a, int64_t z) {
  WeightBase r{a.w, (const uint16_t*)a.scales, (const uint16_t*)a.biases, false};
  if (a.w_index) {
    const int e = __builtin_amdgcn_readfirstlane(a.w_index[z]);
    r.bad = e < 0 || e >= a.num_experts;
    const int64_t ec = r.bad ? 0 : e;
    r.w += ec * a.w_expert_stride;
    r.s += ec * a.sb_expert_stride;
    r.b += ec * a.sb_expert_stride;
  }
  return r;
}

// ---- fused argmax.  A key orders (value, column) pairs: the value's float32 bits mapped to
// an unsigned order (NaN above everything) in the high half, the complement of the column in
// the low half, so the largest key is the largest value and, among equal values, the
// smallest column -- the first maximum, as an argmax returns it.
__device__ inline unsigned long long argmax_key(float v, int64_t n) {
  uint32_t b = __float_as_uint(v);
  if (v != v) b = 0x7FC00000u;
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)n);
}

// Fold one tile's values (rows mt*16 + 4*lg + r, column n) into the lane's running keys;
// the value is the one stored in y (rounded to the output dtype).
template <class T, int MT>
__device__ inline void argmax_update(unsigned long long (&best)[MT][4], const f32x4 (&acc)[MT], int64_t n,
                                     bool valid) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const unsigned long long k = argmax_key(T::to_f32(T::from_f32(acc[mt][r])), n);
      best[mt][r] = (valid && k > best[mt][r]) ? k : best[mt][r];
    }
}

__device__ inline unsigned long long shfl_xor_u64(unsigned long long v, int mask) {
  const uint32_t lo = __shfl_xor((uint32_t)v, mask), hi = __shfl_xor((uint32_t)(v >> 32), mask);
  return ((unsigned long long)hi << 32) | lo;
}

// Merge a workgroup's key for one row into the global key (a device-scope atomic maximum;
// argmax_complete orders it before the workgroup counts itself done).
__device__ inline void argmax_publish(unsigned long long* key, unsigned long long v) {
  __hip_atomic_fetch_max(key, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Completion of the fused argmax inside the decode kernel.  Every thread's key merges
// (argmax_publish) happen before the workgroup barrier, which happens before thread 0's count;
// the count is an acquire-release read-modify-write at device scope, whose release half orders
// the whole workgroup's merges before it (one L2 write-back per workgroup rather than one per
// wave); the last workgroup to count issues an acquire fence at device scope in every thread
// before it reads the keys.  That workgroup turns each row's key into (index, value) and sets the
// keys and the counter back to zero, so the workspace is all-zero again when the kernel
// ends.  `last` is a workgroup-shared word that is free once every thread has arrived here
// (it is first written after the barrier below).  Called by every thread.
__device__ inline void argmax_complete(const MatArgs& a, int64_t total_rows, unsigned* last) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned wgs = gridDim.x * gridDim.y * gridDim.z;
    const unsigned done = __hip_atomic_fetch_add(a.argmax_count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *last = done + 1 == wgs ? 1u : 0u;
  }
  __syncthreads();
  if (*last == 0u) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int64_t i = threadIdx.x; i < total_rows; i += blockDim.x) {
    const unsigned long long k =
        __hip_atomic_exchange(&a.argmax_keys[i], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ord = (uint32_t)(k >> 32);
    a.argmax_index[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
    if (a.argmax_value) a.argmax_value[i] = __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
  }
  if (threadIdx.x == 0) __hip_atomic_store(a.argmax_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reduce the wave's keys over the 16 columns of each lane group and merge them into the
// workgroup's LDS keys `kl` (MROWS entries).
template <int MT>
__device__ inline void argmax_merge_wave(unsigned long long (&best)[MT][4], unsigned long long* kl, int lg, int col) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      unsigned long long k = best[mt][r];
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        const unsigned long long o = shfl_xor_u64(k, m);
        k = o > k ? o : k;
      }
      if (col == 0) atomicMax(&kl[mt * 16 + 4 * lg + r], k);
    }
}

template <int MT>
__device__ inline void poison(f32x4 (&acc)[MT]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
}

template <class T, int MT>
__device__ inline void store_tile(const f32x4 (&acc)[MT], uint16_t* yb, int rows, int64_t n, int64_t N,
                                  int lg) {
  if (n >= N) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mt * 16 + 4 * lg + r;
      if (m < rows) yb[(int64_t)m * N + n] = T::from_f32(acc[mt][r]);
    }
}

// The outputs of a whole tile pair (both tiles' rows below N, N a multiple of 8, y 16-byte
// aligned) pass through an LDS area of 16 * MT activation rows x kYAreaStride halfwords per
// pair: the MFMA layout (4 activation rows of one column per lane) becomes 8 consecutive
// columns of one activation row per lane, so the pair takes 16-byte stores (2 * MT per lane
// instead of 8 * MT 2-byte ones).  The padded row stride spreads the four lane groups'
// 2-byte writes over distinct banks.  A wave's area holds either one pair (stored right
// away) or every pair of its range (stored after its weight stream ends, so no output
// store waits in the wave's memory queue ahead of the weight refills).
constexpr int kYAreaStride = 40;
template <int MT>
constexpr int y_pair_halves() { return 16 * MT * kYAreaStride; }
template <int MT>
constexpr int y_area_bytes(int waves, int pairs) { return waves * pairs * y_pair_halves<MT>() * 2; }

template <class T, int MT>
__device__ inline void stage_pair_lds(const f32x4 (&acc)[2][MT], uint16_t* area, int lg, int col) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) area[(mt * 16 + 4 * lg + r) * kYAreaStride + t * 16 + col] = T::from_f32(acc[t][mt][r]);
}

// the area is the wave's own: its LDS accesses complete in order, the fences only keep the
// compiler from moving them across one another
__device__ inline void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int MT>
__device__ inline void flush_pair_lds(uint16_t* yb, int rows, int64_t n0, int64_t N, const uint16_t* area,
                                      int lane) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane >> 2);
    const int c = lane & 3;
    const u32x4 v = *(const u32x4*)(area + m * kYAreaStride + c * 8);
    if (m < rows) *(u32x4*)(yb + (int64_t)m * N + n0 + c * 8) = v;
  }
}

template <class T, int MT>
__device__ inline void store_pair_lds(const f32x4 (&acc)[2][MT], uint16_t* yb, int rows, int64_t n0, int64_t N,
                                      uint16_t* area, int lane, int lg, int col) {
  stage_pair_lds<T, MT>(acc, area, lg, col);
  wave_lds_order();
  flush_pair_lds<MT>(yb, rows, n0, N, area, lane);
  wave_lds_order();
}

}  // namespace decode
}  // namespace qmm
