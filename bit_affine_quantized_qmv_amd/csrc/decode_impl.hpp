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
//   * sum_{k in g} x     : the same MFMA chain against an all-ones operand (each x widened
//                          by the matrix core, accumulated in float32);
//   * acc = fma(s, sum xq, acc); acc = fma(b, sum x, acc), group by group in k order;
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
  // 8-bit: one 16-byte load per lane = 64 k; group 128 takes two.
  // other widths: two words per lane per 32-k step.
  static constexpr int kSpan = BITS == 4 ? 128 : (BITS == 8 ? (GS == 128 ? 128 : 64) : GS);
  static constexpr int kSteps = kSpan / 32;
  static constexpr int kGroups = kSpan / GS;                       // groups ending in a slot
  static constexpr int kVec = BITS == 4 ? 1 : (BITS == 8 ? kSpan / 64 : 0);   // u32x4 loads
  static constexpr int kWords = BITS == 4 || BITS == 8 ? 4 * kVec : 2 * kSteps;  // regs of codes
  static constexpr int kRowWordsPerSlot = kSpan * BITS / 32;
};

template <int N>
struct SbRegs;  // scale or bias values of the groups in a slot, raw 16-bit patterns
template <>
struct SbRegs<1> { uint16_t v; __device__ uint32_t get(int) const { return v; } };
template <>
struct SbRegs<2> { uint32_t v; __device__ uint32_t get(int i) const { return (v >> (16 * i)) & 0xFFFFu; } };
template <>
struct SbRegs<4> {
  uint32_t v0, v1;
  __device__ uint32_t get(int i) const { return ((i < 2 ? v0 : v1) >> (16 * (i & 1))) & 0xFFFFu; }
};

template <int N>
__device__ inline SbRegs<N> load_sb(const uint16_t* p) {
  SbRegs<N> r;
  if constexpr (N == 1) {
    r.v = *p;
  } else if constexpr (N == 2) {
    r.v = *(const uint32_t*)p;
  } else {
    const uint2 u = *(const uint2*)p;
    r.v0 = u.x;
    r.v1 = u.y;
  }
  return r;
}

template <int BITS, int GS>
struct SlotData {
  uint32_t w[Slot<BITS, GS>::kWords];
  SbRegs<Slot<BITS, GS>::kGroups> s, b;
};

// Issue the loads of one slot: weight row `wrow` (already offset to the slot's first word),
// scales/biases at `srow`/`brow` (offset to the slot's first group).  `lg` = lane group.
template <int BITS, int GS>
__device__ inline void load_slot(SlotData<BITS, GS>& d, const uint32_t* wrow, const uint16_t* srow,
                                 const uint16_t* brow, int lg, int generic_word, int row_words_left) {
  using S = Slot<BITS, GS>;
  if constexpr (BITS == 4 || BITS == 8) {
#pragma unroll
    for (int v = 0; v < S::kVec; ++v) {
      const u32x4 u = *(const u32x4*)(wrow + 16 * v + 4 * lg);
      d.w[4 * v + 0] = u.x;
      d.w[4 * v + 1] = u.y;
      d.w[4 * v + 2] = u.z;
      d.w[4 * v + 3] = u.w;
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
  d.s = load_sb<S::kGroups>(srow);
  d.b = load_sb<S::kGroups>(brow);
}

// Buffer-descriptor variant of load_slot: `w_rs`, `s_rs`, `b_rs` describe one 16-row tile
// (rows past N lie outside the descriptor's range and read as zero); the lane's row offset
// is in `w_voff` / `sb_voff` (bytes), the slot's offset inside the row in `w_soff` / `sb_soff`.
template <int BITS, int GS>
__device__ inline void load_slot_buf(SlotData<BITS, GS>& d, __amdgpu_buffer_rsrc_t w_rs,
                                     __amdgpu_buffer_rsrc_t s_rs, __amdgpu_buffer_rsrc_t b_rs, int w_voff,
                                     int w_soff, int sb_voff, int sb_soff) {
  using S = Slot<BITS, GS>;
  static_assert(BITS == 4 || BITS == 8, "buffer path is for 4- and 8-bit codes");
#pragma unroll
  for (int v = 0; v < S::kVec; ++v) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b128(w_rs, w_voff + 64 * v, w_soff, 0);
    d.w[4 * v + 0] = u[0];
    d.w[4 * v + 1] = u[1];
    d.w[4 * v + 2] = u[2];
    d.w[4 * v + 3] = u[3];
  }
  if constexpr (S::kGroups == 1) {
    d.s.v = __builtin_amdgcn_raw_buffer_load_b16(s_rs, sb_voff, sb_soff, 0);
    d.b.v = __builtin_amdgcn_raw_buffer_load_b16(b_rs, sb_voff, sb_soff, 0);
  } else if constexpr (S::kGroups == 2) {
    d.s.v = __builtin_amdgcn_raw_buffer_load_b32(s_rs, sb_voff, sb_soff, 0);
    d.b.v = __builtin_amdgcn_raw_buffer_load_b32(b_rs, sb_voff, sb_soff, 0);
  } else {
    const auto sv = __builtin_amdgcn_raw_buffer_load_b64(s_rs, sb_voff, sb_soff, 0);
    const auto bv = __builtin_amdgcn_raw_buffer_load_b64(b_rs, sb_voff, sb_soff, 0);
    d.s.v0 = sv[0];
    d.s.v1 = sv[1];
    d.b.v0 = bv[0];
    d.b.v1 = bv[1];
  }
}

// Raw buffer descriptor (gfx9 family word 3) over [base, base + bytes).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Exact code values of MFMA step c of a slot, in operand order.
template <class T, int BITS, int GS>
__device__ inline u32x4 slot_codes(const SlotData<BITS, GS>& d, int c, uint32_t generic_shift) {
  if constexpr (BITS == 4) {
    return codes4_to_v8<T>(d.w[c]);
  } else if constexpr (BITS == 8) {
    const int v = c >> 1;
    return (c & 1) ? codes8_to_v8<T>(d.w[4 * v + 2], d.w[4 * v + 3])
                   : codes8_to_v8<T>(d.w[4 * v + 0], d.w[4 * v + 1]);
  } else {
    return codesN_to_v8<T, BITS>(d.w[2 * c], d.w[2 * c + 1], generic_shift);
  }
}

// Cross-lane reordering that follows the loads (done right before use).
template <int BITS, int GS>
__device__ inline void slot_reorder(SlotData<BITS, GS>& d) {
  if constexpr (BITS == 4) {
    u32x4 u = {d.w[0], d.w[1], d.w[2], d.w[3]};
    u = transpose_lane_groups(u);
    d.w[0] = u.x; d.w[1] = u.y; d.w[2] = u.z; d.w[3] = u.w;
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int v = 0; v < Slot<BITS, GS>::kVec; ++v) {
      u32x4 u = {d.w[4 * v], d.w[4 * v + 1], d.w[4 * v + 2], d.w[4 * v + 3]};
      u = swap_halves(u);
      d.w[4 * v] = u.x; d.w[4 * v + 1] = u.y; d.w[4 * v + 2] = u.z; d.w[4 * v + 3] = u.w;
    }
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

// Staging of activation rows [0, MROWS) x k in [k_begin, k_begin + k_len) into LDS in MFMA
// operand order: entry ((step * 4 + lane_group) * MROWS + m) holds 8 values.
//
// Thread t always handles activation row m = t % MROWS (the thread count is a multiple of
// MROWS) and 8-k chunks j8 = t / MROWS, t / MROWS + nthreads / MROWS, ...  Loads are issued
// in batches of kStageBatch with clamped (always valid) addresses and no branches, so a
// caller can issue a batch, then other loads, and only then wait for the batch: the memory
// counter retires loads in issue order, and a load issued after the weight prefetch would
// make the activation staging wait for the whole prefetch.
constexpr int kStageBatch = 8;

template <int MROWS>
struct XStage {
  u32x4 v[kStageBatch];
};

template <class T, int BITS, int MROWS>
__device__ inline const uint16_t* stage_row(const MatArgs& a, const uint16_t* xb, int rows, int tid) {
  const int m = tid % MROWS;
  const int mr = m < rows ? m : 0;   // rows past the call's rows read row 0, stored as zero
  return xb + (mr / a.seg_rows) * a.seg_stride + (mr % a.seg_rows) * a.row_stride;
}

template <class T, int BITS, int MROWS>
__device__ inline void stage_x_issue(XStage<MROWS>& st, const uint16_t* xr, int k_begin, int k_len, int batch,
                                     int tid, int nthreads) {
  const int c8 = k_len >> 3;
  const int per = nthreads / MROWS;       // chunks advanced per pass
  const int j0 = tid / MROWS + batch * kStageBatch * per;
#pragma unroll
  for (int b = 0; b < kStageBatch; ++b) {
    int j8 = j0 + b * per;
    j8 = j8 < c8 ? j8 : 0;
    st.v[b] = *(const u32x4*)(xr + k_begin + 8 * j8);
  }
}

template <class T, int BITS, int MROWS>
__device__ inline void stage_x_commit(const XStage<MROWS>& st, u32x4* xs, int rows, int k_len, int batch, int tid,
                                      int nthreads) {
  const int c8 = k_len >> 3;
  const int per = nthreads / MROWS;
  const int m = tid % MROWS;
  const int j0 = tid / MROWS + batch * kStageBatch * per;
#pragma unroll
  for (int b = 0; b < kStageBatch; ++b) {
    const int j8 = j0 + b * per;
    if (j8 < c8) {
      u32x4 u = m < rows ? st.v[b] : u32x4{0u, 0u, 0u, 0u};
      if (BITS == 4) u = interleave_even_odd(u);
      xs[((j8 >> 2) * 4 + lane_group_of_sub<BITS>(j8 & 3)) * MROWS + m] = u;
    }
  }
}

// Number of staging batches for a chunk of k_len.
template <int MROWS>
__device__ inline int stage_batches(int k_len, int nthreads) {
  const int per = nthreads / MROWS;
  const int c8 = k_len >> 3;
  return (c8 + kStageBatch * per - 1) / (kStageBatch * per);
}

// Whole staging in one call (used where nothing is in flight that must not be waited for).
template <class T, int BITS, int MROWS>
__device__ inline void stage_x(u32x4* xs, const MatArgs& a, const uint16_t* xb, int rows, int k_begin,
                               int k_len, int tid, int nthreads) {
  const uint16_t* xr = stage_row<T, BITS, MROWS>(a, xb, rows, tid);
  const int nb = stage_batches<MROWS>(k_len, nthreads);
  for (int batch = 0; batch < nb; ++batch) {
    XStage<MROWS> st;
    stage_x_issue<T, BITS, MROWS>(st, xr, k_begin, k_len, batch, tid, nthreads);
    stage_x_commit<T, BITS, MROWS>(st, xs, rows, k_len, batch, tid, nthreads);
  }
}

// Per (row, group) sums of the staged activations: MFMA against an all-ones operand, one
// chain per (16-row tile, group), shared out over the workgroup's waves.
template <class T, int GS, int MT>
__device__ inline void sum_x(const u32x4* xs, float* sxs, int k_len, int wave, int nwaves, int lane) {
  constexpr int MROWS = 16 * MT;
  constexpr int SPG = GS / 32;
  const int lg = lane >> 4, col = lane & 15;
  const int ng = k_len / GS;
  const uint32_t one2 = T::pack2(1.0f, 1.0f);
  const u32x4 ones = {one2, one2, one2, one2};
  for (int p = wave; p < MT * ng; p += nwaves) {
    const int mt = p / ng, g = p - mt * ng;
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < SPG; ++c)
      d = T::mfma(as_v8<T>(xs[((g * SPG + c) * 4 + lg) * MROWS + mt * 16 + col]), as_v8<T>(ones), d);
    if (col == 0) *(f32x4*)&sxs[g * MROWS + mt * 16 + 4 * lg] = d;
  }
}

// Consume one slot: MFMAs of its steps, and the scale/bias update at each group end.
// k_local = k offset of the slot inside the staged activation chunk.
template <class T, int BITS, int GS, int MT>
__device__ inline void consume_slot(SlotData<BITS, GS>& d, const u32x4* xs, const float* sxs, int k_local,
                                    f32x4 (&acc)[MT], f32x4 (&part)[MT], int lg, int col,
                                    uint32_t generic_shift) {
  using S = Slot<BITS, GS>;
  constexpr int MROWS = 16 * MT;
  constexpr int SPG = GS / 32;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  slot_reorder<BITS, GS>(d);
  const int step0 = k_local >> 5;
#pragma unroll
  for (int c = 0; c < S::kSteps; ++c) {
    const typename T::v8 bq = as_v8<T>(slot_codes<T, BITS, GS>(d, c, generic_shift));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const typename T::v8 av = as_v8<T>(xs[((step0 + c) * 4 + lg) * MROWS + mt * 16 + col]);
      part[mt] = T::mfma(av, bq, (c % SPG) == 0 ? zero4 : part[mt]);
    }
    if ((c + 1) % SPG == 0) {
      const int gi = c / SPG;
      const float sv = T::to_f32(d.s.get(gi));
      const float bv = T::to_f32(d.b.get(gi));
      const int gl = k_local / GS + gi;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 sx = *(const f32x4*)&sxs[gl * MROWS + mt * 16 + 4 * lg];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[mt][r] = __builtin_fmaf(sv, part[mt][r], acc[mt][r]);
          acc[mt][r] = __builtin_fmaf(bv, sx[r], acc[mt][r]);
        }
      }
    }
  }
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

}  // namespace decode
}  // namespace qmm
