// Dequantization of 32-code runs, shared by the prefill kernel (which stages w~ in LDS) and
// the standalone dequantize / embedding kernels.
//
// w~ = RNE_dtype(fl32(fma(s, q, b))): one float32 fused multiply-add, then one rounding to
// the storage dtype.
#pragma once

#include "device_common.hpp"

namespace qmm {

// BITS consecutive code words (32 codes) of one weight row, starting at a 32-code boundary.
template <int BITS>
__device__ inline void load_codes(uint32_t (&w)[BITS], const uint32_t* p) {
  if constexpr (BITS % 4 == 0) {
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) {
      const u32x4 u = *(const u32x4*)(p + 4 * i);
      w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
    }
  } else if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int i = 0; i < BITS / 2; ++i) {
      const uint2 u = *(const uint2*)(p + 2 * i);
      w[2 * i] = u.x; w[2 * i + 1] = u.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = p[i];
  }
}

// 32 codes -> w~ = RNE_dtype(fma(s, q, b)) as four 8-value MFMA operand chunks, k order.
template <class T, int BITS>
__device__ inline void dequant32(const uint32_t (&w)[BITS], float s, float b, u32x4 (&out)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float q[8];
    if constexpr (BITS == 4) {
      // nibbles to bytes, then the fp8 conversion: byte patterns 0..15 are c * 2^-9 in e4m3
      const uint32_t even = w[c] & 0x0F0F0F0Fu, odd = (w[c] >> 4) & 0x0F0F0F0Fu;
      const auto e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(even, 512.0f, false);
      const auto e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(even, 512.0f, true);
      const auto o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(odd, 512.0f, false);
      const auto o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(odd, 512.0f, true);
      q[0] = e0[0]; q[2] = e0[1]; q[4] = e1[0]; q[6] = e1[1];
      q[1] = o0[0]; q[3] = o0[1]; q[5] = o1[0]; q[7] = o1[1];
    } else if constexpr (BITS == 8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q[e] = (float)((w[2 * c] >> (8 * e)) & 0xFFu);
        q[4 + e] = (float)((w[2 * c + 1] >> (8 * e)) & 0xFFu);
      }
    } else {
      // codes 8c .. 8c+7 start at bit 8*c*BITS of the 32-code run
      const int bit0 = 8 * c * BITS;
      const uint32_t lo = w[bit0 >> 5];
      const uint32_t hi = (bit0 >> 5) + 1 < BITS ? w[(bit0 >> 5) + 1] : 0u;
      const uint64_t v = ((((uint64_t)hi) << 32) | lo) >> (bit0 & 31);
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = (float)((uint32_t)(v >> (e * BITS)) & ((1u << BITS) - 1u));
    }
    out[c].x = T::pack2(__builtin_fmaf(s, q[0], b), __builtin_fmaf(s, q[1], b));
    out[c].y = T::pack2(__builtin_fmaf(s, q[2], b), __builtin_fmaf(s, q[3], b));
    out[c].z = T::pack2(__builtin_fmaf(s, q[4], b), __builtin_fmaf(s, q[5], b));
    out[c].w = T::pack2(__builtin_fmaf(s, q[6], b), __builtin_fmaf(s, q[7], b));
  }
}

// Eight codes starting at code k0 of a row (any k0 that is a multiple of 8) -> one 8-value
// output chunk, w~ = RNE_dtype(fma(s, q, b)) as in dequant32.  The codes occupy 8*BITS bits
// from bit k0*BITS of the row's word stream; the second word is read only when they reach
// into it (so nothing past the row's last code is touched).
template <class T, int BITS>
__device__ inline u32x4 dequant8(const uint32_t* row, int64_t k0, float s, float b) {
  const int64_t bit0 = k0 * BITS;
  const uint32_t* p = row + (bit0 >> 5);
  const int sh = (int)(bit0 & 31);
  const uint32_t lo = p[0];
  const uint32_t hi = sh + 8 * BITS > 32 ? p[1] : 0u;
  const uint64_t v = ((((uint64_t)hi) << 32) | lo) >> sh;
  float q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = (float)((uint32_t)(v >> (e * BITS)) & ((1u << BITS) - 1u));
  u32x4 out;
  out.x = T::pack2(__builtin_fmaf(s, q[0], b), __builtin_fmaf(s, q[1], b));
  out.y = T::pack2(__builtin_fmaf(s, q[2], b), __builtin_fmaf(s, q[3], b));
  out.z = T::pack2(__builtin_fmaf(s, q[4], b), __builtin_fmaf(s, q[5], b));
  out.w = T::pack2(__builtin_fmaf(s, q[6], b), __builtin_fmaf(s, q[7], b));
  return out;
}

}  // namespace qmm
