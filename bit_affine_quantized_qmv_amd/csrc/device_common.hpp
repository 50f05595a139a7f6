// Device-side types and conversions shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element-type traits.  Both formats go through the same 16x16x32 MFMA shape, so a row's
// arithmetic never depends on how many rows share the call.
struct Bf16 {
  using v8 = bf16x8;
  using v2 = bf16x2;
  static constexpr int kDtype = 1;
  __device__ static inline f32x4 mfma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline float to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
  }
  // float -> bf16, round to nearest even (finite inputs).
  __device__ static inline uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    v2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  // Two small non-negative integers (< 256, exact in 8 significand bits) as a bf16 pair:
  // the upper halves of their float32 patterns, joined with one byte permute.
  __device__ static inline uint32_t pack2_int(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  // Two fp8 (e4m3) bytes of `w` -> two values, times 2^9.  e4m3 byte patterns 0..15 encode
  // exactly c * 2^-9 (subnormals and the first normal binade share that spacing), so a
  // 4-bit code placed in a byte comes back as the exact integer code.
  __device__ static inline uint32_t fp8x2_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, false));
  }
  __device__ static inline uint32_t fp8x2_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, true));
  }
};

struct Fp16 {
  using v8 = f16x8;
  using v2 = f16x2;
  static constexpr int kDtype = 2;
  __device__ static inline f32x4 mfma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline float to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  }
  __device__ static inline uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    v2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  // Two small non-negative integers (< 2048, exact in binary16) as an fp16 pair; the
  // truncating pack is exact here.
  __device__ static inline uint32_t pack2_int(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  __device__ static inline uint32_t fp8x2_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 512.0f, false));
  }
  __device__ static inline uint32_t fp8x2_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 512.0f, true));
  }
};

// Workgroup barrier that orders LDS only: it waits for this wave's LDS operations, not for
// its outstanding global/buffer loads (a plain __syncthreads() also drains those, which
// would stall weight prefetches issued before the barrier).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <class T>
__device__ inline typename T::v8 as_v8(u32x4 u) {
  return __builtin_bit_cast(typename T::v8, u);
}

// Eight 4-bit codes of one word -> eight exact values in the element order
// [q0, q2, q4, q6, q1, q3, q5, q7]; the activation side is stored in the same order.
template <class T>
__device__ inline u32x4 codes4_to_v8(uint32_t w) {
  const uint32_t even = w & 0x0F0F0F0Fu;         // q0, q2, q4, q6 in bytes 0..3
  const uint32_t odd = (w >> 4) & 0x0F0F0F0Fu;   // q1, q3, q5, q7
  u32x4 r;
  r.x = T::fp8x2_lo(even);
  r.y = T::fp8x2_hi(even);
  r.z = T::fp8x2_lo(odd);
  r.w = T::fp8x2_hi(odd);
  return r;
}

// Eight 8-bit codes (two words, natural order) -> eight exact values.
template <class T>
__device__ inline u32x4 codes8_to_v8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r.x = T::pack2_int((float)(w0 & 0xFFu), (float)((w0 >> 8) & 0xFFu));
  r.y = T::pack2_int((float)((w0 >> 16) & 0xFFu), (float)(w0 >> 24));
  r.z = T::pack2_int((float)(w1 & 0xFFu), (float)((w1 >> 8) & 0xFFu));
  r.w = T::pack2_int((float)((w1 >> 16) & 0xFFu), (float)(w1 >> 24));
  return r;
}

// Eight consecutive BITS-bit codes starting at bit `shift` of the 64-bit window hi:lo
// -> eight exact values, natural order.
template <class T, int BITS>
__device__ inline u32x4 codesN_to_v8(uint32_t lo, uint32_t hi, uint32_t shift) {
  const uint64_t v = ((((uint64_t)hi) << 32) | lo) >> shift;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)((uint32_t)(v >> (i * BITS)) & mask);
  u32x4 r;
  r.x = T::pack2_int(f[0], f[1]);
  r.y = T::pack2_int(f[2], f[3]);
  r.z = T::pack2_int(f[4], f[5]);
  r.w = T::pack2_int(f[6], f[7]);
  return r;
}

// [x0..x7] (four words of 16-bit pairs) -> [x0, x2, x4, x6, x1, x3, x5, x7]
__device__ inline u32x4 interleave_even_odd(u32x4 u) {
  u32x4 r;
  r.x = (u.x & 0xFFFFu) | (u.y << 16);
  r.y = (u.z & 0xFFFFu) | (u.w << 16);
  r.z = (u.x >> 16) | (u.y & 0xFFFF0000u);
  r.w = (u.z >> 16) | (u.w & 0xFFFF0000u);
  return r;
}

}  // namespace qmm
