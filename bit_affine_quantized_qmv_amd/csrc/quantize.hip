// Min/max affine group quantizer (transformers issue 47331, "Root cause": the probe
// quantizes W per group, then casts scales and biases to bf16).
//
// One thread per (row, group).  The float32 operations are written one at a time with
// contraction disabled and IEEE division, so the codes and parameters are a deterministic
// function of W:
//   s = (max - min) / (2^bits - 1),  b = min,
//   q = clamp(rint((w - b) / s), 0, 2^bits - 1), q = 0 when s == 0,
// then s and b are rounded to nearest-even in the storage dtype.  Codes go into the row's
// little-endian bitstream (Metal Kernel Bits=8 final report, section 3.1, for 4 and 8 bits);
// a group of gs codes is gs*bits/32 whole words, so threads never share a word.
#include "device_common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace qmm {
namespace {

template <class T, int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const QuantArgs a) {
  const int64_t n_groups = a.K / a.group_size;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.N * n_groups) return;
  const int64_t n = gid / n_groups;
  const int64_t gi = gid - n * n_groups;
  const int gs = a.group_size;
  const float* wr = a.w + n * a.w_row_stride + gi * gs;

  float lo = wr[0];
  float hi = lo;
  for (int i = 1; i < gs; ++i) {
    const float v = wr[i];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  const float qmax = (float)((1 << BITS) - 1);
  const float range = hi - lo;
  const float s = range / qmax;

  uint32_t* out = a.w_packed + n * ((a.K * BITS) >> 5) + ((gi * gs * BITS) >> 5);
  uint64_t pending = 0;
  int nbits = 0;
  int wo = 0;
  for (int i = 0; i < gs; ++i) {
    uint32_t q = 0;
    if (s != 0.0f) {
      const float d = wr[i] - lo;
      const float t = d / s;
      const float r = fminf(fmaxf(__builtin_rintf(t), 0.0f), qmax);
      q = (uint32_t)r;
    }
    pending |= (uint64_t)q << nbits;
    nbits += BITS;
    if (nbits >= 32) {
      out[wo++] = (uint32_t)pending;
      pending >>= 32;
      nbits -= 32;
    }
  }
  ((uint16_t*)a.scales)[n * n_groups + gi] = T::from_f32(s);
  ((uint16_t*)a.biases)[n * n_groups + gi] = T::from_f32(lo);
}

template <class T, int BITS>
hipError_t launch_bits(const QuantArgs& a, hipStream_t stream) {
  const int64_t total = a.N * (a.K / a.group_size);
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quantize_kernel<T, BITS>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <class T>
hipError_t launch_dtype(const QuantArgs& a, hipStream_t stream) {
  switch (a.bits) {
    case 2: return launch_bits<T, 2>(a, stream);
    case 3: return launch_bits<T, 3>(a, stream);
    case 4: return launch_bits<T, 4>(a, stream);
    case 5: return launch_bits<T, 5>(a, stream);
    case 6: return launch_bits<T, 6>(a, stream);
    case 8: return launch_bits<T, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  return a.dtype == 1 ? launch_dtype<Bf16>(a, stream) : launch_dtype<Fp16>(a, stream);
}

}  // namespace qmm
