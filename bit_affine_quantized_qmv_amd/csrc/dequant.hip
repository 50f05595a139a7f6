// Standalone dequantization and quantized embedding row gather (bandwidth-bound).
//
// Output row r is dequant(W[src(r), :]) rounded to the storage dtype, src(r) = r for the
// whole-matrix form (transformers issue 47331, "Root cause": the probe dequantizes the
// packed weight back to a dense tensor) and src(r) = index[r] for the row gather of a
// quantized embedding table (Metal Kernel Bits=8 final report, section 3.2: dequantizing
// single rows).  A gather index outside [0, N) gives a NaN row.  One thread handles one
// 32-code run: it loads BITS code words, the run's scale and bias, and stores 64 bytes.
#include <algorithm>

#include "dequant_impl.hpp"
#include "kernels.hpp"

namespace qmm {
namespace {

constexpr int kThreads = 256;

template <class T, int BITS>
__global__ __launch_bounds__(kThreads) void dequant_rows_kernel(const DequantArgs a) {
  const uint32_t units_per_row = (uint32_t)(a.K / 32);
  const int64_t total = a.rows * (int64_t)units_per_row;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += (int64_t)gridDim.x * kThreads) {
    const int64_t r = u / units_per_row;
    const int j = (int)(u - r * units_per_row);
    int64_t src = a.index ? (int64_t)a.index[r] : r;
    const bool bad = src < 0 || src >= a.N;
    src = bad ? 0 : src;
    uint32_t w[BITS];
    load_codes<BITS>(w, a.w + src * a.w_row_stride + (int64_t)j * BITS);
    const int g = (32 * j) / a.group_size;
    const uint16_t* sp = (const uint16_t*)a.scales + src * a.sb_row_stride + g;
    const uint16_t* bp = (const uint16_t*)a.biases + src * a.sb_row_stride + g;
    u32x4 v[4];
    dequant32<T, BITS>(w, T::to_f32(*sp), T::to_f32(*bp), v);
    if (bad) {
      const uint32_t nan2 = T::kDtype == 1 ? 0x7FC07FC0u : 0x7E007E00u;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = u32x4{nan2, nan2, nan2, nan2};
    }
    u32x4* dst = (u32x4*)((uint16_t*)a.out + r * a.out_row_stride + 32 * j);
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = v[c];
  }
}

template <class T, int BITS>
hipError_t launch_bits(const DequantArgs& a, hipStream_t stream) {
  const int64_t total = a.rows * (a.K / 32);
  const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 256 * 16);
  hipLaunchKernelGGL((dequant_rows_kernel<T, BITS>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <class T>
hipError_t launch_dtype(const DequantArgs& a, hipStream_t stream) {
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

hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  return a.dtype == 1 ? launch_dtype<Bf16>(a, stream) : launch_dtype<Fp16>(a, stream);
}

}  // namespace qmm
