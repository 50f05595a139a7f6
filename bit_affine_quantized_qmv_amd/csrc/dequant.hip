// Standalone dequantization and quantized embedding row gather (bandwidth-bound).
//
// Output row r is dequant(W[src(r), :]) rounded to the storage dtype, src(r) = r for the
// whole-matrix form (transformers issue 47331, "Root cause": the probe dequantizes the
// packed weight back to a dense tensor) and src(r) = index[r] for the row gather of a
// quantized embedding table (Metal Kernel Bits=8 final report, section 3.2: dequantizing
// single rows).  A gather index outside [0, N) gives a NaN row.  One thread handles one
// 8-code chunk (16 output bytes), consecutive threads consecutive chunks of a row, so each
// wave's store covers 1 KB of contiguous output.
#include <algorithm>
#include <climits>

#include "dequant_impl.hpp"
#include "kernels.hpp"

namespace qmm {
namespace {

constexpr int kThreads = 256;

template <class T, int BITS, class I>
__device__ inline void dequant_chunks(const DequantArgs& a, I total, I chunks_per_row) {
  const int gs_shift = __builtin_ctz((unsigned)a.group_size);   // group sizes are powers of two
  for (I c = (I)blockIdx.x * kThreads + threadIdx.x; c < total; c += (I)gridDim.x * kThreads) {
    const I r = c / chunks_per_row;
    const I kc = c - r * chunks_per_row;
    int64_t src = a.index ? (int64_t)a.index[r] : (int64_t)r;
    const bool bad = src < 0 || src >= a.N;
    src = bad ? 0 : src;
    const int64_t k0 = 8 * (int64_t)kc;
    const int64_t g = k0 >> gs_shift;
    const float s = T::to_f32(((const uint16_t*)a.scales)[src * a.sb_row_stride + g]);
    const float b = T::to_f32(((const uint16_t*)a.biases)[src * a.sb_row_stride + g]);
    u32x4 v = dequant8<T, BITS>(a.w + src * a.w_row_stride, k0, s, b);
    if (bad) {
      const uint32_t nan2 = T::kDtype == 1 ? 0x7FC07FC0u : 0x7E007E00u;
      v = u32x4{nan2, nan2, nan2, nan2};
    }
    *(u32x4*)((uint16_t*)a.out + (int64_t)r * a.out_row_stride + k0) = v;
  }
}

template <class T, int BITS>
__global__ __launch_bounds__(kThreads) void dequant_rows_kernel(const DequantArgs a) {
  const int64_t cpr = a.K / 8;
  const int64_t total = a.rows * cpr;
  // 32-bit index arithmetic whenever the chunk count fits
  if (total <= (int64_t)UINT_MAX - (int64_t)gridDim.x * kThreads)
    dequant_chunks<T, BITS, uint32_t>(a, (uint32_t)total, (uint32_t)cpr);
  else
    dequant_chunks<T, BITS, uint64_t>(a, (uint64_t)total, (uint64_t)cpr);
}

template <class T, int BITS>
hipError_t launch_bits(const DequantArgs& a, hipStream_t stream) {
  const int64_t total = a.rows * (a.K / 8);
  const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 256 * 32);
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
