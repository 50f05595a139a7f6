// Set-up and read-out of the fused per-row argmax keys (see argmax_key in decode_impl.hpp).
// A fill kernel rather than a memset, so the sequence can also be recorded in a HIP graph.
#include <algorithm>

#include "kernels.hpp"

namespace qmm {
namespace {

__global__ void argmax_init_kernel(unsigned long long* keys, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) keys[i] = 0ull;
}

__global__ void argmax_finish_kernel(const unsigned long long* keys, int64_t count, int32_t* index, float* value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const unsigned long long k = keys[i];
  const uint32_t ord = (uint32_t)(k >> 32);
  const uint32_t bits = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  index[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
  if (value) value[i] = __uint_as_float(bits);
}

}  // namespace

hipError_t launch_argmax_init(unsigned long long* keys, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_init_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, keys, count);
  return hipGetLastError();
}

hipError_t launch_argmax_finish(const unsigned long long* keys, int64_t count, int32_t* index, float* value,
                                hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_finish_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, keys, count,
                     index, value);
  return hipGetLastError();
}

}  // namespace qmm
