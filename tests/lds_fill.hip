// Test helper (not part of the library): fills the LDS of every compute unit with a 32-bit
// pattern, and copies out LDS that a dispatch finds at its start without having written it.
// With these a test shows that a library kernel's results do not depend on what an earlier
// dispatch left in LDS: every LDS word a kernel reads must have been written by that kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kLdsBytes = 160 * 1024;   // all of a gfx950 compute unit's LDS
constexpr int kWords = kLdsBytes / 4;

// One workgroup takes the whole LDS of its compute unit and writes the pattern to every word
// (volatile stores: the compiler may not drop them although nothing reads them back).
__global__ __launch_bounds__(kThreads) void fill_kernel(uint32_t pattern) {
  extern __shared__ uint32_t lds[];
  volatile uint32_t* p = lds;
  for (int i = threadIdx.x; i < kWords; i += kThreads) p[i] = pattern;
}

// Workgroup b copies the first `words` LDS words it finds at its start to out[b * words, ...).
__global__ __launch_bounds__(kThreads) void peek_kernel(uint32_t* out, int words) {
  extern __shared__ uint32_t lds[];
  volatile uint32_t* p = lds;
  for (int i = threadIdx.x; i < words; i += kThreads) out[(int64_t)blockIdx.x * words + i] = p[i];
}

}  // namespace

// Fills the LDS with `pattern` in `blocks` workgroups of the whole LDS each (a few times the
// number of compute units reaches every one of them).  Returns a hipError_t code.
extern "C" int lds_fill(uint32_t pattern, int blocks, void* stream) {
  if (blocks < 1) return (int)hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)fill_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(kThreads), kLdsBytes, (hipStream_t)stream, pattern);
  return (int)hipGetLastError();
}

// Copies the first `words` (at most 40960) LDS words each of `blocks` workgroups finds at its
// start into out, which holds blocks * words 32-bit words.  Returns a hipError_t code.
extern "C" int lds_peek(uint32_t* out, int blocks, int words, void* stream) {
  if (blocks < 1 || words < 1 || words > kWords) return (int)hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)peek_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(peek_kernel, dim3((unsigned)blocks), dim3(kThreads), kLdsBytes, (hipStream_t)stream, out, words);
  return (int)hipGetLastError();
}
