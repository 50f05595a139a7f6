// Decode with a fused per-row argmax whose workspace is a library-owned device array, for
// callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  The kernels are those of qmm_qmv_argmax; only
// the workspace's origin differs.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <string>

#include "../../include/qmm.h"
#include "capi_internal.hpp"
#include "kernels.hpp"

namespace {

// Per-row argmax keys followed by the workgroup completion counter: 8 * (rows + 1) bytes for
// at most QMM_NOALLOC_MAX_ROWS rows.  Each GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` is only a handle for hipGetSymbolAddress; the
// kernels receive the device address obtained from it.
constexpr int kScratchWords = 64;
static_assert(kScratchWords >= QMM_NOALLOC_MAX_ROWS + 1, "scratch holds the keys and the counter");
static __device__ __align__(256) unsigned long long scratch[kScratchWords];

std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch`, looked up once per device (with that
// device current, which it is: the calling thread's current device).
hipError_t scratch_address(unsigned long long** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  static std::map<int, unsigned long long*> addr;
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    it = addr.emplace(dev, (unsigned long long*)p).first;
  }
  *out = it->second;
  return hipSuccess;
}

// Zero the first `words` words of the scratch copy at `p` (a kernel rather than a memset, so
// the call can be captured into a graph).
__global__ void clear_words(unsigned long long* p, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) p[i] = 0ull;
}

}  // namespace

extern "C" int32_t qmm_qmv_argmax_noalloc(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w,
                                          void* y, const qmm_tensor_desc_t* y_desc, int32_t* out_index,
                                          float* out_value, void* stream) {
  qmm::MatArgs a;
  int64_t rows = 0;
  const int32_t rc = qmm::prepare_qmv_argmax(x, x_desc, w, y, y_desc, out_index, out_value, &a, &rows);
  if (rc != QMM_OK || rows == 0) return rc;
  if (rows > QMM_NOALLOC_MAX_ROWS)
    return qmm::report(QMM_ERR_SHAPE, "qmv_argmax_noalloc: " + std::to_string(rows) + " activation rows exceed the " +
                                          std::to_string(QMM_NOALLOC_MAX_ROWS) + " its scratch holds");
  unsigned long long* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return qmm::report_launch(e);
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(clear_words, dim3(1), dim3(64), 0, s, ws, (int)rows + 1);
  e = hipGetLastError();
  if (e != hipSuccess) return qmm::report_launch(e);
  a.argmax_keys = ws;
  a.argmax_count = (unsigned int*)(ws + rows);
  return qmm::report_launch(qmm::launch_decode(a, s));
}
