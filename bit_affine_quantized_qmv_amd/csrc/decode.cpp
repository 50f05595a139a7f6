// Decode-family entry: route by code width to the per-width kernel files.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <set>
#include <tuple>
#include <utility>

#include "kernels.hpp"

namespace qmm {
namespace decode {

hipError_t launch_decode_b4(const MatArgs& a, hipStream_t stream);
hipError_t launch_decode_b8(const MatArgs& a, hipStream_t stream);
hipError_t launch_decode_bn(const MatArgs& a, hipStream_t stream);

namespace {
std::mutex g_launch_mu;   // guards the launch-setting caches below
}

// Compute units of the current device (cached per device id).
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::lock_guard<std::mutex> lock(g_launch_mu);
  static std::map<int, int> cached;
  auto it = cached.find(dev);
  if (it != cached.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cached[dev] = n;
  return n;
}

// Workgroups of `threads` threads per CU for kernel `kern` at `lds` bytes of dynamic LDS.
// The kernel's dynamic-LDS limit is raised to `lds_max` once per device; occupancies are
// cached per (device, kernel, LDS size).
hipError_t kernel_wgs_per_cu(const void* kern, int threads, int lds, int lds_max, int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::lock_guard<std::mutex> lock(g_launch_mu);
  static std::set<std::pair<int, const void*>> raised;
  static std::map<std::tuple<int, const void*, int>, int> occ;
  if (!raised.count({dev, kern})) {
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_max);
    if (e != hipSuccess) return e;
    raised.insert({dev, kern});
  }
  const auto key = std::make_tuple(dev, kern, lds);
  auto it = occ.find(key);
  if (it == occ.end()) {
    int nb = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, lds);
    if (e != hipSuccess) return e;
    it = occ.emplace(key, nb > 0 ? nb : 1).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace decode

hipError_t launch_decode(const MatArgs& a, hipStream_t stream) {
  if (a.rows_per_batch > 32 || a.rows_per_batch <= 0 || a.batches > 65535) return hipErrorInvalidValue;
  // rows start on 16-byte boundaries; K is a multiple of the group size (>= 32)
  if (a.K % 32 != 0 || a.w_row_stride % 4 != 0) return hipErrorInvalidValue;
  if (a.bits == 4) return decode::launch_decode_b4(a, stream);
  if (a.bits == 8) return decode::launch_decode_b8(a, stream);
  return decode::launch_decode_bn(a, stream);
}

}  // namespace qmm
