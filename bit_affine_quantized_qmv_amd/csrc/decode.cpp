// Decode-family entry: route by code width to the per-width kernel files.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace qmm {
namespace decode {

hipError_t launch_decode_b4(const MatArgs& a, hipStream_t stream);
hipError_t launch_decode_b8(const MatArgs& a, hipStream_t stream);
hipError_t launch_decode_bn(const MatArgs& a, hipStream_t stream);

// Compute units of the current device (cached per device id).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
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
