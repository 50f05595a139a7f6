// Decode-family kernels for 2-, 3-, 5- and 6-bit codes (words shared between codes).
#include "decode_kernels.hpp"

namespace qmm {
namespace decode {

hipError_t launch_decode_bn(const MatArgs& a, hipStream_t stream) {
  switch (a.bits) {
    case 2: return launch_bits<2>(a, stream);
    case 3: return launch_bits<3>(a, stream);
    case 5: return launch_bits<5>(a, stream);
    case 6: return launch_bits<6>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace decode
}  // namespace qmm
