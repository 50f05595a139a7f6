// Decode-family kernels for 4-bit codes.
#include "decode_kernels.hpp"

namespace qmm {
namespace decode {

hipError_t launch_decode_b4(const MatArgs& a, hipStream_t stream) { return launch_bits<4>(a, stream); }

}  // namespace decode
}  // namespace qmm
