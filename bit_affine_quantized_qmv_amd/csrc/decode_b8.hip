// Decode-family kernels for 8-bit codes.
#include "decode_kernels.hpp"

namespace qmm {
namespace decode {

hipError_t launch_decode_b8(const MatArgs& a, hipStream_t stream) { return launch_bits<8>(a, stream); }

}  // namespace decode
}  // namespace qmm
