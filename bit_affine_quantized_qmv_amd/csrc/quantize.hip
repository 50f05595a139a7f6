// Min/max affine group quantizer (transformers issue 47331, "Root cause": the probe
// quantizes W per group, then casts scales and biases to bf16).
//
// One wave per segment of 256 consecutive elements of a row, 4 per lane, read with one
// 16-byte load per lane when the rows are 16-byte aligned.  A group's minimum and maximum
// come from a butterfly over its gs / 4 lanes (minimum and maximum are exact, so the order
// does not matter).  The float32 operations are written one at a time with contraction
// disabled and IEEE division, so the codes and parameters are a deterministic function of W:
//   s = (max - min) / (2^bits - 1),  b = min,
//   q = clamp(rint((w - b) / s), 0, 2^bits - 1), q = 0 when s == 0,
// then s and b are rounded to nearest-even in the storage dtype.  Codes go into the row's
// little-endian bitstream (Metal Kernel Bits=8 final report, section 3.1, for 4 and 8 bits):
// lane l's four codes are bits [4 * bits * l, 4 * bits * (l + 1)) of the segment, which
// starts on a word boundary (256 * bits is a multiple of 32); the lanes OR their bits into
// the segment's words in LDS, then store them whole.
#include "device_common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace qmm {
namespace {

constexpr int kSegment = 256;             // elements per wave
constexpr int kQuantThreads = 256;        // four waves, four segments per workgroup

template <class T, int BITS>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(const QuantArgs a, const int64_t segs_per_row,
                                                                 const bool vec) {
  __shared__ uint32_t words[kQuantThreads / 64][8 * BITS];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t seg = (int64_t)blockIdx.x * (kQuantThreads / 64) + wave;
  if (seg >= a.N * segs_per_row) return;   // whole waves leave; no barrier follows
  const int64_t n = seg / segs_per_row;
  const int64_t e0 = (seg - n * segs_per_row) * kSegment;
  const int64_t e = e0 + 4 * lane;
  const bool live = e < a.K;               // K is a multiple of the group size (>= 32)
  const float* wr = a.w + n * a.w_row_stride;
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (live) {
    if (vec) {
      const float4 f = *(const float4*)(wr + e);
      v[0] = f.x;
      v[1] = f.y;
      v[2] = f.z;
      v[3] = f.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = wr[e + i];
    }
  }
  // group minimum and maximum over the group's gs / 4 lanes (aligned runs of lanes)
  float lo = fminf(fminf(v[0], v[1]), fminf(v[2], v[3]));
  float hi = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
  const int lanes = a.group_size >> 2;
  for (int d = 1; d < lanes; d <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, d));
    hi = fmaxf(hi, __shfl_xor(hi, d));
  }
  const float qmax = (float)((1 << BITS) - 1);
  const float range = hi - lo;
  const float s = range / qmax;
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t q = 0;
    if (s != 0.0f) {
      const float d = v[i] - lo;
      const float t = d / s;
      const float r = fminf(fmaxf(__builtin_rintf(t), 0.0f), qmax);
      q = (uint32_t)r;
    }
    bits |= q << (BITS * i);
  }
  // the segment's words: zero them, OR in each lane's 4 * BITS bits, store the live ones
  uint32_t* wl = words[wave];
  for (int j = lane; j < 8 * BITS; j += 64) wl[j] = 0u;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  if (live) {
    const int bit0 = 4 * BITS * lane;
    const int w0 = bit0 >> 5, sh = bit0 & 31;
    atomicOr(&wl[w0], bits << sh);
    if (sh + 4 * BITS > 32) atomicOr(&wl[w0 + 1], bits >> (32 - sh));
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const int64_t live_elems = a.K - e0 < kSegment ? a.K - e0 : kSegment;
  const int n_words = (int)((live_elems * BITS) >> 5);
  uint32_t* out = a.w_packed + n * ((a.K * BITS) >> 5) + ((e0 * BITS) >> 5);
  for (int j = lane; j < n_words; j += 64) out[j] = wl[j];
  if (live && (lane & (lanes - 1)) == 0) {
    const int64_t n_groups = a.K / a.group_size;
    const int64_t g = e / a.group_size;
    ((uint16_t*)a.scales)[n * n_groups + g] = T::from_f32(s);
    ((uint16_t*)a.biases)[n * n_groups + g] = T::from_f32(lo);
  }
}

template <class T, int BITS>
hipError_t launch_bits(const QuantArgs& a, hipStream_t stream) {
  const int64_t segs_per_row = (a.K + kSegment - 1) / kSegment;
  const int64_t per_block = kQuantThreads / 64;
  const int64_t blocks = (a.N * segs_per_row + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool vec = ((uintptr_t)a.w & 15u) == 0u && a.w_row_stride % 4 == 0;
  hipLaunchKernelGGL((quantize_kernel<T, BITS>), dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, a,
                     segs_per_row, vec);
  return hipGetLastError();
}

template <class T>
hipError_t launch_dtype(const QuantArgs& a, hipStream_t stream) {
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

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  return a.dtype == 1 ? launch_dtype<Bf16>(a, stream) : launch_dtype<Fp16>(a, stream);
}

}  // namespace qmm
