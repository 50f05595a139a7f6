// Per-row top-k of stored logits: the k largest values of each row, largest first, equal
// values by lower column (so k = 1 is the fused argmax's first maximal column), NaN above
// every number, +0 above -0.  This is the top-k form of the decode epilogue on lm_head
// logits (transformers issue 47331, "Reproduction": the next-token choice that collapses
// to token 0; keeping per-row candidates instead of whole logit rows is what a sharded
// lm_head exchanges).
//
// One 1024-thread workgroup per row, three passes over the row's 16-bit values mapped to
// order keys (unsigned, larger key = larger value):
//   1. histogram of the key's high byte -> the bin that holds the k-th largest key;
//   2. histogram of the low byte inside that bin -> the k-th largest key itself (t) and
//      the number of keys above it (g < k);
//   3. the g keys above t go to candidate slots [0, g) in any order; the first k - g keys
//      equal to t in column order (a block-wide prefix count over consecutive column runs)
//      go to slots [g, k).
// The k candidates, as (key << 32 | ~column) words, are sorted in LDS (bitonic) and
// written out.  The result does not depend on the order in which threads run.
#include <climits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace qmm {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRun = 8;   // consecutive columns per thread in the collecting pass

template <bool FP16>
__device__ inline uint32_t order_key(uint32_t b) {
  const bool nan = FP16 ? ((b & 0x7C00u) == 0x7C00u && (b & 0x03FFu) != 0u)
                        : ((b & 0x7F80u) == 0x7F80u && (b & 0x007Fu) != 0u);
  if (nan) b = FP16 ? 0x7E00u : 0x7FC0u;   // every NaN counts as the largest value
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ inline uint32_t key_bits(uint32_t o) { return (o & 0x8000u) ? (o & 0x7FFFu) : (~o & 0xFFFFu); }

// Exclusive prefix sum of v over the workgroup in thread order; *total gets the sum.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_sums, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t s = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(s, d);
    if (lane >= d) s += t;
  }
  if (lane == 63) wave_sums[wave] = s;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t ws = wave_sums[w];
    before += w < wave ? ws : 0u;
    all += ws;
  }
  __syncthreads();   // wave_sums is reused by the next call
  *total = all;
  return before + s - v;
}

template <bool FP16>
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(const TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_sums[kWaves];
  __shared__ uint32_t sel[4];
  __shared__ uint32_t n_above_slot;
  __shared__ unsigned long long cand[kTopkMax];
  const int tid = threadIdx.x;
  const uint16_t* row = (const uint16_t*)a.logits + (int64_t)blockIdx.x * a.row_stride;
  const int64_t n = a.n;
  const uint32_t k = (uint32_t)a.k;

  // 1. high-byte histogram
  if (tid < 256) hist[tid] = 0u;
  __syncthreads();
  for (int64_t i = tid; i < n; i += kThreads) atomicAdd(&hist[order_key<FP16>(row[i]) >> 8], 1u);
  __syncthreads();
  if (tid == 0) {
    uint32_t above = 0u;
    int b = 255;
    for (; b > 0 && above + hist[b] < k; --b) above += hist[b];
    sel[0] = (uint32_t)b;
    sel[1] = above;
  }
  __syncthreads();
  const uint32_t hi = sel[0];
  // 2. low-byte histogram inside bin hi
  if (tid < 256) hist[tid] = 0u;
  __syncthreads();
  for (int64_t i = tid; i < n; i += kThreads) {
    const uint32_t o = order_key<FP16>(row[i]);
    if ((o >> 8) == hi) atomicAdd(&hist[o & 255u], 1u);
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t above = sel[1];
    int l = 255;
    for (; l > 0 && above + hist[l] < k; --l) above += hist[l];
    sel[2] = (hi << 8) | (uint32_t)l;
    sel[3] = above;
    n_above_slot = 0u;
  }
  __syncthreads();
  const uint32_t t = sel[2], g = sel[3], need_eq = k - g;

  // 3. collect
  uint32_t eq_seen = 0u;   // keys equal to t in earlier runs (the same in every thread)
  for (int64_t base = 0; base < n; base += (int64_t)kThreads * kRun) {
    const int64_t i0 = base + (int64_t)tid * kRun;
    uint32_t o[kRun];
    uint32_t neq = 0u;
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      const int64_t i = i0 + e;
      o[e] = i < n ? order_key<FP16>(row[i]) : 0u;   // keys of real values are never 0
      if (o[e] > t) cand[atomicAdd(&n_above_slot, 1u)] = ((unsigned long long)o[e] << 32) | (0xFFFFFFFFu - (uint32_t)i);
      neq += o[e] == t ? 1u : 0u;
    }
    uint32_t total;
    uint32_t r = eq_seen + block_exclusive_scan(neq, wave_sums, &total);
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      if (o[e] == t) {
        if (r < need_eq) cand[g + r] = ((unsigned long long)t << 32) | (0xFFFFFFFFu - (uint32_t)(i0 + e));
        ++r;
      }
    }
    eq_seen += total;
  }
  // pad to a power of two with words below every candidate, then sort ascending
  uint32_t kp = 1u;
  while (kp < k) kp <<= 1;
  for (uint32_t j = k + tid; j < kp; j += kThreads) cand[j] = 0ull;
  for (uint32_t size = 2u; size <= kp; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0u; stride >>= 1) {
      __syncthreads();
      const uint32_t i = (uint32_t)tid, j = i ^ stride;
      if (i < kp && j > i) {
        const unsigned long long x = cand[i], y = cand[j];
        if ((x > y) == ((i & size) == 0u)) {
          cand[i] = y;
          cand[j] = x;
        }
      }
    }
  }
  __syncthreads();
  for (uint32_t j = tid; j < k; j += kThreads) {
    const unsigned long long c = cand[kp - 1u - j];
    const uint32_t bits = key_bits((uint32_t)(c >> 32));
    a.out_index[(int64_t)blockIdx.x * k + j] = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
    if (a.out_value) a.out_value[(int64_t)blockIdx.x * k + j] = FP16 ? Fp16::to_f32(bits) : Bf16::to_f32(bits);
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.k < 1 || a.k > kTopkMax || a.k > a.n || a.rows > INT_MAX) return hipErrorInvalidValue;
  if (a.dtype == 2)
    hipLaunchKernelGGL((topk_rows_kernel<true>), dim3((unsigned)a.rows), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((topk_rows_kernel<false>), dim3((unsigned)a.rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qmm
