// Per-row top-k of stored logits: the k largest values of each row, largest first, equal
// values by lower column (so k = 1 is the fused argmax's first maximal column), NaN above
// every number, +0 above -0.  This is the top-k form of the decode epilogue on lm_head
// logits (transformers issue 47331, "Reproduction": the next-token choice that collapses
// to token 0; keeping per-row candidates instead of whole logit rows is what a sharded
// lm_head exchanges).
//
// A 1024-thread workgroup per row (or per column chunk of a row), over the row's 16-bit
// values mapped to order keys (unsigned, larger key = larger value), read 8 at a time when
// the row is 16-byte aligned:
//   1. histogram of the key's high 11 bits (2048 bins, so that the values of a typical
//      logit row spread over many LDS counters) -> the bin that holds the k-th largest key,
//      found with a block-wide suffix count;
//   2. usual case, at most 4096 keys in that bin and above: all of them are the candidates;
//   3. otherwise, a histogram of the low 5 bits inside that bin gives the k-th largest key
//      itself (t) and the number of keys above it (g < k); the g keys above t are the
//      candidates [0, g) in any order, and the first k - g keys equal to t in column order
//      (a block-wide prefix count over consecutive column runs) are [g, k).
// The candidates, as (key << 32 | ~column) words, are ranked: up to 512 by counting the
// larger words, more by a bitonic sort in LDS; the first k are written out.  With a
// workspace, long rows are cut into column chunks handled by workgroups of their own
// (enough for about one workgroup per compute unit); the row's last workgroup ranks the
// chunks' candidates.  The result does not depend on the order in which threads or
// workgroups run.
#include <climits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace qmm {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRun = 8;   // consecutive columns per thread in the collecting pass
constexpr int kCand = 4096;   // candidates the one-pass collection takes

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

constexpr int kHiShift = 5;
constexpr int kHiBins = 1 << (16 - kHiShift);
constexpr int kLoBins = 1 << kHiShift;

// Calls f(column, key) for every column of the row; each thread takes 8 consecutive
// columns per step (one 16-byte load when the row is 16-byte aligned).
template <bool FP16, class F>
__device__ inline void for_each_key(const uint16_t* row, int64_t n, F&& f) {
  const bool vec = ((uintptr_t)row & 15u) == 0u;
  const int64_t n8 = vec ? (n & ~(int64_t)7) : 0;
  for (int64_t i = (int64_t)threadIdx.x * 8; i < n8; i += (int64_t)kThreads * 8) {
    const u32x4 v = *(const u32x4*)(row + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f(i + 2 * e, order_key<FP16>(w[e] & 0xFFFFu));
      f(i + 2 * e + 1, order_key<FP16>(w[e] >> 16));
    }
  }
  for (int64_t i = n8 + threadIdx.x; i < n; i += kThreads) f(i, order_key<FP16>(row[i]));
}

// Workgroup-shared state of one selection.
struct TopkSmem {
  uint32_t hist[kHiBins];
  uint32_t wave_sums[kWaves];
  uint32_t sel[4];
  uint32_t slot;
  uint32_t last;
  unsigned long long cand[kCand];
};

// Sorts the m words cand[0, m) (m <= kCand) ascending, padded to a power of two mp with
// zero words (below every candidate), and returns mp: cand[mp - 1 - j] is the j-th largest.
__device__ inline uint32_t sort_words(unsigned long long* cand, uint32_t m) {
  const uint32_t tid = threadIdx.x;
  uint32_t mp = 1u;
  while (mp < m) mp <<= 1;
  __syncthreads();
  for (uint32_t j = m + tid; j < mp; j += kThreads) cand[j] = 0ull;
  for (uint32_t size = 2u; size <= mp; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0u; stride >>= 1) {
      __syncthreads();
      for (uint32_t i = tid; i < mp; i += kThreads) {
        const uint32_t j = i ^ stride;
        if (j > i) {
          const unsigned long long x = cand[i], y = cand[j];
          if ((x > y) == ((i & size) == 0u)) {
            cand[i] = y;
            cand[j] = x;
          }
        }
      }
    }
  }
  __syncthreads();
  return mp;
}

// Writes word w as entry j of output row r.
template <bool FP16>
__device__ inline void store_word(unsigned long long w, uint32_t j, uint32_t k, int64_t r, const TopkArgs& a) {
  const uint32_t bits = key_bits((uint32_t)(w >> 32));
  a.out_index[r * k + j] = (int32_t)(0xFFFFFFFFu - (uint32_t)w);
  if (a.out_value) a.out_value[r * k + j] = FP16 ? Fp16::to_f32(bits) : Bf16::to_f32(bits);
}

// Calls f(j, word) for the j-th largest of the m distinct words cand[0, m), j < kk.  Up to
// 512 words each thread ranks one word by counting the larger ones (no barriers); beyond
// that the words are sorted.
constexpr uint32_t kRankMax = 512;
template <class F>
__device__ inline void emit_largest(unsigned long long* cand, uint32_t m, uint32_t kk, F&& f) {
  if (m <= kRankMax) {
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < m; i += kThreads) {
      const unsigned long long w = cand[i];
      uint32_t r = 0u;
      for (uint32_t j = 0; j < m; ++j) r += cand[j] > w ? 1u : 0u;
      if (r < kk) f(r, w);
    }
    return;
  }
  const uint32_t mp = sort_words(cand, m);
  for (uint32_t j = threadIdx.x; j < kk; j += kThreads) f(j, cand[mp - 1u - j]);
}

// Collects candidate (key << 32 | ~column) words of columns [col0, col0 + len) of a row into
// cand and returns their number m >= kk; the kk largest of them are the kk largest of the
// columns.  `row` points at column col0.
template <bool FP16>
__device__ __forceinline__ uint32_t select_words(const uint16_t* row, int64_t col0, int64_t len, uint32_t kk, TopkSmem& sm) {
  const int tid = threadIdx.x;
  const uint32_t k = kk;
  auto word = [&](uint32_t o, int64_t i) {
    return ((unsigned long long)o << 32) | (0xFFFFFFFFu - (uint32_t)(col0 + i));
  };

  // 1. histogram of the high bits; the bin of the k-th largest key by a suffix count
  for (int b = tid; b < kHiBins; b += kThreads) sm.hist[b] = 0u;
  __syncthreads();
  for_each_key<FP16>(row, len, [&](int64_t, uint32_t o) { atomicAdd(&sm.hist[o >> kHiShift], 1u); });
  __syncthreads();
  {
    static_assert(kHiBins == 2 * kThreads, "two bins per thread");
    const int b_hi = kHiBins - 1 - 2 * tid, b_lo = b_hi - 1;   // thread 0 holds the top bins
    const uint32_t c_hi = sm.hist[b_hi], c_lo = sm.hist[b_lo];
    uint32_t total;
    const uint32_t above = block_exclusive_scan(c_hi + c_lo, sm.wave_sums, &total);
    if (above < k && above + c_hi >= k) {
      sm.sel[0] = (uint32_t)b_hi;
      sm.sel[1] = above;
      sm.sel[2] = above + c_hi;
    } else if (above + c_hi < k && above + c_hi + c_lo >= k) {
      sm.sel[0] = (uint32_t)b_lo;
      sm.sel[1] = above + c_hi;
      sm.sel[2] = above + c_hi + c_lo;
    }
    if (tid == 0) sm.slot = 0u;
  }
  __syncthreads();
  const uint32_t hi = sm.sel[0];
  const uint32_t n_ge = sm.sel[2];   // keys in bin hi or above
  if (n_ge <= (uint32_t)kCand) {
    // Usual case: every key in bin hi or above is a candidate (collected in any order; the
    // word carries the column), then sort them all.
    for_each_key<FP16>(row, len, [&](int64_t i, uint32_t o) {
      if ((o >> kHiShift) >= hi) sm.cand[atomicAdd(&sm.slot, 1u)] = word(o, i);
    });
    return n_ge;
  }
  // Otherwise (a huge tie block at the threshold) find the exact k-th key first.
  // 2. histogram of the low bits inside bin hi
  if (tid < kLoBins) sm.hist[tid] = 0u;
  __syncthreads();
  for_each_key<FP16>(row, len, [&](int64_t, uint32_t o) {
    if ((o >> kHiShift) == hi) atomicAdd(&sm.hist[o & (kLoBins - 1)], 1u);
  });
  __syncthreads();
  if (tid == 0) {
    uint32_t above = sm.sel[1];
    int l = kLoBins - 1;
    for (; l > 0 && above + sm.hist[l] < k; --l) above += sm.hist[l];
    sm.sel[2] = (hi << kHiShift) | (uint32_t)l;
    sm.sel[3] = above;
  }
  __syncthreads();
  const uint32_t t = sm.sel[2], g = sm.sel[3], need_eq = k - g;

  // 3. collect: keys above t anywhere in [0, g), the first need_eq keys equal to t in
  // column order in [g, k)
  const bool vec = ((uintptr_t)row & 15u) == 0u;
  uint32_t eq_seen = 0u;   // keys equal to t in earlier runs (the same in every thread)
  for (int64_t base = 0; base < len; base += (int64_t)kThreads * kRun) {
    const int64_t i0 = base + (int64_t)tid * kRun;
    uint32_t o[kRun];
    if (vec && i0 + kRun <= len) {
      const u32x4 v = *(const u32x4*)(row + i0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = order_key<FP16>(w[e] & 0xFFFFu);
        o[2 * e + 1] = order_key<FP16>(w[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kRun; ++e) o[e] = i0 + e < len ? order_key<FP16>(row[i0 + e]) : 0u;   // real keys are never 0
    }
    uint32_t neq = 0u;
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      if (o[e] > t) sm.cand[atomicAdd(&sm.slot, 1u)] = word(o[e], i0 + e);
      neq += o[e] == t ? 1u : 0u;
    }
    uint32_t total;
    uint32_t r = eq_seen + block_exclusive_scan(neq, sm.wave_sums, &total);
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      if (o[e] == t) {
        if (r < need_eq) sm.cand[g + r] = word(t, i0 + e);
        ++r;
      }
    }
    eq_seen += total;
  }
  return k;
}

// One workgroup per row.
template <bool FP16>
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(const TopkArgs a) {
  __shared__ TopkSmem sm;
  const int64_t r = blockIdx.x;
  const uint16_t* row = (const uint16_t*)a.logits + r * a.row_stride;
  const uint32_t k = (uint32_t)a.k;
  const uint32_t m = select_words<FP16>(row, 0, a.n, k, sm);
  emit_largest(sm.cand, m, k, [&](uint32_t j, unsigned long long w) { store_word<FP16>(w, j, k, r, a); });
}

// Rows cut into `parts` column chunks of `chunk` columns (a multiple of 8), one workgroup
// per (chunk, row).  Each writes its chunk's k largest words (zero words past a short
// chunk) to the workspace, then counts itself done on the row's counter; the row's last
// workgroup sorts the parts * k words (at most kCand) and writes the row's result, then
// clears the counter.  Ordering: every writer thread's words happen before the workgroup
// barrier, which happens before thread 0's count; the count is an acquire-release
// read-modify-write at device scope whose release half orders the workgroup's words before
// it; the last workgroup's threads issue an acquire fence at device scope before reading the
// words.
template <bool FP16>
__global__ __launch_bounds__(kThreads) void topk_parts_kernel(const TopkArgs a, const int parts, const int64_t chunk) {
  __shared__ TopkSmem sm;
  const int c = blockIdx.x;
  const int64_t r = blockIdx.y;
  const uint32_t k = (uint32_t)a.k;
  const int64_t col0 = (int64_t)c * chunk;
  const int64_t len = a.n - col0 < chunk ? a.n - col0 : chunk;
  const uint32_t kk = (int64_t)k < len ? k : (uint32_t)len;
  const uint16_t* row = (const uint16_t*)a.logits + r * a.row_stride + col0;
  const uint32_t mc = select_words<FP16>(row, col0, len, kk, sm);
  unsigned int* counters = (unsigned int*)a.workspace;
  unsigned long long* words = (unsigned long long*)a.workspace + kTopkWsHeader * a.rows + (r * parts + c) * (int64_t)k;
  emit_largest(sm.cand, mc, kk, [&](uint32_t j, unsigned long long w) {
    __hip_atomic_store(&words[j], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
  for (uint32_t j = kk + threadIdx.x; j < k; j += kThreads)   // a chunk shorter than k
    __hip_atomic_store(&words[j], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned done = __hip_atomic_fetch_add(&counters[2 * r], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = done + 1u == (unsigned)parts ? 1u : 0u;
  }
  __syncthreads();
  if (sm.last == 0u) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const unsigned long long* row_words = (const unsigned long long*)a.workspace + kTopkWsHeader * a.rows + r * parts * (int64_t)k;
  const uint32_t m = (uint32_t)parts * k;
  for (uint32_t j = threadIdx.x; j < m; j += kThreads)
    sm.cand[j] = __hip_atomic_load(&row_words[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  emit_largest(sm.cand, m, k, [&](uint32_t j, unsigned long long w) { store_word<FP16>(w, j, k, r, a); });
  if (threadIdx.x == 0) __hip_atomic_store(&counters[2 * r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// Columns per part: enough parts for about one workgroup per compute unit over all rows,
// parts of at least 4096 columns, and parts * k within what one workgroup sorts.
int64_t topk_chunk(int64_t n, int k, int64_t rows, int* parts) {
  int64_t p = (256 + rows - 1) / rows;
  const int64_t p_cols = (n + 4095) / 4096;
  if (p > p_cols) p = p_cols;
  const int64_t p_max = kCand / k;
  if (p > p_max) p = p_max;
  if (p < 1) p = 1;
  int64_t chunk = (n + p - 1) / p;
  chunk = (chunk + 7) / 8 * 8;   // 16-byte aligned chunk starts
  *parts = (int)((n + chunk - 1) / chunk);
  return chunk;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.k < 1 || a.k > kTopkMax || a.k > a.n || a.rows > INT_MAX) return hipErrorInvalidValue;
  int parts = 1;
  const int64_t chunk = topk_chunk(a.n, a.k, a.rows, &parts);
  if (a.workspace && parts > 1 && a.rows <= 65535) {
    const dim3 grid((unsigned)parts, (unsigned)a.rows);
    if (a.dtype == 2)
      hipLaunchKernelGGL((topk_parts_kernel<true>), grid, dim3(kThreads), 0, stream, a, parts, chunk);
    else
      hipLaunchKernelGGL((topk_parts_kernel<false>), grid, dim3(kThreads), 0, stream, a, parts, chunk);
    return hipGetLastError();
  }
  if (a.dtype == 2)
    hipLaunchKernelGGL((topk_rows_kernel<true>), dim3((unsigned)a.rows), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((topk_rows_kernel<false>), dim3((unsigned)a.rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qmm
