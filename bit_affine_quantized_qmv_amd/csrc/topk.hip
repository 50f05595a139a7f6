// Per-row top-k of stored logits: the k largest values of each row, largest first, equal
// values by lower column (so k = 1 is the fused argmax's first maximal column), NaN above
// every number, +0 above -0.  This is the top-k form of the decode epilogue on lm_head
// logits (transformers issue 47331, "Reproduction": the next-token choice that collapses
// to token 0; keeping per-row candidates instead of whole logit rows is what a sharded
// lm_head exchanges).
//
// Each workgroup selects from one span of columns (a whole row, or one column chunk of it),
// over the 16-bit values mapped to order keys (unsigned, larger key = larger value):
//   0. spans of up to 8 * threads * 4 columns are loaded once into registers (8 consecutive
//      columns per run, one 16-byte load when the row is 16-byte aligned, two keys per
//      register, converted two at a time; runs past the span's end are skipped by whole
//      waves); longer spans are read from global memory on each pass;
//   1. with the keys in registers, a threshold t from the threads' largest keys: each wave
//      holding columns finds the c = ceil(k / such waves) largest of its threads' maxima
//      (repeated wave maxima), and t is the k-th largest of all those values (a ballot
//      radix select in one wave) or, when they do not fit one wave, the least of the waves'
//      c-th values: at least k keys reach t either way.  The keys >= t are the candidates when there are at least k of
//      them and they fit the candidate buffer (4096 words, the usual case); a wave collects
//      them register by register, with one ballot test per register and one slot
//      reservation per register that holds any;
//   2. otherwise, a histogram of every key's high 11 bits (2048 bins, so that the values of
//      a typical logit row spread over many LDS counters) -> the bin that holds the k-th
//      largest key, found with a block-wide suffix count; at most 4096 keys in that bin and
//      above: all of them are the candidates;
//   3. otherwise, a histogram of the low 5 bits inside that bin gives the k-th largest key
//      itself (t) and the number of keys above it (g < k); the g keys above t are the
//      candidates [0, g) in any order, and the first k - g keys equal to t in column order
//      (a block-wide prefix count over consecutive column runs) are [g, k).
// The candidates, as (key << 32 | ~column) words, are ranked: while there are at most as
// many as threads by counting the larger words, beyond that by a bitonic sort in LDS; the
// first k are the span's result.  With a workspace, long rows are cut into column chunks
// (about one workgroup per compute unit in all): a select kernel writes each chunk's k
// best words to the workspace, largest first, and a merge kernel, one workgroup per row,
// merges the row's lists pairwise, level by level.  The kernel boundary orders the two, so
// no workgroup waits for another.
// The result does not depend on the order in which threads or workgroups run.
#include <climits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace qmm {
namespace {

constexpr int kRowThreads = 1024;     // one workgroup per whole row
constexpr int kSelThreads = 1024;     // one workgroup per column chunk of a row
constexpr int kMergeThreads = 1024;   // one workgroup per row, merging its chunks' words
constexpr int kRun = 8;               // consecutive columns per thread and step
constexpr int kSelRuns = 4;           // 8-column runs per thread held in registers: chunks
constexpr int kRowRuns = 4;           // ... and whole rows (up to 32768 columns)
constexpr int kCand = 4096;           // candidates the one-pass collection takes
constexpr int kTargetWorkgroups = 256;   // chunk workgroups over all rows: about one per CU
constexpr int64_t kMinChunk = 2048;      // columns per chunk, at least

// Columns a workgroup of THREADS threads holds in registers at RUNS runs per thread.
template <int THREADS, int RUNS>
constexpr int64_t reg_cols() { return (int64_t)THREADS * kRun * RUNS; }

template <bool FP16>
__device__ inline uint32_t order_key(uint32_t b) {
  const bool nan = FP16 ? ((b & 0x7C00u) == 0x7C00u && (b & 0x03FFu) != 0u)
                        : ((b & 0x7F80u) == 0x7F80u && (b & 0x007Fu) != 0u);
  if (nan) b = FP16 ? 0x7E00u : 0x7FC0u;   // every NaN counts as the largest value
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ inline uint32_t key_bits(uint32_t o) { return (o & 0x8000u) ? (o & 0x7FFFu) : (~o & 0xFFFFu); }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// Order keys of the two 16-bit values of w (low and high half) at once: the sign bit of each
// half selects the mask (0xFFFF for negative values, 0x8000 for positive ones).  Exact for
// every value but NaN, which the caller detects with has_nan2 and handles with order_key.
__device__ inline uint32_t order_keys2(uint32_t w) {
  const i16x2 s = __builtin_bit_cast(i16x2, w) >> (short)15;
  return w ^ (__builtin_bit_cast(uint32_t, s) | 0x80008000u);
}

template <bool FP16>
__device__ inline bool has_nan2(uint32_t w) {
  constexpr uint32_t kInf2 = FP16 ? 0x7C007C00u : 0x7F807F80u;   // magnitudes above this are NaN
  const u16x2 m = __builtin_elementwise_max(__builtin_bit_cast(u16x2, w & 0x7FFF7FFFu), __builtin_bit_cast(u16x2, kInf2));
  return __builtin_bit_cast(uint32_t, m) != kInf2;
}

// Largest v over the wave (in every lane): row-local DPP steps, then the row broadcasts.
__device__ inline uint32_t wave_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));   // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The k-th largest of the wave's nonzero 16-bit values u (one per lane), 0 when fewer than k
// lanes hold one: a radix select from the top bit, counting lanes with ballots (the same
// result in every lane).
__device__ inline uint32_t wave_kth_largest(uint32_t u, uint32_t k) {
  uint64_t cand = __builtin_amdgcn_ballot_w64(u != 0u);
  if ((uint32_t)__builtin_popcountll(cand) < k) return 0u;
  uint32_t prefix = 0u, need = k;
  for (int bit = 15; bit >= 0; --bit) {
    const uint64_t ones = __builtin_amdgcn_ballot_w64(((u >> bit) & 1u) != 0u) & cand;
    const uint32_t n = (uint32_t)__builtin_popcountll(ones);
    if (n >= need) {
      cand = ones;
      prefix |= 1u << bit;
    } else {
      need -= n;
      cand &= ~ones;
    }
  }
  return prefix;
}

// Exclusive prefix sum of v over the workgroup in thread order; *total gets the sum.
template <int THREADS>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_sums, uint32_t* total) {
  constexpr int kWaves = THREADS / 64;
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

// The order keys of columns [i0, i0 + 8) of a span of len columns (0 past its end; real keys
// are never 0): one 16-byte load when the span is 16-byte aligned and the run is whole.
template <bool FP16>
__device__ inline void load_run(const uint16_t* row, int64_t i0, int64_t len, bool vec, uint32_t (&o)[kRun]) {
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
    for (int e = 0; e < kRun; ++e) o[e] = i0 + e < len ? order_key<FP16>(row[i0 + e]) : 0u;
  }
}

// Keys of a span read from global memory on every pass.  Step j of thread t covers columns
// 8 * (t + THREADS * j) .. + 7.
template <bool FP16, int THREADS>
struct GlobalKeys {
  static constexpr bool kHeldKeys = false;   // no cheap per-thread maximum (a pass of its own)
  const uint16_t* row;
  int64_t len;
  __device__ uint32_t max_key() const { return 0u; }
  // f(column in span, key) for every column
  template <class F>
  __device__ void each(F&& f) const {
    const bool vec = ((uintptr_t)row & 15u) == 0u;
    for (int64_t i0 = (int64_t)threadIdx.x * kRun; i0 < len; i0 += (int64_t)THREADS * kRun) {
      uint32_t o[kRun];
      load_run<FP16>(row, i0, len, vec, o);
#pragma unroll
      for (int e = 0; e < kRun; ++e)
        if (o[e]) f(i0 + e, o[e]);
    }
  }
  // f(first column, keys of the run) for every step, the same number of calls in every thread
  template <class F>
  __device__ void steps(F&& f) const {
    const bool vec = ((uintptr_t)row & 15u) == 0u;
    for (int64_t base = 0; base < len; base += (int64_t)THREADS * kRun) {
      const int64_t i0 = base + (int64_t)threadIdx.x * kRun;
      uint32_t o[kRun];
      load_run<FP16>(row, i0, len, vec, o);
      f(i0, o);
    }
  }
};

// Keys of a span of at most reg_cols<THREADS, RUNS>() columns, loaded once into registers
// with the same column assignment (run j of thread t: columns 8 * (t + THREADS * j) .. + 7),
// two 16-bit keys per register (column 2e in the low half, 2e + 1 in the high half).  Runs
// that hold no column of any thread of the wave are skipped by the whole wave.
template <bool FP16, int THREADS, int RUNS>
struct RegKeys {
  static constexpr bool kHeldKeys = true;
  uint32_t p[RUNS][4];
  int runs;   // runs holding a column of this wave's threads (the same in the whole wave)
  __device__ __forceinline__ static uint32_t pack(uint32_t w) {
    return order_key<FP16>(w & 0xFFFFu) | (order_key<FP16>(w >> 16) << 16);
  }
  __device__ __forceinline__ void load(const uint16_t* row, int64_t len) {
    const bool vec = ((uintptr_t)row & 15u) == 0u;
    const int64_t wave_first = (int64_t)(__builtin_amdgcn_readfirstlane((int)threadIdx.x) & ~63);
    runs = 0;
#pragma unroll
    for (int j = 0; j < RUNS; ++j)
      if ((int64_t)kRun * (wave_first + THREADS * j) < len) runs = j + 1;
    bool whole[RUNS];
    // every whole run's load is issued before any key is formed
#pragma unroll
    for (int j = 0; j < RUNS; ++j) {
      const int64_t i0 = (int64_t)kRun * (threadIdx.x + THREADS * j);
      whole[j] = j < runs && vec && i0 + kRun <= len;
      if (whole[j]) {
        const u32x4 v = *(const u32x4*)(row + i0);
        p[j][0] = v.x;
        p[j][1] = v.y;
        p[j][2] = v.z;
        p[j][3] = v.w;
      }
    }
    bool nan = false;
#pragma unroll
    for (int j = 0; j < RUNS; ++j) {
      const int64_t i0 = (int64_t)kRun * (threadIdx.x + THREADS * j);
      if (j >= runs) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[j][e] = 0u;
      } else if (whole[j]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nan = nan || has_nan2<FP16>(p[j][e]);
          p[j][e] = order_keys2(p[j][e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t c = i0 + 2 * e;
          const uint32_t lo = c < len ? order_key<FP16>(row[c]) : 0u;
          const uint32_t hi = c + 1 < len ? order_key<FP16>(row[c + 1]) : 0u;
          p[j][e] = lo | (hi << 16);
        }
      }
    }
    if (nan) {   // a NaN among the thread's whole runs: their keys again, NaN by NaN
#pragma unroll
      for (int j = 0; j < RUNS; ++j) {
        if (whole[j]) {
          const u32x4 v = *(const u32x4*)(row + (int64_t)kRun * (threadIdx.x + THREADS * j));
          p[j][0] = pack(v.x);
          p[j][1] = pack(v.y);
          p[j][2] = pack(v.z);
          p[j][3] = pack(v.w);
        }
      }
    }
  }
  // the thread's largest key (0 when it holds none)
  __device__ __forceinline__ uint32_t max_key() const {
    u16x2 m = {0, 0};
#pragma unroll
    for (int j = 0; j < RUNS; ++j)
      if (j < runs)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, p[j][e]));
    return max((uint32_t)m.x, (uint32_t)m.y);
  }
  // Writes the word of every key >= t (t > 0) to cand[*slot ...] (words past kCand are
  // counted, not written), *slot counting them.  A register is looked at by the whole wave
  // only when some lane's register holds such a key; then the wave reserves its slots with
  // one atomic and places its lanes' keys by their rank in the ballots.
  __device__ __forceinline__ void collect_ge(uint32_t t, int64_t col0, uint32_t* slot,
                                             unsigned long long* cand) const {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t tt = (t - 1u) * 0x10001u;   // both halves t - 1: max(key, t - 1) > t - 1 iff key >= t
#pragma unroll
    for (int j = 0; j < RUNS; ++j)
      if (j < runs)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = p[j][e];
          const u16x2 mx = __builtin_elementwise_max(__builtin_bit_cast(u16x2, w), __builtin_bit_cast(u16x2, tt));
          if (__builtin_amdgcn_ballot_w64(__builtin_bit_cast(uint32_t, mx) != tt) != 0ull) {
            const uint32_t lo = w & 0xFFFFu, hi = w >> 16;
            const uint64_t mlo = __builtin_amdgcn_ballot_w64(lo >= t);
            const uint64_t mhi = __builtin_amdgcn_ballot_w64(hi >= t);
            const uint32_t nlo = (uint32_t)__builtin_popcountll(mlo);
            uint32_t base = 0u;
            if (lane == 0u) base = atomicAdd(slot, nlo + (uint32_t)__builtin_popcountll(mhi));
            base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
            const int64_t c = (int64_t)kRun * (threadIdx.x + THREADS * j) + 2 * e;
            const uint32_t below = (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(mlo >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mlo, 0u));
            const uint32_t below_hi = (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(mhi >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mhi, 0u));
            const uint32_t plo = base + below, phi = base + nlo + below_hi;
            if (lo >= t && plo < (uint32_t)kCand)
              cand[plo] = ((unsigned long long)lo << 32) | (0xFFFFFFFFu - (uint32_t)(col0 + c));
            if (hi >= t && phi < (uint32_t)kCand)
              cand[phi] = ((unsigned long long)hi << 32) | (0xFFFFFFFFu - (uint32_t)(col0 + c + 1));
          }
        }
  }
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
#pragma unroll
    for (int j = 0; j < RUNS; ++j)
      if (j < runs)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t o = (p[j][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          if (o) f((int64_t)kRun * (threadIdx.x + THREADS * j) + e, o);
        }
  }
};

// Workgroup-shared state of one selection.
struct TopkSmem {
  uint32_t hist[kHiBins];
  uint32_t wave_sums[16];
  uint32_t top[64];
  uint32_t sel[4];
  uint32_t slot;
  unsigned long long cand[kCand];
};

// Sorts the m words cand[0, m) (m <= kCand) ascending, padded to a power of two mp with
// zero words (below every candidate), and returns mp: cand[mp - 1 - j] is the j-th largest.
template <int THREADS>
__device__ inline uint32_t sort_words(unsigned long long* cand, uint32_t m) {
  const uint32_t tid = threadIdx.x;
  uint32_t mp = 1u;
  while (mp < m) mp <<= 1;
  __syncthreads();
  for (uint32_t j = m + tid; j < mp; j += THREADS) cand[j] = 0ull;
  for (uint32_t size = 2u; size <= mp; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0u; stride >>= 1) {
      __syncthreads();
      for (uint32_t i = tid; i < mp; i += THREADS) {
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
// THREADS words each thread ranks one word by counting the larger ones (no barriers);
// beyond that the words are sorted.
template <int THREADS, class F>
__device__ inline void emit_largest(unsigned long long* cand, uint32_t m, uint32_t kk, F&& f) {
  if (m <= (uint32_t)THREADS) {
    __syncthreads();
    const uint32_t i = threadIdx.x;
    if (i < m) {
      const unsigned long long w = cand[i];
      uint32_t r = 0u, j = 0u;
      for (; j + 8u <= m; j += 8u) {   // eight words read at once, then compared
        unsigned long long c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = cand[j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) r += c[u] > w ? 1u : 0u;
      }
      for (; j < m; ++j) r += cand[j] > w ? 1u : 0u;
      if (r < kk) f(r, w);
    }
    return;
  }
  const uint32_t mp = sort_words<THREADS>(cand, m);
  for (uint32_t j = threadIdx.x; j < kk; j += THREADS) f(j, cand[mp - 1u - j]);
}

// From the per-bin counts in sm.hist, the bin where the count from the top reaches k:
// sm.sel[0] = that bin, sm.sel[1] = count in the bins above it, sm.sel[2] = count in it and
// above; sm.sel[2] stays below k when the counts total less than k.  Also zeroes sm.slot.
template <int THREADS>
__device__ inline void find_bin(uint32_t k, TopkSmem& sm) {
  const int tid = threadIdx.x;
  constexpr int kPer = kHiBins / THREADS;   // bins per thread, thread 0 holding the top ones
  static_assert(kPer * THREADS == kHiBins, "whole bins per thread");
  if (tid == 0) {
    sm.sel[2] = 0u;
    sm.slot = 0u;
  }
  uint32_t c[kPer], sum = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    c[j] = sm.hist[kHiBins - 1 - kPer * tid - j];
    sum += c[j];
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan<THREADS>(sum, sm.wave_sums, &total);   // barriers inside
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (run < k && run + c[j] >= k) {
      sm.sel[0] = (uint32_t)(kHiBins - 1 - kPer * tid - j);
      sm.sel[1] = run;
      sm.sel[2] = run + c[j];
    }
    run += c[j];
  }
  __syncthreads();
}

// Collects candidate (key << 32 | ~column) words of the span [col0, col0 + len) of a row,
// whose keys come from ks (the exact-threshold pass, rare, reads them from gk in column
// order), into cand and returns their number m >= kk; the kk largest of them are the kk
// largest of the span.
template <bool FP16, int THREADS, class KS>
__device__ __forceinline__ uint32_t select_words(const KS& ks, const GlobalKeys<FP16, THREADS>& gk, int64_t col0,
                                                 uint32_t kk, TopkSmem& sm) {
  const int tid = threadIdx.x;
  const uint32_t k = kk;
  auto word = [&](uint32_t o, int64_t i) {
    return ((unsigned long long)o << 32) | (0xFFFFFFFFu - (uint32_t)(col0 + i));
  };

  if constexpr (KS::kHeldKeys) {
    // 0. A threshold from the threads' largest keys: each wave holding columns finds the c
    // largest of its threads' maxima (c = ceil(k / such waves)).  When these values fit one wave,
    // the threshold t is the k-th largest of them (maxima of distinct threads, so at least k
    // keys reach it), else t = the least of the waves' c-th largest values (each wave has c
    // keys reaching its own).  The keys >= t are the candidates when there are at least k of
    // them and they fit the candidate buffer (the usual case; the count is checked, so the
    // threshold needs no other guarantee), else the histogram passes below decide.  Each
    // thread counts its candidates, reserves that many slots with one atomic, and writes
    // them there.
    constexpr uint32_t kWaves = THREADS / 64;
    const int lane = tid & 63, wave = tid >> 6;
    // computed over the first nw waves (those holding columns: the first run of wave w starts
    // at column 64 * kRun * w); the copy for all waves has the count folded in
    auto threshold = [&](const uint32_t nw) -> uint32_t {
      const uint32_t c = (k + nw - 1) / nw;   // at most 64 threads per wave: c > 64 gives no threshold
      const bool pooled = nw * c <= 64u;
      uint32_t tw = 0u;
      if ((uint32_t)wave < nw && c <= 64u) {
        uint32_t v = (ks.max_key() << 6) | (uint32_t)lane;   // distinct per lane
        for (uint32_t i = 0; i < c; ++i) {
          const uint32_t top = wave_max(v);
          tw = top >> 6;
          if (pooled && lane == 0) sm.top[wave * c + i] = tw;
          if (v == top) v = 0u;   // that thread's maximum is taken
        }
      }
      if (lane == 0) sm.wave_sums[wave] = tw;
      if (tid == 0) sm.slot = 0u;
      __syncthreads();
      if (c > 64u) return 0u;
      if (pooled) return wave_kth_largest((uint32_t)lane < nw * c ? sm.top[lane] : 0u, k);
      uint32_t least = 0xFFFFFFFFu;
      for (uint32_t w = 0; w < nw; ++w) least = min(least, sm.wave_sums[w]);
      return least;
    };
    // With waves that hold no columns, the copy for all waves still works when its pooled
    // values from the waves that do hold columns number at least k (the others add zeros).
    const uint32_t nw = gk.len >= (int64_t)THREADS * kRun ? kWaves : (uint32_t)((gk.len + 64 * kRun - 1) / (64 * kRun));
    const uint32_t c_all = (k + kWaves - 1) / kWaves;
    const bool all_works = nw == kWaves || (kWaves * c_all <= 64u && nw * c_all >= k);
    const uint32_t t = all_works ? threshold(kWaves) : threshold(nw);
    if (t > 0u) {
      ks.collect_ge(t, col0, &sm.slot, sm.cand);
      __syncthreads();
      const uint32_t m = sm.slot;
      if (m >= k && m <= (uint32_t)kCand) return m;
      __syncthreads();   // every thread has read sm.slot before the histogram pass resets it
    }
  }

  // 1. histogram of the high bits; the bin of the k-th largest key by a suffix count
  for (int b = tid; b < kHiBins; b += THREADS) sm.hist[b] = 0u;
  __syncthreads();
  ks.each([&](int64_t, uint32_t o) { atomicAdd(&sm.hist[o >> kHiShift], 1u); });
  __syncthreads();
  find_bin<THREADS>(k, sm);
  const uint32_t hi = sm.sel[0];
  const uint32_t n_ge = sm.sel[2];   // keys in bin hi or above
  if (n_ge <= (uint32_t)kCand) {
    // Usual case: every key in bin hi or above is a candidate (collected in any order; the
    // word carries the column).
    ks.each([&](int64_t i, uint32_t o) {
      if ((o >> kHiShift) >= hi) sm.cand[atomicAdd(&sm.slot, 1u)] = word(o, i);
    });
    return n_ge;
  }
  // Otherwise (a huge tie block at the threshold) find the exact k-th key first.
  // 2. histogram of the low bits inside bin hi
  if (tid < kLoBins) sm.hist[tid] = 0u;
  __syncthreads();
  ks.each([&](int64_t, uint32_t o) {
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
  // column order in [g, k) (steps cover consecutive column ranges, threads in column order)
  uint32_t eq_seen = 0u;   // keys equal to t in earlier steps (the same in every thread)
  gk.steps([&](int64_t i0, const uint32_t (&o)[kRun]) {
    uint32_t neq = 0u;
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      if (o[e] > t) sm.cand[atomicAdd(&sm.slot, 1u)] = word(o[e], i0 + e);
      neq += o[e] == t ? 1u : 0u;
    }
    uint32_t total;
    uint32_t r = eq_seen + block_exclusive_scan<THREADS>(neq, sm.wave_sums, &total);
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      if (o[e] == t) {
        if (r < need_eq) sm.cand[g + r] = word(t, i0 + e);
        ++r;
      }
    }
    eq_seen += total;
  });
  return k;
}

// Candidates of the span [col0, col0 + len) of a row (starting at `row`): from registers when
// the span fits RUNS runs per thread, else from global memory on each pass.
template <bool FP16, int THREADS, int RUNS>
__device__ __forceinline__ uint32_t select_span(const uint16_t* row, int64_t col0, int64_t len, uint32_t kk,
                                                TopkSmem& sm) {
  const GlobalKeys<FP16, THREADS> gk{row, len};
  if (len <= reg_cols<THREADS, RUNS>()) {
    RegKeys<FP16, THREADS, RUNS> ks;
    ks.load(row, len);
    return select_words<FP16, THREADS>(ks, gk, col0, kk, sm);
  }
  return select_words<FP16, THREADS>(gk, gk, col0, kk, sm);
}

// One workgroup per row.
template <bool FP16>
__global__ __launch_bounds__(kRowThreads) void topk_rows_kernel(const TopkArgs a) {
  __shared__ TopkSmem sm;
  const int64_t r = blockIdx.x;
  const uint16_t* row = (const uint16_t*)a.logits + r * a.row_stride;
  const uint32_t k = (uint32_t)a.k;
  const uint32_t m = select_span<FP16, kRowThreads, kRowRuns>(row, 0, a.n, k, sm);
  emit_largest<kRowThreads>(sm.cand, m, k, [&](uint32_t j, unsigned long long w) { store_word<FP16>(w, j, k, r, a); });
}

// Rows cut into `parts` column chunks of `chunk` columns (a multiple of 8), one workgroup per
// (chunk, row): each writes its chunk's k largest words to the workspace, largest first
// (zero words after them when the chunk is shorter than k).
template <bool FP16>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const TopkArgs a, const int parts,
                                                                  const int64_t chunk) {
  __shared__ TopkSmem sm;
  const int c = blockIdx.x;
  const int64_t r = blockIdx.y;
  const uint32_t k = (uint32_t)a.k;
  const int64_t col0 = (int64_t)c * chunk;
  const int64_t len = a.n - col0 < chunk ? a.n - col0 : chunk;
  const uint32_t kk = (int64_t)k < len ? k : (uint32_t)len;
  const uint16_t* row = (const uint16_t*)a.logits + r * a.row_stride + col0;
  unsigned long long* words = (unsigned long long*)a.workspace + r * kTopkWsRowWords + (int64_t)c * k;
  const uint32_t m = select_span<FP16, kSelThreads, kSelRuns>(row, col0, len, kk, sm);
  emit_largest<kSelThreads>(sm.cand, m, kk, [&](uint32_t j, unsigned long long w) { words[j] = w; });
  for (uint32_t j = kk + threadIdx.x; j < k; j += kSelThreads) words[j] = 0ull;
}

// One workgroup per row: the row's parts lists of k words, each sorted largest first, are
// merged pairwise, level by level, keeping the k largest of each pair (an odd list passes to
// the next level as it is).  In a pair, a word's place is its index in its own list plus the
// number of larger words in the other list (a binary search); the words are distinct (they
// carry the column), so the places of the k largest are distinct.  Zero words (padding of
// short chunks) are below every candidate: they only fill the places after the real words,
// and the last level stores none of them.
template <bool FP16>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(const TopkArgs a, const int parts) {
  __shared__ unsigned long long buf[2][kMergeThreads];
  const int64_t r = blockIdx.x;
  const uint32_t k = (uint32_t)a.k;
  const uint32_t tid = threadIdx.x;
  uint32_t nl = (uint32_t)parts;   // lists at this level, nl * k <= kMergeThreads
  const unsigned long long* src = (const unsigned long long*)a.workspace + r * kTopkWsRowWords;
  if (tid < nl * k) buf[0][tid] = src[tid];
  int cur = 0;
  for (;;) {
    __syncthreads();
    const uint32_t pairs = nl >> 1, odd = nl & 1u;
    const bool last = nl == 2u;
    const unsigned long long* s = buf[cur];
    unsigned long long* d = buf[cur ^ 1];
    if (tid < nl * k) {
      const uint32_t list = tid / k, i = tid - list * k;
      const unsigned long long x = s[tid];
      if (odd && list == nl - 1u) {
        d[pairs * k + i] = x;
      } else {
        const unsigned long long* o = s + (list ^ 1u) * k;
        uint32_t lo = 0u, hi = k;   // first entry of the other list not larger than x
        while (lo < hi) {
          const uint32_t mid = (lo + hi) >> 1;
          if (o[mid] > x)
            lo = mid + 1u;
          else
            hi = mid;
        }
        const uint32_t pos = i + lo;
        if (pos < k) {
          if (!last)
            d[(list >> 1) * k + pos] = x;
          else if (x != 0ull)
            store_word<FP16>(x, pos, k, r, a);
        }
      }
    }
    if (last) break;
    nl = pairs + odd;
    cur ^= 1;
  }
}

}  // namespace

// Columns per chunk: about kTargetWorkgroups chunk workgroups over all rows, chunks of at
// least kMinChunk columns, and parts * k within what the merge workgroup ranks.
int64_t topk_chunk(int64_t n, int k, int64_t rows, int* parts) {
  int64_t p = (kTargetWorkgroups + rows - 1) / rows;
  const int64_t p_cols = (n + kMinChunk - 1) / kMinChunk;
  if (p > p_cols) p = p_cols;
  const int64_t p_max = kMergeThreads / k;
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
      hipLaunchKernelGGL((topk_select_kernel<true>), grid, dim3(kSelThreads), 0, stream, a, parts, chunk);
    else
      hipLaunchKernelGGL((topk_select_kernel<false>), grid, dim3(kSelThreads), 0, stream, a, parts, chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dtype == 2)
      hipLaunchKernelGGL((topk_merge_kernel<true>), dim3((unsigned)a.rows), dim3(kMergeThreads), 0, stream, a, parts);
    else
      hipLaunchKernelGGL((topk_merge_kernel<false>), dim3((unsigned)a.rows), dim3(kMergeThreads), 0, stream, a, parts);
    return hipGetLastError();
  }
  if (a.dtype == 2)
    hipLaunchKernelGGL((topk_rows_kernel<true>), dim3((unsigned)a.rows), dim3(kRowThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((topk_rows_kernel<false>), dim3((unsigned)a.rows), dim3(kRowThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qmm
