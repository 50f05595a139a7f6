// Prefill family: y = x . dequant(W)^T for more than 32 activation rows (qmm_t).
//
// A dense bf16/fp16 GEMM on the matrix cores (16x16x32 MFMA, float32 accumulators, one
// fixed K order, no split-K).  Each K tile of the packed weight is unpacked and
// dequantized, w~ = s*q + b rounded to the storage dtype, into LDS next to the activation
// tile; the products then see ordinary half-precision operands.  The epilogue stores each
// output row through the plan's row addressing, which also serves strided batches such as
// a view narrowed on the sequence dimension (transformers issue 47331, layout table: every
// row of every batch element must be computed).
#include "dequant_impl.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace qmm {
namespace {

constexpr int BM = 256;           // output rows per workgroup
constexpr int BN = 256;           // output columns (weight rows) per workgroup
constexpr int BK = 64;            // k per main-loop step
constexpr int WM = 4, WN = 2;     // waves along M and N; each wave owns a (BM/WM) x (BN/WN) tile
constexpr int kThreads = 64 * WM * WN;

template <class T, int BITS>
__global__ __launch_bounds__(kThreads, 1) void qmm_prefill_kernel(const MatArgs a, const int m_tiles) {
  // operand layout in LDS: [buffer][k step (32)][lane group (8 k)][row] of 8 elements
  __shared__ u32x4 As[2][BK / 32][4][BM];
  __shared__ u32x4 Bs[2][BK / 32][4][BN];
  constexpr int TM = BM / WM, TN = BN / WN;      // wave tile
  constexpr int FM = TM / 16, FN = TN / 16;      // 16x16 MFMA blocks per wave tile
  constexpr int A_PER = BM * (BK / 8) / kThreads;   // 16-byte activation chunks per thread
  static_assert(BN * 2 == kThreads, "one thread per 32 codes of a weight row");
  static_assert(A_PER <= FM && FM == 4, "activation and weight chunks are stored one per MFMA row");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lg = lane >> 4;
  const int col = lane & 15;
  const int wm = wave / WN;
  const int wn = wave % WN;
  // M-tile fastest: consecutive workgroups (which the dispatcher spreads over the XCDs)
  // share a weight tile, and each XCD keeps seeing the same activation rows
  const int mt = (int)(blockIdx.x % (unsigned)m_tiles);
  const int nt = (int)(blockIdx.x / (unsigned)m_tiles);
  const int64_t z = blockIdx.z;
  const int64_t rows = a.rows_per_batch;
  const int64_t N = a.N;
  const int K = (int)a.K;
  const int gs = a.group_size;
  const int64_t bm0 = (int64_t)mt * BM;
  const int64_t bn0 = (int64_t)nt * BN;
  const uint16_t* xb = (const uint16_t*)a.x + z * a.batch_stride;

  // activation chunks: q -> row (q % 16) + 16 * (q / 128), chunk (q / 16) % 8, so a wave
  // reads 64 contiguous bytes of 16 rows and writes four 256-byte runs of LDS
  // rows past the call's rows read row 0 (always valid) and are zeroed after the load
  const uint16_t* arow[A_PER];
  int ar[A_PER], ac[A_PER];
  uint32_t amask[A_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int q = tid + kThreads * i;
    ar[i] = (q & 15) + 16 * (q >> 7);
    ac[i] = (q >> 4) & 7;
    const int64_t m = bm0 + ar[i];
    const int64_t mr = m < rows ? m : 0;
    amask[i] = m < rows ? 0xFFFFFFFFu : 0u;
    arow[i] = xb + (mr / a.seg_rows) * a.seg_stride + (mr % a.seg_rows) * a.row_stride;
  }
  // weight: thread -> row wr, 32-code half wh of the 64 k of a step
  const int wr = tid >> 1, wh = tid & 1;
  const int64_t wn_row = bn0 + wr < N ? bn0 + wr : N - 1;
  const uint32_t* wrow = a.w + wn_row * a.w_row_stride;
  const uint16_t* srow = (const uint16_t*)a.scales + wn_row * a.sb_row_stride;
  const uint16_t* brow = (const uint16_t*)a.biases + wn_row * a.sb_row_stride;

  u32x4 ra[A_PER];
  uint32_t rw[BITS];
  uint32_t rs = 0, rb = 0;
  // When K is not a multiple of BK the last step is partial: activation chunks and code
  // runs at k >= K read the row's first chunk / run instead and are zeroed (K is a multiple
  // of 32, so a chunk or run is either wholly inside or wholly outside the row).
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int k = k0 + 8 * ac[i];
      const bool kv = k < K;
      ra[i] = *(const u32x4*)(arow[i] + (kv ? k : 0)) & (kv ? amask[i] : 0u);
    }
    const int kw = k0 + 32 * wh;
    const bool wv_ok = kw < K;
    load_codes<BITS>(rw, wrow + (wv_ok ? kw / 32 * BITS : 0));
    const int g = wv_ok ? kw / gs : 0;
    rs = wv_ok ? srow[g] : 0u;
    rb = wv_ok ? brow[g] : 0u;
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) As[buf][ac[i] >> 2][ac[i] & 3][ar[i]] = ra[i];
    u32x4 wv[4];
    dequant32<T, BITS>(rw, T::to_f32(rs), T::to_f32(rb), wv);
#pragma unroll
    for (int c = 0; c < 4; ++c) Bs[buf][wh][c][wr] = wv[c];
  };

  f32x4 acc[FM][FN];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = zero4;

  // Software pipeline over k steps: while the MFMAs of step kt read LDS buffer kt & 1, the
  // registers holding step kt+1's global data are dequantized and written to the other
  // buffer, interleaved with the first half of the MFMAs; the loads of step kt+2 are then
  // issued into the freed registers.  One barrier per step.  The body has no branches: the
  // last step reloads a clamped step and writes it into the buffer no one reads any more.
  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  gload(nk > 1 ? 1 : 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    typename T::v8 av[FM], bv[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) av[i] = as_v8<T>(As[buf][0][lg][wm * TM + 16 * i + col]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bv[j] = as_v8<T>(Bs[buf][0][lg][wn * TN + 16 * j + col]);
    u32x4 wv[4];
    dequant32<T, BITS>(rw, T::to_f32(rs), T::to_f32(rb), wv);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = T::mfma(av[i], bv[j], acc[i][j]);
      // one activation chunk and one weight chunk per MFMA row
      if (i < A_PER) As[buf ^ 1][ac[i] >> 2][ac[i] & 3][ar[i]] = ra[i];
      Bs[buf ^ 1][wh][i][wr] = wv[i];
    }
    // spread the dequantization and the LDS writes between the MFMAs of the first half
#pragma unroll
    for (int t = 0; t < FM * FN; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // three VALU
      if (t % 4 == 3) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // one LDS write
    }
    gload(kt + 2 < nk ? kt + 2 : nk - 1);
#pragma unroll
    for (int i = 0; i < FM; ++i) av[i] = as_v8<T>(As[buf][1][lg][wm * TM + 16 * i + col]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bv[j] = as_v8<T>(Bs[buf][1][lg][wn * TN + 16 * j + col]);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = T::mfma(av[i], bv[j], acc[i][j]);
    __syncthreads();
  }

  uint16_t* yb = (uint16_t*)a.y + z * rows * N;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = bm0 + wm * TM + 16 * i + 4 * lg + r;
        const int64_t n = bn0 + wn * TN + 16 * j + col;
        if (m < rows && n < N) yb[m * N + n] = T::from_f32(acc[i][j][r]);
      }
}

template <class T, int BITS>
hipError_t launch_bits(const MatArgs& a, hipStream_t stream) {
  const int64_t m_tiles = (a.rows_per_batch + BM - 1) / BM;
  const int64_t n_tiles = (a.N + BN - 1) / BN;
  if (m_tiles * n_tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((qmm_prefill_kernel<T, BITS>), dim3((unsigned)(m_tiles * n_tiles), 1, (unsigned)a.batches),
                     dim3(kThreads), 0, stream, a, (int)m_tiles);
  return hipGetLastError();
}

template <class T>
hipError_t launch_dtype(const MatArgs& a, hipStream_t stream) {
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

hipError_t launch_prefill(const MatArgs& a, hipStream_t stream) {
  if (a.rows_per_batch <= 0 || a.batches > 65535 || a.K % 32 != 0) return hipErrorInvalidValue;
  return a.dtype == 1 ? launch_dtype<Bf16>(a, stream) : launch_dtype<Fp16>(a, stream);
}

}  // namespace qmm
