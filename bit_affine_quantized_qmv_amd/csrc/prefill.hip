// Prefill family: y = x . dequant(W)^T for more than 32 activation rows (qmm_t).
//
// A dense bf16/fp16 GEMM on the matrix cores (16x16x32 MFMA, float32 accumulators, one
// fixed K order, no split-K).  Each K tile of the packed weight is unpacked and
// dequantized, w~ = s*q + b rounded to the storage dtype, into LDS next to the activation
// tile; the products then see ordinary half-precision operands.  The epilogue stores each
// output row through the plan's row addressing, which also serves strided batches such as
// a view narrowed on the sequence dimension (transformers issue 47331, layout table: every
// row of every batch element must be computed).
#include "device_common.hpp"
#include "kernels.hpp"

namespace qmm {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 256;

template <class T, int BITS>
__global__ __launch_bounds__(kThreads) void qmm_prefill_kernel(const MatArgs a) {
  // operand layout in LDS: [buffer][k step (32)][lane group (8 k)][row] of 8 elements
  __shared__ u32x4 As[2][BK / 32][4][BM];
  __shared__ u32x4 Bs[2][BK / 32][4][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lg = lane >> 4;
  const int col = lane & 15;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int64_t z = blockIdx.z;
  const int64_t rows = a.rows_per_batch;
  const int64_t N = a.N;
  const int K = (int)a.K;
  const int gs = a.group_size;
  const int64_t bm0 = (int64_t)blockIdx.y * BM;
  const int64_t bn0 = (int64_t)blockIdx.x * BN;
  const uint16_t* xb = (const uint16_t*)a.x + z * a.batch_stride;

  // Global-load assignments: 4 chunks of 8 k per thread for A and for W.
  const uint16_t* arow[4];
  const uint32_t* wrow[4];
  const uint16_t* srow[4];
  const uint16_t* brow[4];
  int jk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + kThreads * i;
    const int r = id >> 3;
    jk[i] = id & 7;
    const int64_t m = bm0 + r;
    arow[i] = m < rows ? xb + (m / a.seg_rows) * a.seg_stride + (m % a.seg_rows) * a.row_stride
                       : nullptr;
    const int64_t n = bn0 + r;
    const int64_t nl = n < N ? n : N - 1;
    wrow[i] = a.w + nl * a.w_row_stride;
    srow[i] = (const uint16_t*)a.scales + nl * a.sb_row_stride;
    brow[i] = (const uint16_t*)a.biases + nl * a.sb_row_stride;
  }

  u32x4 ra[4];
  uint32_t rw0[4], rw1[4], rsb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + 8 * jk[i];
      ra[i] = arow[i] ? *(const u32x4*)(arow[i] + k) : u32x4{0u, 0u, 0u, 0u};
      if (BITS == 4) {
        rw0[i] = wrow[i][k >> 3];
        rw1[i] = 0u;
      } else if (BITS == 8) {
        rw0[i] = wrow[i][k >> 2];
        rw1[i] = wrow[i][(k >> 2) + 1];
      } else {
        const int row_words = (K * BITS) >> 5;
        const int bit0 = k * BITS;
        const int idx = bit0 >> 5;
        rw0[i] = wrow[i][idx];
        rw1[i] = wrow[i][min(idx + 1, row_words - 1)];
      }
      const int gi = k / gs;
      rsb[i] = (uint32_t)srow[i][gi] | ((uint32_t)brow[i][gi] << 16);
    }
  };
  auto lstore = [&](int buf, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid + kThreads * i) >> 3;
      const int ks = jk[i] >> 2;
      const int g = jk[i] & 3;
      As[buf][ks][g][r] = ra[i];
      const float s = T::to_f32(rsb[i] & 0xFFFFu);
      const float b = T::to_f32(rsb[i] >> 16);
      float q[8];
      if (BITS == 4) {
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (float)((rw0[i] >> (4 * e)) & 0xFu);
      } else if (BITS == 8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          q[e] = (float)((rw0[i] >> (8 * e)) & 0xFFu);
          q[4 + e] = (float)((rw1[i] >> (8 * e)) & 0xFFu);
        }
      } else {
        const int k = k0 + 8 * jk[i];
        const uint64_t v = ((((uint64_t)rw1[i]) << 32) | rw0[i]) >> ((k * BITS) & 31);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (float)((uint32_t)(v >> (e * BITS)) & ((1u << BITS) - 1u));
      }
      u32x4 wv;
      wv.x = T::pack2(__builtin_fmaf(s, q[0], b), __builtin_fmaf(s, q[1], b));
      wv.y = T::pack2(__builtin_fmaf(s, q[2], b), __builtin_fmaf(s, q[3], b));
      wv.z = T::pack2(__builtin_fmaf(s, q[4], b), __builtin_fmaf(s, q[5], b));
      wv.w = T::pack2(__builtin_fmaf(s, q[6], b), __builtin_fmaf(s, q[7], b));
      Bs[buf][ks][g][r] = wv;
    }
  };

  f32x4 acc[4][4];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4;

  const int nk = K / BK;
  gload(0);
  lstore(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      typename T::v8 av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = as_v8<T>(As[buf][ks][lg][wm * 64 + 16 * i + col]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = as_v8<T>(Bs[buf][ks][lg][wn * 64 + 16 * j + col]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = T::mfma(av[i], bv[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1, (kt + 1) * BK);
    __syncthreads();
  }

  uint16_t* yb = (uint16_t*)a.y + z * rows * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = bm0 + wm * 64 + 16 * i + 4 * lg + r;
        const int64_t n = bn0 + wn * 64 + 16 * j + col;
        if (m < rows && n < N) yb[m * N + n] = T::from_f32(acc[i][j][r]);
      }
}

template <class T, int BITS>
hipError_t launch_bits(const MatArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.rows_per_batch + BM - 1) / BM),
            (unsigned)a.batches);
  hipLaunchKernelGGL((qmm_prefill_kernel<T, BITS>), grid, dim3(kThreads), 0, stream, a);
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
  if (a.rows_per_batch <= 0 || a.batches > 65535 || (a.rows_per_batch + BM - 1) / BM > 65535)
    return hipErrorInvalidValue;
  return a.dtype == 1 ? launch_dtype<Bf16>(a, stream) : launch_dtype<Fp16>(a, stream);
}

}  // namespace qmm
