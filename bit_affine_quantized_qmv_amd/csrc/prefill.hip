// Prefill family: y = x . dequant(W)^T for more than 32 activation rows (qmm_t).
//
// A dense bf16/fp16 GEMM on the matrix cores (16x16x32 MFMA, float32 accumulators, one
// fixed K order, no split-K).  Each K tile of the packed weight is unpacked and
// dequantized, w~ = s*q + b rounded to the storage dtype, into LDS next to the activation
// tile; the products then see ordinary half-precision operands.  The epilogue stores each
// output row through the plan's row addressing, which also serves strided batches such as
// a view narrowed on the sequence dimension (transformers issue 47331, layout table: every
// row of every batch element must be computed).
//
// Two kernels share this arithmetic and the 256 x 256 x 64 tiling.  qmm_prefill_kernel
// stages the activation tile through registers.  qmm_prefill_dma_kernel (2-, 4- and 8-bit
// codes) moves it with direct global-to-LDS loads a whole step ahead, and keeps the weight
// codes of two steps in registers, so both loads have a full step of MFMAs to land behind.
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

// Epilogue: a wave's 64 x 128 outputs pass through 16 KB of LDS that the main loop no
// longer reads, 32 rows at a time with a padded row stride (the four lane groups' 2-byte
// writes land in distinct banks), and leave as 16-byte stores of 8 consecutive columns of
// one output row; columns past N, or a y that does not allow 16-byte stores, take 2-byte
// stores of the same values.
constexpr int kYStride = 136;   // halfwords per staged output row (128 + 8)

// the area is the wave's own: its LDS accesses complete in order, the fences only keep the
// compiler from moving them across one another
__device__ inline void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <class T, int FM, int FN>
__device__ inline void store_wave_tile(const f32x4 (&acc)[FM][FN], uint16_t* area, uint16_t* yb, int64_t rows,
                                       int64_t N, int64_t m0, int64_t n0, int lane, bool vec_ok) {
  static_assert(FM == 4 && FN == 8, "a 64 x 128 wave tile, staged as two halves of 32 rows");
  const int lg = lane >> 4, col = lane & 15;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          area[(16 * ii + 4 * lg + r) * kYStride + 16 * j + col] = T::from_f32(acc[2 * h + ii][j][r]);
    wave_lds_order();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int rr = 4 * q + lg;
      const u32x4 v = *(const u32x4*)(area + rr * kYStride + 8 * col);
      const int64_t m = m0 + 32 * h + rr;
      const int64_t n = n0 + 8 * col;
      if (m < rows) {
        uint16_t* dst = yb + m * N + n;
        if (vec_ok && n + 8 <= N) {
          *(u32x4*)dst = v;
        } else {
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
    wave_lds_order();
  }
}

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

  // the main loop's last barrier is behind every LDS read of its operands: each wave takes
  // 16 KB of the operand buffers for its outputs
  uint16_t* yb = (uint16_t*)a.y + z * rows * N;
  const bool vec_ok = N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0u;
  uint16_t* area = (uint16_t*)(wave < 4 ? (u32x4*)As : (u32x4*)Bs) + (wave & 3) * 8192;
  store_wave_tile<T, FM, FN>(acc, area, yb, rows, N, bm0 + wm * TM, bn0 + wn * TN, lane, vec_ok);
}

// Bytes the activation descriptor of the direct-load kernel spans from a batch's first
// row; the launcher checks that the rows it reads lie inside.
constexpr uint32_t kXRange = 0x7FFFFF00u;

typedef __attribute__((address_space(3))) void lds_void_t;

template <class T, int BITS>
__global__ __launch_bounds__(kThreads, 1) void qmm_prefill_dma_kernel(const MatArgs a, const int m_tiles) {
  // Activation tile: row-major, 256 rows x 64 k (eight 16-byte chunks per row); chunk c of
  // row r sits at position c ^ ((r >> 1) & 7), so the 16 rows one MFMA operand read touches
  // fall in distinct LDS banks.  It is filled by direct global-to-LDS loads: one 64-lane
  // load writes 1 KB of LDS (8 whole rows), reading 8 whole 128-byte lines of x.
  // Weight tile: [k half (32)][lane group (8 k)][row] of 8 dequantized values.
  // Separate arrays per buffer let the compiler see that reading one buffer does not
  // depend on the direct loads still landing in the other.
  __shared__ u32x4 As0[BM * 8], As1[BM * 8];
  __shared__ u32x4 Bs0[BK / 32][4][BN], Bs1[BK / 32][4][BN];
  constexpr int TM = BM / WM, TN = BN / WN;      // wave tile
  constexpr int FM = TM / 16, FN = TN / 16;      // 16x16 MFMA blocks per wave tile
  constexpr int A_LOADS = BM * 8 / 64 / (kThreads / 64);   // 64-lane activation loads per wave
  static_assert(BN * 2 == kThreads, "one thread per 32 codes of a weight row");
  static_assert(FM == 4 && A_LOADS == 4, "tile shape");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int gs_shift = __builtin_ctz((unsigned)a.group_size);   // group sizes are powers of two
  const int64_t bm0 = (int64_t)mt * BM;
  const int64_t bn0 = (int64_t)nt * BN;
  const uint16_t* xb = (const uint16_t*)a.x + z * a.batch_stride;

  // activation loads: load j of this wave covers tile rows r0 = 8 * (4 * wave + j) .. r0 + 7;
  // lane i fills position i % 8 of row r0 + i / 8, i.e. logical chunk (i % 8) ^ ((r >> 1) & 7)
  // Byte offsets into the batch's activations (a descriptor of 2 GiB, which the host checks
  // the rows fit in); lanes past the call's rows or past K get an offset past the
  // descriptor's end and so read zeros.
  const __amdgpu_buffer_rsrc_t x_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xb), (short)0,
                                                                       (int)kXRange, 0x00020000);
  constexpr uint32_t kPast = kXRange;   // at or past the end: the whole chunk reads zero
  uint32_t aoff[A_LOADS];
  int ak[A_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int r = 8 * (A_LOADS * wave + j) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int64_t m = bm0 + r;
    const int64_t mr = m < rows ? m : 0;
    ak[j] = 8 * c;
    aoff[j] = m < rows ? (uint32_t)(2 * ((mr / a.seg_rows) * a.seg_stride + (mr % a.seg_rows) * a.row_stride + 8 * c))
                       : kPast;
  }
  // When K is not a multiple of BK the last step is partial: activation chunks at k >= K
  // read zeros, and code runs at k >= K read the row's first run and are zeroed (K is a
  // multiple of 32, so a chunk or run is either wholly inside or wholly outside the row).
  uint32_t aoff_k[A_LOADS];   // this step's offsets, kept allocated until the step's wait
  auto load_a = [&](int kt, u32x4* dst) {
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
      aoff_k[j] = (k0 + ak[j] < K && aoff[j] != kPast) ? aoff[j] + 2u * (uint32_t)k0 : kPast;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rs, (lds_void_t*)(dst + 64 * (A_LOADS * wave + j)), 16, aoff_k[j], 0,
                                               0, 0);
    }
  };
  // weight: thread -> row wr, 32-code half wh of the 64 k of a step
  const int wr = tid >> 1, wh = tid & 1;
  const int64_t wn_row = bn0 + wr < N ? bn0 + wr : N - 1;
  const uint32_t* wrow = a.w + wn_row * a.w_row_stride;
  const uint16_t* srow = (const uint16_t*)a.scales + wn_row * a.sb_row_stride;
  const uint16_t* brow = (const uint16_t*)a.biases + wn_row * a.sb_row_stride;
  // two register sets of weight codes, scale and bias, used by alternate steps
  uint32_t rwA[BITS], rwB[BITS];
  uint32_t rsA = 0, rbA = 0, rsB = 0, rbB = 0;
  // (a run at k >= K reads the row's first run; its scale and bias are zeroed at use)
  auto load_w = [&](int kt, uint32_t(&rw)[BITS], uint32_t& rs, uint32_t& rb) {
    const int kw = kt * BK + 32 * wh;
    const bool wv_ok = kw < K;
    load_codes<BITS>(rw, wrow + (wv_ok ? kw / 32 * BITS : 0));
    const int g = wv_ok ? kw >> gs_shift : 0;
    rs = srow[g];
    rb = brow[g];
  };
  // w~ of the run loaded for step kt, zero past K
  auto dequant_w = [&](int kt, const uint32_t(&rw)[BITS], uint32_t rs, uint32_t rb, u32x4(&wv)[4]) {
    const bool wv_ok = kt * BK + 32 * wh < K;
    dequant32<T, BITS>(rw, wv_ok ? T::to_f32(rs) : 0.f, wv_ok ? T::to_f32(rb) : 0.f, wv);
  };

  f32x4 acc[FM][FN];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = zero4;

  // MFMA operand positions: row R = wm * TM + 16 * i + col has (R >> 1) & 7 == col >> 1
  const int aswz = col >> 1;
  const int nk = (K + BK - 1) / BK;

  // One k step.  The MFMAs read buffer `cur`; the weights of step kt+1 (registers rw/rs/rb,
  // loaded two steps earlier) are dequantized and written to the other buffer between the
  // first half of the MFMAs, and the activations of step kt+1 land there through direct
  // loads issued right after that dequantization; the weight registers are refilled with
  // step kt+3 at the end of the step.
  // Before the barrier every load of this wave older than that refill has landed (the
  // direct loads included), so one barrier per step orders everything.
  auto step = [&](int kt, u32x4* Acur, u32x4* Anxt, u32x4(&Bcur)[BK / 32][4][BN], u32x4(&Bnxt)[BK / 32][4][BN],
                  uint32_t(&rw)[BITS], uint32_t& rs, uint32_t& rb) {
    typename T::v8 av[FM], bv[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) av[i] = as_v8<T>(Acur[(wm * TM + 16 * i + col) * 8 + (lg ^ aswz)]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bv[j] = as_v8<T>(Bcur[0][lg][wn * TN + 16 * j + col]);
    // The weight registers are read through an opaque zero made here, so no use of them is
    // moved above the previous step's barrier, where it would wait for the loads still
    // landing (the other register set's, and the direct activation loads).
    uint32_t opq;
    asm volatile("s_mov_b32 %0, 0" : "=s"(opq));
    uint32_t rwo[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) rwo[i] = rw[i] ^ opq;
    u32x4 wv[4];
    dequant_w(kt + 1, rwo, rs ^ opq, rb ^ opq, wv);
    load_a(kt + 1, Anxt);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = T::mfma(av[i], bv[j], acc[i][j]);
      Bnxt[wh][i][wr] = wv[i];
    }
#pragma unroll
    for (int t = 0; t < FM * FN; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // three VALU
      if (t % 8 == 7) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // one LDS write
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) av[i] = as_v8<T>(Acur[(wm * TM + 16 * i + col) * 8 + ((4 + lg) ^ aswz)]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bv[j] = as_v8<T>(Bcur[1][lg][wn * TN + 16 * j + col]);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = T::mfma(av[i], bv[j], acc[i][j]);
    // vmcnt(0): the direct activation loads of step kt+1 (and the weights of step kt+2).
    // Their offset registers stay allocated until here: the compiler counts a direct load
    // as writing its offset register, so a value placed in that register while the load is
    // in flight would make it wait for the load there.
    // The accumulators pass through empty statements first, so that the step's MFMAs are
    // not moved below the wait.  (The fp16 instantiation keeps the compiler's order: with
    // the pin it no longer fits 256 registers.)
    if constexpr (T::kDtype == 1) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(acc[i][j]));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) asm volatile("" ::"v"(aoff_k[j]));
    load_w(kt + 3, rw, rs, rb);
    lds_barrier();
  };

  // prologue: activations and weights of step 0 in buffer 0, weights of steps 1 and 2 in
  // registers
  load_w(0, rwA, rsA, rbA);
  load_a(0, As0);
  load_w(1, rwB, rsB, rbB);
  {
    u32x4 wv[4];
    dequant_w(0, rwA, rsA, rbA, wv);
#pragma unroll
    for (int c = 0; c < 4; ++c) Bs0[wh][c][wr] = wv[c];
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  load_w(2, rwA, rsA, rbA);
  lds_barrier();
  // Steps run in pairs, so that every register set and buffer is named statically; an odd
  // step count gets one more step whose operands are all zero (activations past K read the
  // zeros through the descriptor, weights past K have zero scale and bias), which adds nothing.
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, As0, As1, Bs0, Bs1, rwB, rsB, rbB);
    step(kt + 1, As1, As0, Bs1, Bs0, rwA, rsA, rbA);
  }

  // the main loop's last barrier is behind every LDS read of its operands and every direct
  // load into them: each wave takes 16 KB of the operand buffers for its outputs
  uint16_t* yb = (uint16_t*)a.y + z * rows * N;
  const bool vec_ok = N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0u;
  const int quarter = wave >> 1;
  u32x4* const base = quarter == 0 ? As0 : quarter == 1 ? As1 : quarter == 2 ? &Bs0[0][0][0] : &Bs1[0][0][0];
  uint16_t* area = (uint16_t*)base + (wave & 1) * 8192;
  store_wave_tile<T, FM, FN>(acc, area, yb, rows, N, bm0 + wm * TM, bn0 + wn * TN, lane, vec_ok);
}

template <class T, int BITS>
hipError_t launch_bits(const MatArgs& a, hipStream_t stream) {
  const int64_t m_tiles = (a.rows_per_batch + BM - 1) / BM;
  const int64_t n_tiles = (a.N + BN - 1) / BN;
  if (m_tiles * n_tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(m_tiles * n_tiles), 1, (unsigned)a.batches);
  // 2-, 4- and 8-bit codes take the kernel with direct activation loads (when a batch's
  // activations fit its descriptor); at 3, 5 and 6 bits its register budget (256 per lane
  // at two waves per SIMD) does not hold without spills
  // activation elements a batch spans (rows through the plan's row addressing, plus K)
  const int64_t rpb = a.rows_per_batch;
  const int64_t seg_rows_used = rpb < a.seg_rows ? rpb : a.seg_rows;
  const int64_t span = (rpb - 1) / a.seg_rows * a.seg_stride + (seg_rows_used - 1) * a.row_stride + a.K;
  if constexpr (BITS == 2 || BITS == 4 || BITS == 8) {
    if (2 * span <= (int64_t)kXRange) {
      hipLaunchKernelGGL((qmm_prefill_dma_kernel<T, BITS>), grid, dim3(kThreads), 0, stream, a, (int)m_tiles);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((qmm_prefill_kernel<T, BITS>), grid, dim3(kThreads), 0, stream, a, (int)m_tiles);
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
