// Decode-family kernels and their launchers (instantiated per code width in decode_b*.hip).
//
// qmv_stream_kernel: the activations (all rows, all K) stay resident in LDS; every wave
//   owns a contiguous range of 16-row weight tiles and streams them through a ring of
//   DEPTH slots of in-flight 16-byte loads, so the HBM stream never waits on the MFMAs.
//   The first loads are issued before the activations are staged.
// qmv_chunk_kernel: for activations too large for LDS; K is processed in chunks staged
//   one after another, each wave keeping TN tiles' accumulators across chunks.
// Both compute exactly the per-element arithmetic described in decode_impl.hpp.
#pragma once

#include <algorithm>

#include "decode_impl.hpp"

namespace qmm {
namespace decode {

constexpr int kChunkTiles = 2;
constexpr int kLdsLimit = 160 * 1024;
constexpr int kChunkXBytes = 64 * 1024;

template <class T, int BITS, int GS, int MT, int D>
__global__ __launch_bounds__(kThreads) void qmv_stream_kernel(const MatArgs a, const int tiles_base,
                                                              const int tiles_rem) {
  // D = slots per block of the main loop; it divides the slots per tile, so a block never
  // straddles two tiles and every in-block slot offset is a compile-time constant.
  using S = Slot<BITS, GS>;
  constexpr int MROWS = 16 * MT;
  constexpr bool kBuf = BITS == 4 || BITS == 8;
  extern __shared__ u32x4 smem[];
  const int K = (int)a.K;
  u32x4* xs = smem;
  float* sxs = (float*)(smem + (K / 32) * 4 * MROWS);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The buffer-descriptor path needs the wave index in a scalar register.  The other code
  // widths keep it per lane: their fp16 instantiations gave run-to-run different results
  // with the scalar form, and that form buys them nothing.
  const int wave = kBuf ? __builtin_amdgcn_readfirstlane(tid >> 6) : (tid >> 6);
  const int lg = lane >> 4;
  const int col = lane & 15;
  const int64_t z = blockIdx.z;
  const uint16_t* xb = (const uint16_t*)a.x + z * a.batch_stride;
  const int rows = (int)a.rows_per_batch;
  const int64_t N = a.N;
  uint16_t* yb = (uint16_t*)a.y + z * (int64_t)rows * N;
  const int w_row_bytes = (int)(a.w_row_stride * 4);
  const int sb_row_bytes = (int)(a.sb_row_stride * 2);
  const int w_voff = col * w_row_bytes + 16 * lg;
  const int sb_voff = col * sb_row_bytes;

  // Balanced split of the 16-row tiles over the grid's waves: tiles_rem waves take
  // tiles_base + 1 tiles, the others tiles_base (both computed on the host).  Ranges are
  // assigned in the order (wave-in-workgroup, workgroup), so the waves holding an extra tile
  // are spread over all workgroups (and CUs) instead of packed into the first ones.
  const int v = wave * (int)gridDim.x + (int)blockIdx.x;
  const int64_t t_begin = (int64_t)v * tiles_base + min(v, tiles_rem);
  const int64_t t_end = t_begin + tiles_base + (v < tiles_rem ? 1 : 0);
  const int nit = K / S::kSpan;              // slots per tile (a multiple of D)
  const int row_words = (K * BITS) >> 5;

  int gword = 0;
  uint32_t gshift = 0;
  if constexpr (!kBuf) generic_lane_offsets<BITS>(lg, gword, gshift);

  // ---- load stream: block (ld_tile, ld_kb); descriptors rebuilt only on a new tile
  const int64_t w_tile_words = 16 * a.w_row_stride;
  const int64_t sb_tile_elems = 16 * a.sb_row_stride;
  __amdgpu_buffer_rsrc_t w_rs, s_rs, b_rs;
  auto make_tile_rsrc = [&](int64_t tile) {
    const int64_t r0 = tile * 16;
    const int valid = (int)(N - r0 < 16 ? N - r0 : 16);
    w_rs = make_rsrc(a.w + tile * w_tile_words, (uint32_t)(valid * w_row_bytes));
    s_rs = make_rsrc((const uint16_t*)a.scales + tile * sb_tile_elems, (uint32_t)(valid * sb_row_bytes));
    b_rs = make_rsrc((const uint16_t*)a.biases + tile * sb_tile_elems, (uint32_t)(valid * sb_row_bytes));
  };
  int64_t ld_tile = t_begin < t_end ? t_begin : 0;
  int ld_kb = 0;   // first slot of the block being loaded
  if constexpr (kBuf) make_tile_rsrc(ld_tile);
  SlotData<BITS, GS> ring[D];
  auto issue_slot = [&](int j) {
    const int kit = ld_kb + j;
    if constexpr (kBuf) {
      load_slot_buf<BITS, GS>(ring[j], w_rs, s_rs, b_rs, w_voff, kit * S::kRowWordsPerSlot * 4, sb_voff,
                              kit * S::kGroups * 2);
    } else {
      const int64_t n = ld_tile * 16 + col;
      const int64_t nl = n < N ? n : N - 1;
      load_slot<BITS, GS>(ring[j], a.w + nl * a.w_row_stride + (int64_t)kit * S::kRowWordsPerSlot,
                          (const uint16_t*)a.scales + nl * a.sb_row_stride + kit * S::kGroups,
                          (const uint16_t*)a.biases + nl * a.sb_row_stride + kit * S::kGroups, lg, gword,
                          row_words - kit * S::kRowWordsPerSlot);
    }
  };
  // move the load stream to the next block.  Past the wave's last block the buffer path
  // switches to empty descriptors, whose loads return zeros without touching memory; the
  // pointer path keeps reloading its last block (cache hits).  Neither is ever consumed.
  auto advance = [&]() {
    if (ld_kb + D < nit) {
      ld_kb += D;
    } else if (ld_tile + 1 < t_end) {
      ++ld_tile;
      ld_kb = 0;
      if constexpr (kBuf) make_tile_rsrc(ld_tile);
    } else if constexpr (kBuf) {
      w_rs = make_rsrc(a.w, 0u);
      s_rs = make_rsrc(a.scales, 0u);
      b_rs = make_rsrc(a.biases, 0u);
    }
  };

  // ---- activations first (their loads must retire before the weight prefetch), then the
  // first block's loads, then the LDS writes of the first staging batch, then any others
  const uint16_t* xr = stage_row<T, BITS, MROWS>(a, xb, rows, tid);
  const int nbatch = stage_batches<MROWS>(K, kThreads);
  {
    XStage<MROWS> st;
    stage_x_issue<T, BITS, MROWS>(st, xr, 0, K, 0, tid, kThreads);
#pragma unroll
    for (int j = 0; j < D; ++j) issue_slot(j);
    stage_x_commit<T, BITS, MROWS>(st, xs, rows, K, 0, tid, kThreads);
  }
  for (int batch = 1; batch < nbatch; ++batch) {
    XStage<MROWS> st;
    stage_x_issue<T, BITS, MROWS>(st, xr, 0, K, batch, tid, kThreads);
    stage_x_commit<T, BITS, MROWS>(st, xs, rows, K, batch, tid, kThreads);
  }
  lds_barrier();
  sum_x<T, GS, MT>(xs, sxs, K, wave, kWaves, lane);
  lds_barrier();
  if (t_end <= t_begin) return;

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[MT], part[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt] = zero4;
    part[mt] = zero4;
  }
  for (int64_t tile = t_begin; tile < t_end; ++tile) {
    for (int kb = 0; kb < nit; kb += D) {
      // consume the block slot by slot, refilling each slot with the next block's slot
      advance();
#pragma unroll
      for (int j = 0; j < D; ++j) {
        consume_slot<T, BITS, GS, MT>(ring[j], xs, sxs, (kb + j) * S::kSpan, acc, part, lg, col, gshift);
        issue_slot(j);
      }
    }
    store_tile<T, MT>(acc, yb, rows, tile * 16 + col, N, lg);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = zero4;
  }
}

template <class T, int BITS, int GS, int MT, int TN>
__global__ __launch_bounds__(kThreads) void qmv_chunk_kernel(const MatArgs a) {
  using S = Slot<BITS, GS>;
  constexpr int MROWS = 16 * MT;
  constexpr int KC = kChunkXBytes / (MROWS * 2);
  __shared__ u32x4 xs[kChunkXBytes / 16];
  __shared__ float sxs[(KC / 32) * MROWS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lg = lane >> 4;
  const int col = lane & 15;
  const int64_t z = blockIdx.z;
  const uint16_t* xb = (const uint16_t*)a.x + z * a.batch_stride;
  const int rows = (int)a.rows_per_batch;
  const int64_t N = a.N;
  const int K = (int)a.K;
  const int row_words = (K * BITS) >> 5;
  uint16_t* yb = (uint16_t*)a.y + z * (int64_t)rows * N;

  int gword = 0;
  uint32_t gshift = 0;
  if constexpr (BITS != 4 && BITS != 8) generic_lane_offsets<BITS>(lg, gword, gshift);

  int64_t nrow[TN], nl[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    nrow[t] = ((int64_t)(blockIdx.x * kWaves + wave) * TN + t) * 16 + col;
    nl[t] = nrow[t] < N ? nrow[t] : N - 1;
  }
  auto issue = [&](SlotData<BITS, GS> (&d)[TN], int kit) {
#pragma unroll
    for (int t = 0; t < TN; ++t)
      load_slot<BITS, GS>(d[t], a.w + nl[t] * a.w_row_stride + (int64_t)kit * S::kRowWordsPerSlot,
                          (const uint16_t*)a.scales + nl[t] * a.sb_row_stride + kit * S::kGroups,
                          (const uint16_t*)a.biases + nl[t] * a.sb_row_stride + kit * S::kGroups, lg, gword,
                          row_words - kit * S::kRowWordsPerSlot);
  };

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[TN][MT], part[TN][MT];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[t][mt] = zero4;
      part[t][mt] = zero4;
    }

  const int nit_total = K / S::kSpan;
  SlotData<BITS, GS> cur[TN], nxt[TN];
  issue(cur, 0);
  for (int kc0 = 0; kc0 < K; kc0 += KC) {
    const int kcl = min(KC, K - kc0);
    lds_barrier();
    stage_x<T, BITS, MROWS>(xs, a, xb, rows, kc0, kcl, tid, kThreads);
    lds_barrier();
    sum_x<T, GS, MT>(xs, sxs, kcl, wave, kWaves, lane);
    lds_barrier();
    const int kit0 = kc0 / S::kSpan;
    const int nit = kcl / S::kSpan;
    for (int i = 0; i < nit; ++i) {
      const int kit = kit0 + i;
      issue(nxt, min(kit + 1, nit_total - 1));
#pragma unroll
      for (int t = 0; t < TN; ++t)
        consume_slot<T, BITS, GS, MT>(cur[t], xs, sxs, i * S::kSpan, acc[t], part[t], lg, col, gshift);
#pragma unroll
      for (int t = 0; t < TN; ++t) cur[t] = nxt[t];
    }
  }
#pragma unroll
  for (int t = 0; t < TN; ++t) store_tile<T, MT>(acc[t], yb, rows, nrow[t], N, lg);
}

// ----------------------------------------------------------------------------- launchers
int device_cus();

template <class T, int BITS, int GS, int MT, int D>
hipError_t launch_stream_d(const MatArgs& a, hipStream_t stream, int lds) {
  auto kern = qmv_stream_kernel<T, BITS, GS, MT, D>;
  static int per_cu = -1;  // occupancy for this instantiation (same LDS class each call)
  static int lds_cached = -1;
  if (lds_cached != lds) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kThreads, lds);
    if (e != hipSuccess) return e;
    per_cu = nb > 0 ? nb : 1;
    lds_cached = lds;
  }
  // one full wave of workgroups (every CU at its occupancy), tiles spread over all waves
  const int64_t n_tiles = (a.N + 15) / 16;
#ifndef QMM_MAX_WG_PER_CU
#define QMM_MAX_WG_PER_CU 8
#endif
  const int64_t full = (int64_t)device_cus() * std::min(per_cu, QMM_MAX_WG_PER_CU);
  const int64_t blocks = std::min<int64_t>(full, (n_tiles + kWaves - 1) / kWaves);
  const int64_t waves_total = blocks * kWaves;
  if (n_tiles / waves_total > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks, 1, (unsigned)a.batches), dim3(kThreads), lds, stream, a,
                     (int)(n_tiles / waves_total), (int)(n_tiles % waves_total));
  return hipGetLastError();
}

// Slots per main-loop block: the largest of 8, 4, 2, 1 dividing the slots per tile.
template <class T, int BITS, int GS, int MT>
hipError_t launch_stream(const MatArgs& a, hipStream_t stream, int lds) {
  const int nit = (int)(a.K / Slot<BITS, GS>::kSpan);
#ifndef QMM_MAX_BLOCK_SLOTS
#define QMM_MAX_BLOCK_SLOTS 4
#endif
  if (QMM_MAX_BLOCK_SLOTS >= 8 && nit % 8 == 0) return launch_stream_d<T, BITS, GS, MT, 8>(a, stream, lds);
  if (QMM_MAX_BLOCK_SLOTS >= 4 && nit % 4 == 0) return launch_stream_d<T, BITS, GS, MT, 4>(a, stream, lds);
  if (nit % 2 == 0) return launch_stream_d<T, BITS, GS, MT, 2>(a, stream, lds);
  return launch_stream_d<T, BITS, GS, MT, 1>(a, stream, lds);
}

template <class T, int BITS, int GS, int MT>
hipError_t launch_chunk(const MatArgs& a, hipStream_t stream) {
  const int64_t rows_per_wg = (int64_t)kWaves * kChunkTiles * 16;
  dim3 grid((unsigned)((a.N + rows_per_wg - 1) / rows_per_wg), 1, (unsigned)a.batches);
  hipLaunchKernelGGL((qmv_chunk_kernel<T, BITS, GS, MT, kChunkTiles>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int MT, int GS>
constexpr int stream_lds_bytes(int K) {
  return 16 * MT * K * 2 + (K / GS) * 16 * MT * 4;
}

template <class T, int BITS, int GS>
hipError_t launch_gs(const MatArgs& a, hipStream_t stream) {
  const int K = (int)a.K;
  if (a.rows_per_batch <= 16) {
    const int lds = stream_lds_bytes<1, GS>(K);
    return lds <= kLdsLimit ? launch_stream<T, BITS, GS, 1>(a, stream, lds) : launch_chunk<T, BITS, GS, 1>(a, stream);
  }
  const int lds = stream_lds_bytes<2, GS>(K);
  return lds <= kLdsLimit ? launch_stream<T, BITS, GS, 2>(a, stream, lds) : launch_chunk<T, BITS, GS, 2>(a, stream);
}

template <int BITS>
hipError_t launch_bits(const MatArgs& a, hipStream_t stream) {
  const bool bf = a.dtype == 1;
  switch (a.group_size) {
    case 32: return bf ? launch_gs<Bf16, BITS, 32>(a, stream) : launch_gs<Fp16, BITS, 32>(a, stream);
    case 64: return bf ? launch_gs<Bf16, BITS, 64>(a, stream) : launch_gs<Fp16, BITS, 64>(a, stream);
    case 128: return bf ? launch_gs<Bf16, BITS, 128>(a, stream) : launch_gs<Fp16, BITS, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_b4(const MatArgs& a, hipStream_t stream);
hipError_t launch_decode_b8(const MatArgs& a, hipStream_t stream);
hipError_t launch_decode_bn(const MatArgs& a, hipStream_t stream);

}  // namespace decode
}  // namespace qmm
