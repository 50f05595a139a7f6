// Decode-family kernels and their launchers (instantiated per code width in decode_b*.hip).
//
// qmv_stream_kernel: the staged activation rows (all K) stay resident in LDS; every wave
//   owns a range of pairs of 16-row weight tiles and streams their whole rows through a
//   register ring of in-flight 16-byte loads, so the HBM stream never waits on the MFMAs.
//   The weight prefetch is issued right behind the activation loads.
// qmv_parts_kernel (decode_parts.hpp): rows cut into parts along K, worked on by several
//   waves at once (matrices with few rows or long K).
// qmv_chunk_kernel: for activations too large for LDS; K is processed in chunks staged
//   one after another, each wave keeping TN tiles' accumulators across chunks.
// All compute exactly the per-element arithmetic described in decode_impl.hpp.
#pragma once

#include <algorithm>

#include "decode_impl.hpp"

namespace qmm {
namespace decode {

constexpr int kChunkTiles = 1;   // 16-row tiles per wave in the chunked kernel (more workgroups)
constexpr int kLdsLimit = 160 * 1024;
constexpr int kChunkXBytes = 64 * 1024;

// Eight waves per workgroup, two per SIMD (the kernels' register budget is 256): more waves
// per workgroup or per SIMD measured slower on the lm_head weight.
constexpr int kStreamWaves = 8;
constexpr int kStreamThreads = 64 * kStreamWaves;
constexpr int kStreamWavesPerSimd = 2;
constexpr int kPair = 2;         // weight tiles consumed together per slot
constexpr int kRingFactor = 2;   // sub-blocks of weight loads in flight
constexpr int kMaxWgPerCu = 8;   // cap on resident workgroups per compute unit in the grid size

template <class T, int BITS, int GS, int MT, int D, bool SBB, int XRL>
__global__ __launch_bounds__(kStreamThreads, kStreamWavesPerSimd) void qmv_stream_kernel(const MatArgs a,
                                                                                     const int pairs_base,
                                                                                     const int pairs_rem,
                                                                                     const int y_area) {
  // The slots of a wave's tile pairs form one stream, consumed in sub-blocks of D slots (D
  // divides the slots per tile, so a pair always ends on a sub-block boundary).  Weight
  // loads run kRingFactor*D slots ahead of consumption (a ring of that many slots); with SBB the scales and
  // biases are loaded once per sub-block, one vector load per tile row, D slots ahead, into
  // two register sets used by alternate sub-blocks; without it each slot carries its own.
  using S = Slot<BITS, GS>;
  constexpr int MROWS = 16 * MT;
  constexpr int TN = kPair;
  // With one 16-row tile of activations (and the per-sub-block scale loads) the registers
  // hold a ring twice as deep, refilled a whole sub-block at a time after it is consumed:
  // 6-7% faster on a 151936 x 1024 weight at 1-16 activation rows.  Two tiles keep the
  // shallower ring with per-slot refills, which measured faster there.
  constexpr bool kDeepRing = MT == 1 && SBB;
  constexpr int RF = kDeepRing ? 2 * kRingFactor : kRingFactor;
  constexpr int R = RF * D;
  // one bias MFMA per two slots (the launcher picks D >= 2 exactly when the slots per row
  // are even, which is when bias_span gives 2)
  constexpr bool kPairBias = GS >= 64 && D >= 2;
  constexpr bool kBuf = BITS == 4 || BITS == 8;
  static_assert(!SBB || kBuf, "block scale/bias loads use the buffer path");
  constexpr int NHB = D * S::kGroups;   // scale (or bias) halfwords per tile row per sub-block
  extern __shared__ u32x4 smem[];
  const int K = (int)a.K;
  const int Kp = (K + S::kSpan - 1) / S::kSpan * S::kSpan;   // K rounded up to whole slots
  constexpr int xrl = XRL;   // 2^xrl activation rows in LDS (x_lds_rows_log2)
  u32x4* xs = smem;
  float* sxs = (float*)(smem + (((Kp / 32) * 4) << xrl));

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
  const int rows = (int)(a.last_rows != 0 && z == a.batches - 1 ? a.last_rows : a.rows_per_batch);
  const int64_t N = a.N;
  uint16_t* yb = (uint16_t*)a.y + z * a.rows_per_batch * N;
  const int w_row_bytes = (int)(a.w_row_stride * 4);
  const int sb_row_bytes = (int)(a.sb_row_stride * 2);
  const bool sb_narrow = !sb_rows_aligned<S::kGroups>(a) || K % S::kSpan != 0;
  int w_voff[TN], sb_voff[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    w_voff[t] = (16 * t + col) * w_row_bytes + 16 * lg;
    sb_voff[t] = (16 * t + col) * sb_row_bytes;
  }

  // Balanced split of the tile pairs (16-row tiles taken two at a time) over the grid's
  // waves: pairs_rem waves take pairs_base + 1 pairs, the others pairs_base (both computed on
  // the host).  Ranges are assigned in the order (wave-in-workgroup, workgroup), so the waves
  // holding an extra pair are spread over all workgroups and, within a workgroup, over
  // different SIMDs first.  Only the very last pair of the matrix can have an empty second
  // tile (zero loads, no store).
  const int v = wave * (int)gridDim.x + (int)blockIdx.x;
  const int64_t n_tiles = (a.N + 15) >> 4;
  const int64_t p_begin = (int64_t)v * pairs_base + min(v, pairs_rem);
  const int64_t p_end = p_begin + pairs_base + (v < pairs_rem ? 1 : 0);
  const int64_t t_begin = p_begin * TN;
  const int64_t t_end = p_end * TN < n_tiles ? p_end * TN : n_tiles;
  const int nit = Kp / S::kSpan;             // slots per tile (a multiple of D)
  const int row_words = (K * BITS) >> 5;
  // fused argmax: per-row keys of the workgroup, after the activation sums
  unsigned long long* kl = (unsigned long long*)(sxs + sx_floats(K / GS, xrl));
  const bool do_argmax = a.argmax_keys != nullptr;
  const bool store_y = a.y != nullptr;
  // Whole tile pairs store through the wave's LDS area when the launch gave it one (it
  // follows the argmax keys).  y_area is the number of pairs the area holds: 1 stores each
  // pair as it completes; more (the launch then holds every pair of the wave's range) keeps
  // them all and stores them after the wave's weight stream ends.
  const bool y_vec = y_area != 0 && N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0u;
  const bool y_defer = y_area > 1;
  constexpr int kPairHalves = y_pair_halves<MT>();
  uint16_t* ys_area = (uint16_t*)(kl + MROWS) + wave * (y_area * kPairHalves);

  int gword = 0;
  uint32_t gshift = 0;
  if constexpr (!kBuf) generic_lane_offsets<BITS>(lg, gword, gshift);

  // Descriptors over the rows of tile pair p that lie in [0, N) and in the wave's range;
  // past the range they are empty (loads return zero without touching memory).
  auto rows_valid = [&](int64_t p) -> uint32_t {
    if (p >= t_end) return 0u;
    int64_t valid = N - p * 16 < 16 * TN ? N - p * 16 : 16 * TN;
    valid = valid < (t_end - p) * 16 ? valid : (t_end - p) * 16;
    return (uint32_t)valid;
  };
  const WeightBase wb = weight_base(a, z);
  auto w_rsrc = [&](int64_t p) { return make_rsrc(wb.w + p * 16 * a.w_row_stride, rows_valid(p) * w_row_bytes); };
  auto s_rsrc = [&](int64_t p) { return make_rsrc(wb.s + p * 16 * a.sb_row_stride, rows_valid(p) * sb_row_bytes); };
  auto b_rsrc = [&](int64_t p) { return make_rsrc(wb.b + p * 16 * a.sb_row_stride, rows_valid(p) * sb_row_bytes); };

  // ---- weight stream: next sub-block to load is slots [w_kb, w_kb + D) of pair w_p
  int64_t w_p = t_begin;
  int w_kb = 0;
  __amdgpu_buffer_rsrc_t w_rs, ws_rs, wb_rs;
  if constexpr (kBuf) {
    w_rs = w_rsrc(w_p);
    if constexpr (!SBB) {
      ws_rs = s_rsrc(w_p);
      wb_rs = b_rsrc(w_p);
    }
  }
  SlotData<BITS, GS> ring[R][TN];
  auto issue_w = [&](int j, int r) {
    const int kit = w_kb + j;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      if constexpr (kBuf) {
        load_slot_buf<BITS, GS, !SBB>(ring[r][t], w_rs, ws_rs, wb_rs, w_voff[t], kit * S::kRowWordsPerSlot * 4,
                                      sb_voff[t], kit * S::kGroups * 2, sb_narrow);
      } else {
        const int64_t n = w_p * 16 + 16 * t + col;
        const int64_t nl = n < N ? n : N - 1;
        load_slot<BITS, GS>(ring[r][t], wb.w + nl * a.w_row_stride + (int64_t)kit * S::kRowWordsPerSlot,
                            wb.s + nl * a.sb_row_stride + kit * S::kGroups,
                            wb.b + nl * a.sb_row_stride + kit * S::kGroups, lg, gword,
                            row_words - kit * S::kRowWordsPerSlot, K - kit * S::kSpan, sb_narrow);
      }
    }
  };
  auto w_next = [&]() __attribute__((always_inline)) {
    w_kb += D;
    if (w_kb == nit) {
      w_kb = 0;
      w_p += TN;
      if constexpr (kBuf) {
        w_rs = w_rsrc(w_p);
        if constexpr (!SBB) {
          ws_rs = s_rsrc(w_p);
          wb_rs = b_rsrc(w_p);
        }
      }
    }
  };

  // ---- scale/bias stream (SBB): next sub-block to load is slots [s_kb, s_kb + D) of pair s_p
  int64_t s_p = t_begin;
  int s_kb = 0;
  __amdgpu_buffer_rsrc_t s_rs, b_rs;
  if constexpr (SBB) {
    s_rs = s_rsrc(s_p);
    b_rs = b_rsrc(s_p);
  }
  SbRegs<NHB> scA[TN], biA[TN], scB[TN], biB[TN];
  auto issue_sb = [&](SbRegs<NHB>(&sc)[TN], SbRegs<NHB>(&bi)[TN]) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      load_sb_buf<NHB>(sc[t], s_rs, sb_voff[t], s_kb * S::kGroups * 2);
      load_sb_buf<NHB>(bi[t], b_rs, sb_voff[t], s_kb * S::kGroups * 2);
    }
    s_kb += D;
    if (s_kb == nit) {
      s_kb = 0;
      s_p += TN;
      s_rs = s_rsrc(s_p);
      b_rs = b_rsrc(s_p);
    }
  };

  // ---- prologue.  When the activations are staged in one batch, every wave issues its
  // activation loads, the workgroup meets at a barrier, and only then is the weight prefetch
  // issued: the weights are in flight during the staging and the Σx pass, and the activation
  // loads, ahead of them in the queue, are not delayed by them.  (A wave still issuing
  // weight loads would hold up any barrier it has not reached, so none comes between the
  // prefetch and the staging waits.)  Larger activations are staged batch by batch first.
  const uint16_t* xr = stage_row<T, BITS, MROWS>(a, xb, rows, tid, xrl);
  const int nbatch = stage_batches(K, kStreamThreads, xrl);
  auto prefetch = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SBB) issue_sb(scA, biA);
#pragma unroll
    for (int rr = 0; rr < RF; ++rr) {
#pragma unroll
      for (int j = 0; j < D; ++j) issue_w(j, rr * D + j);
      w_next();
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  if (nbatch == 1) {
    // activation loads first, the weight prefetch right behind them (loads return in issue
    // order, so waiting for the activations does not wait for the weights)
    XStage<MROWS> st;
    stage_x_issue<T, BITS, MROWS>(st, xr, 0, K, 0, tid, kStreamThreads, rows, xrl);
    // every wave's activation loads are issued before any weight load enters the queue
    lds_barrier();
    prefetch();
    stage_x_commit<T, BITS, MROWS>(st, xs, rows, K, 0, tid, kStreamThreads, xrl);
    zero_x_pad<BITS>(xs, K, Kp, tid, kStreamThreads, xrl);
    zero_sx_pad(sxs, K / GS, tid, xrl);
    if (do_argmax && tid < MROWS) kl[tid] = 0ull;
    lds_barrier();
    sum_x<T, GS, MT>(xs, sxs, K, wave, kStreamWaves, lane, xrl);
    lds_barrier();
  } else {
    for (int batch = 0; batch < nbatch; ++batch) {
      XStage<MROWS> st;
      stage_x_issue<T, BITS, MROWS>(st, xr, 0, K, batch, tid, kStreamThreads, rows, xrl);
      stage_x_commit<T, BITS, MROWS>(st, xs, rows, K, batch, tid, kStreamThreads, xrl);
    }
    zero_x_pad<BITS>(xs, K, Kp, tid, kStreamThreads, xrl);
    zero_sx_pad(sxs, K / GS, tid, xrl);
    if (do_argmax && tid < MROWS) kl[tid] = 0ull;
    lds_barrier();
    sum_x<T, GS, MT>(xs, sxs, K, wave, kStreamWaves, lane, xrl);
    lds_barrier();
    prefetch();
  }
  // (waves without tiles still take part in the argmax barrier below)
  if (t_end <= t_begin && !do_argmax) return;

  unsigned long long best[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) best[mt][r] = 0ull;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[TN][MT], part[TN][MT];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[t][mt] = zero4;
      part[t][mt] = zero4;
    }

  // ---- consumption: sub-block = D slots of ring part `rbase`, scale/bias set (sc, bi);
  // the next sub-block's scales/biases go to the other set, each consumed slot (or, with
  // the deep ring, the whole sub-block) is refilled right away with the slots R ahead (the
  // scheduling barriers keep the refills there)
  int64_t c_p = t_begin;
  int c_kb = 0;
  auto sub_block = [&](int rbase, const SbRegs<NHB>(&sc)[TN], const SbRegs<NHB>(&bi)[TN],
                       SbRegs<NHB>(&sc_next)[TN], SbRegs<NHB>(&bi_next)[TN]) {
    if constexpr (SBB) issue_sb(sc_next, bi_next);
    SbRegs<S::kGroups> b_first[TN];   // bias halfwords of the first slot of a bias pair
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if constexpr (SBB) {
        consume_slot<T, BITS, GS, MT, TN, NHB, !kPairBias>(ring[rbase + j], sc, bi, j * S::kGroups, xs, sxs,
                                                           (c_kb + j) * S::kSpan, K, acc, part, lg, col, gshift, xrl);
        if (kPairBias && j % 2 == 1) {
          const int g0 = (c_kb + j - 1) * S::kSpan / GS;
          const bool g_ok = (g0 + lg) * GS < K;   // groups past K add nothing
          uint32_t bh[TN];
#pragma unroll
          for (int t = 0; t < TN; ++t)
            bh[t] = g_ok ? bi[t].template lane_half<2 * S::kGroups>((j - 1) * S::kGroups, lg) : 0u;
          bias_mfma<T, MT, TN>(bh, sxs, g0, acc, lg, col, xrl);
        }
      } else {
        SbRegs<S::kGroups> s1[TN], b1[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          s1[t] = ring[rbase + j][t].s;
          b1[t] = ring[rbase + j][t].b;
        }
        consume_slot<T, BITS, GS, MT, TN, S::kGroups, !kPairBias>(ring[rbase + j], s1, b1, 0, xs, sxs,
                                                                  (c_kb + j) * S::kSpan, K, acc, part, lg, col,
                                                                  gshift, xrl);
        if (kPairBias && j % 2 == 0) {
#pragma unroll
          for (int t = 0; t < TN; ++t) b_first[t] = b1[t];
        }
        if (kPairBias && j % 2 == 1) {
          const int g0 = (c_kb + j - 1) * S::kSpan / GS;
          const bool g_ok = (g0 + lg) * GS < K;
          uint32_t bh[TN];
#pragma unroll
          for (int t = 0; t < TN; ++t) bh[t] = g_ok ? pair_lane_half<S::kGroups>(b_first[t], b1[t], lg) : 0u;
          bias_mfma<T, MT, TN>(bh, sxs, g0, acc, lg, col, xrl);
        }
      }
      if constexpr (!kDeepRing) {
        __builtin_amdgcn_sched_barrier(0);
        issue_w(j, rbase + j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (kDeepRing) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < D; ++j) issue_w(j, rbase + j);
      __builtin_amdgcn_sched_barrier(0);
    }
    w_next();
    c_kb += D;
    if (c_kb == nit) {
      if (wb.bad) {
#pragma unroll
        for (int t = 0; t < TN; ++t) poison<MT>(acc[t]);
      }
      if (do_argmax) {
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const int64_t n = (c_p + t) * 16 + col;
          argmax_update<T, MT>(best, acc[t], n, c_p + t < t_end && n < N);
        }
      }
      if (store_y) {
        if (y_vec && c_p + TN <= t_end && (c_p + TN) * 16 <= N) {
          if (y_defer)
            stage_pair_lds<T, MT>(acc, ys_area + (int)((c_p - t_begin) / TN) * kPairHalves, lg, col);
          else
            store_pair_lds<T, MT>(acc, yb, rows, c_p * 16, N, ys_area, lane, lg, col);
        } else {
#pragma unroll
          for (int t = 0; t < TN; ++t)
            if (c_p + t < t_end) store_tile<T, MT>(acc[t], yb, rows, (c_p + t) * 16 + col, N, lg);
        }
      }
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = zero4;
      c_kb = 0;
      c_p += TN;
    }
  };
  const int64_t nsub = (t_end - t_begin + TN - 1) / TN * (nit / D);
  // one loop trip walks the ring once (twice when RF is odd, so the scale/bias sets, which
  // alternate per sub-block, line up again)
  constexpr int UB = RF % 2 == 0 ? RF : 2 * RF;
  for (int64_t i = 0; i < nsub; i += UB) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (u == 0 || i + u < nsub) {
        if (u % 2 == 0)
          sub_block((u % RF) * D, scA, biA, scB, biB);
        else
          sub_block((u % RF) * D, scB, biB, scA, biA);
      }
    }
  }
  if (store_y && y_vec && y_defer) {
    wave_lds_order();
    for (int64_t p = t_begin; p + TN <= t_end && (p + TN) * 16 <= N; p += TN)
      flush_pair_lds<MT>(yb, rows, p * 16, N, ys_area + (int)((p - t_begin) / TN) * kPairHalves, lane);
  }
  if (do_argmax) {
    argmax_merge_wave<MT>(best, kl, lg, col);
    lds_barrier();
    if (tid < rows) argmax_publish(&a.argmax_keys[z * a.rows_per_batch + tid], kl[tid]);
    argmax_complete(a, a.batches * rows, (unsigned*)kl);   // kl is free again after the barrier inside
  }
}

template <class T, int BITS, int GS, int MT, int TN>
__global__ __launch_bounds__(kThreads) void qmv_chunk_kernel(const MatArgs a) {
  using S = Slot<BITS, GS>;
  constexpr int MROWS = 16 * MT;
  constexpr int KC = kChunkXBytes / (MROWS * 2);
  __shared__ u32x4 xs[kChunkXBytes / 16];
  __shared__ float sxs[(KC / 32 + kSxPad) * MROWS];
  __shared__ unsigned long long kl[MROWS];
  constexpr int xrl = MT == 1 ? 4 : 5;   // every row of the tiles staged

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
  const bool sb_narrow = !sb_rows_aligned<S::kGroups>(a);
  uint16_t* yb = (uint16_t*)a.y + z * (int64_t)rows * N;

  int gword = 0;
  uint32_t gshift = 0;
  if constexpr (BITS != 4 && BITS != 8) generic_lane_offsets<BITS>(lg, gword, gshift);

  const WeightBase wb = weight_base(a, z);
  int64_t nrow[TN], nl[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    nrow[t] = ((int64_t)(blockIdx.x * kWaves + wave) * TN + t) * 16 + col;
    nl[t] = nrow[t] < N ? nrow[t] : N - 1;
  }
  auto issue = [&](SlotData<BITS, GS> (&d)[TN], int kit) {
#pragma unroll
    for (int t = 0; t < TN; ++t)
      load_slot<BITS, GS>(d[t], wb.w + nl[t] * a.w_row_stride + (int64_t)kit * S::kRowWordsPerSlot,
                          wb.s + nl[t] * a.sb_row_stride + kit * S::kGroups,
                          wb.b + nl[t] * a.sb_row_stride + kit * S::kGroups, lg, gword,
                          row_words - kit * S::kRowWordsPerSlot, K - kit * S::kSpan, sb_narrow);
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

  const int nit_total = (K + S::kSpan - 1) / S::kSpan;   // the last slot may end past K
  // rows cut into parts (see row_parts): part sums added in part order, as the parts kernel does
  const int n_parts = row_parts<BITS, GS>(K, weight_rows(a));
  const int spp = part_slots<BITS, GS>(K, weight_rows(a));
  bool have_total = false;
  f32x4 total[TN][MT];
  const bool pair_bias = bias_span<GS>(nit_total) == 2;
  SbRegs<S::kGroups> b_first[TN];   // bias halfwords of the first slot of a bias pair
  SlotData<BITS, GS> cur[TN], nxt[TN];
  issue(cur, 0);
  for (int kc0 = 0; kc0 < K; kc0 += KC) {
    const int kcl = min(KC, K - kc0);
    lds_barrier();
    const int kclp = (kcl + S::kSpan - 1) / S::kSpan * S::kSpan;
    stage_x<T, BITS, MROWS>(xs, a, xb, rows, kc0, kcl, tid, kThreads, xrl);
    zero_x_pad<BITS>(xs, kcl, kclp, tid, kThreads, xrl);
    zero_sx_pad(sxs, kcl / GS, tid, xrl);
    lds_barrier();
    sum_x<T, GS, MT>(xs, sxs, kcl, wave, kWaves, lane, xrl);
    lds_barrier();
    const int kit0 = kc0 / S::kSpan;
    const int nit = kclp / S::kSpan;
    for (int i = 0; i < nit; ++i) {
      const int kit = kit0 + i;
      issue(nxt, min(kit + 1, nit_total - 1));
      {
        SbRegs<S::kGroups> sc[TN], bi[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          sc[t] = cur[t].s;
          bi[t] = cur[t].b;
        }
        if (!pair_bias) {
          consume_slot<T, BITS, GS, MT, TN, S::kGroups>(cur, sc, bi, 0, xs, sxs, i * S::kSpan, kcl, acc, part, lg,
                                                        col, gshift, xrl);
        } else {
          consume_slot<T, BITS, GS, MT, TN, S::kGroups, false>(cur, sc, bi, 0, xs, sxs, i * S::kSpan, kcl, acc, part,
                                                               lg, col, gshift, xrl);
          if (kit % 2 == 0) {
#pragma unroll
            for (int t = 0; t < TN; ++t) b_first[t] = bi[t];
          } else {
            // chunks hold a whole number of slot pairs, so the pair's first slot is in this chunk
            const int g0 = (i - 1) * S::kSpan / GS;
            const bool g_ok = (g0 + lg) * GS < kcl;
            uint32_t bh[TN];
#pragma unroll
            for (int t = 0; t < TN; ++t) bh[t] = g_ok ? pair_lane_half<S::kGroups>(b_first[t], bi[t], lg) : 0u;
            bias_mfma<T, MT, TN>(bh, sxs, g0, acc, lg, col, xrl);
          }
        }
      }
      if (n_parts > 1 && (kit + 1) % spp == 0) {
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            total[t][mt] = have_total ? total[t][mt] + acc[t][mt] : acc[t][mt];
            acc[t][mt] = zero4;
          }
        have_total = true;
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) cur[t] = nxt[t];
    }
  }
  if (n_parts > 1) {
    // the last part ends past the row's slots when they are not a whole number of parts
    const bool open_part = nit_total % spp != 0;
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = open_part ? total[t][mt] + acc[t][mt] : total[t][mt];
  }
  if (wb.bad) {
#pragma unroll
    for (int t = 0; t < TN; ++t) poison<MT>(acc[t]);
  }
  if (a.y) {
#pragma unroll
    for (int t = 0; t < TN; ++t) store_tile<T, MT>(acc[t], yb, rows, nrow[t], N, lg);
  }
  if (a.argmax_keys) {
    unsigned long long best[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) best[mt][r] = 0ull;
#pragma unroll
    for (int t = 0; t < TN; ++t) argmax_update<T, MT>(best, acc[t], nrow[t], nrow[t] < N);
    if (tid < MROWS) kl[tid] = 0ull;
    lds_barrier();
    argmax_merge_wave<MT>(best, kl, lg, col);
    lds_barrier();
    if (tid < rows) argmax_publish(&a.argmax_keys[z * rows + tid], kl[tid]);
    argmax_complete(a, a.batches * rows, (unsigned*)kl);   // kl is free again after the barrier inside
  }
}

}  // namespace decode
}  // namespace qmm

#include "decode_parts.hpp"

namespace qmm {
namespace decode {

// ----------------------------------------------------------------------------- launchers
int device_cus();
hipError_t kernel_wgs_per_cu(const void* kern, int threads, int lds, int lds_max, int* out);

template <class T, int BITS, int GS, int MT, int D, bool SBB, int XRL>
hipError_t launch_stream_sb(const MatArgs& a, hipStream_t stream, int lds) {
  auto kern = qmv_stream_kernel<T, BITS, GS, MT, D, SBB, XRL>;
  int per_cu = 1;
  const hipError_t occ = kernel_wgs_per_cu((const void*)kern, kStreamThreads, lds, kLdsLimit, &per_cu);
  if (occ != hipSuccess) return occ;
  // one full wave of workgroups (every CU at its occupancy), tile pairs spread over all waves
  const int64_t n_pairs = ((a.N + 15) / 16 + kPair - 1) / kPair;
  const int64_t full = (int64_t)device_cus() * std::min(per_cu, kMaxWgPerCu);
  const int64_t blocks = std::min<int64_t>(full, (n_pairs + kStreamWaves - 1) / kStreamWaves);
  const int64_t waves_total = blocks * kStreamWaves;
  if (n_pairs / waves_total > 0x7FFFFFFF) return hipErrorInvalidValue;
  // The output staging area, when the LDS has room for it at the same occupancy: every pair
  // of a wave's range (stores after the weight stream), else one pair at a time.
  int y_area = 0;
  if (a.y != nullptr) {
    const int64_t max_pairs = n_pairs / waves_total + (n_pairs % waves_total != 0 ? 1 : 0);
    const int64_t tries[2] = {max_pairs > 1 ? max_pairs : 0, 1};
    for (const int64_t yp : tries) {
      if (yp < 1 || yp > 64) continue;
      const int lds_y = lds + y_area_bytes<MT>(kStreamWaves, (int)yp);
      if (lds_y > kLdsLimit) continue;
      int per_cu_y = 0;
      const hipError_t e = kernel_wgs_per_cu((const void*)kern, kStreamThreads, lds_y, kLdsLimit, &per_cu_y);
      if (e != hipSuccess) return e;
      if (std::min(per_cu_y, kMaxWgPerCu) == std::min(per_cu, kMaxWgPerCu)) {
        y_area = (int)yp;
        lds = lds_y;
        break;
      }
    }
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks, 1, (unsigned)a.batches), dim3(kStreamThreads), lds, stream, a,
                     (int)(n_pairs / waves_total), (int)(n_pairs % waves_total), y_area);
  return hipGetLastError();
}

// Scales/biases per sub-block when their rows and bases are aligned to the load width.
template <class T, int BITS, int GS, int MT, int D, int XRL>
hipError_t launch_stream_d(const MatArgs& a, hipStream_t stream, int lds) {
  if constexpr (BITS == 4 || BITS == 8) {
    constexpr int bytes = D * Slot<BITS, GS>::kGroups * 2;
    constexpr int align = bytes < 16 ? bytes : 16;
    if ((a.sb_row_stride * 2) % align == 0 && (a.sb_expert_stride * 2) % align == 0 &&
        (uintptr_t)a.scales % align == 0 && (uintptr_t)a.biases % align == 0)
      return launch_stream_sb<T, BITS, GS, MT, D, true, XRL>(a, stream, lds);
  }
  return launch_stream_sb<T, BITS, GS, MT, D, false, XRL>(a, stream, lds);
}

// Slots per main-loop block (block_slots): 2 when the slots per tile are even, else 1.
template <class T, int BITS, int GS, int MT, int XRL>
hipError_t launch_stream(const MatArgs& a, hipStream_t stream, int lds) {
  const int nit = (int)((a.K + Slot<BITS, GS>::kSpan - 1) / Slot<BITS, GS>::kSpan);
  if (block_slots(nit) == 2) return launch_stream_d<T, BITS, GS, MT, 2, XRL>(a, stream, lds);
  return launch_stream_d<T, BITS, GS, MT, 1, XRL>(a, stream, lds);
}

template <class T, int BITS, int GS, int MT, int D, bool SBB, int XRL>
hipError_t launch_parts_sb(const MatArgs& a, hipStream_t stream, int lds, int P, int spp) {
  auto kern = qmv_parts_kernel<T, BITS, GS, MT, D, SBB, XRL>;
  int per_cu = 1;
  const hipError_t occ = kernel_wgs_per_cu((const void*)kern, kStreamThreads, lds, kLdsLimit, &per_cu);
  if (occ != hipSuccess) return occ;
  const int64_t n_pairs = ((a.N + 15) / 16 + kPair - 1) / kPair;
  const int64_t groups = kStreamWaves / P;
  const int64_t full = (int64_t)device_cus() * std::min(per_cu, kMaxWgPerCu);
  const int64_t blocks = std::min<int64_t>(full, (n_pairs + groups - 1) / groups);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks, 1, (unsigned)a.batches), dim3(kStreamThreads), lds, stream, a, P,
                     spp);
  return hipGetLastError();
}

template <class T, int BITS, int GS, int MT, int XRL>
hipError_t launch_parts(const MatArgs& a, hipStream_t stream, int lds) {
  const int P = row_parts<BITS, GS>(a.K, weight_rows(a));
  const int spp = part_slots<BITS, GS>(a.K, weight_rows(a));
  const int nit = (int)((a.K + Slot<BITS, GS>::kSpan - 1) / Slot<BITS, GS>::kSpan);
  if (block_slots(nit) == 2) {
    if constexpr (BITS == 4 || BITS == 8) {
      constexpr int bytes = 2 * Slot<BITS, GS>::kGroups * 2;
      constexpr int align = bytes < 16 ? bytes : 16;
      if ((a.sb_row_stride * 2) % align == 0 && (a.sb_expert_stride * 2) % align == 0 &&
          (uintptr_t)a.scales % align == 0 && (uintptr_t)a.biases % align == 0)
        return launch_parts_sb<T, BITS, GS, MT, 2, true, XRL>(a, stream, lds, P, spp);
    }
    return launch_parts_sb<T, BITS, GS, MT, 2, false, XRL>(a, stream, lds, P, spp);
  }
  if constexpr (BITS == 4 || BITS == 8) {
    constexpr int bytes = Slot<BITS, GS>::kGroups * 2;
    constexpr int align = bytes < 16 ? bytes : 16;
    if ((a.sb_row_stride * 2) % align == 0 && (a.sb_expert_stride * 2) % align == 0 &&
        (uintptr_t)a.scales % align == 0 && (uintptr_t)a.biases % align == 0)
      return launch_parts_sb<T, BITS, GS, MT, 1, true, XRL>(a, stream, lds, P, spp);
  }
  return launch_parts_sb<T, BITS, GS, MT, 1, false, XRL>(a, stream, lds, P, spp);
}

template <class T, int BITS, int GS, int MT>
hipError_t launch_chunk(const MatArgs& a, hipStream_t stream) {
  const int64_t rows_per_wg = (int64_t)kWaves * kChunkTiles * 16;
  dim3 grid((unsigned)((a.N + rows_per_wg - 1) / rows_per_wg), 1, (unsigned)a.batches);
  hipLaunchKernelGGL((qmv_chunk_kernel<T, BITS, GS, MT, kChunkTiles>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int BITS, int MT, int GS>
constexpr int stream_lds_bytes(int K, int xrl) {
  const int Kp = (K + Slot<BITS, GS>::kSpan - 1) / Slot<BITS, GS>::kSpan * Slot<BITS, GS>::kSpan;
  return ((Kp * 2) << xrl) + sx_floats(K / GS, xrl) * 4 + 16 * MT * 8;
}

template <class T, int BITS, int GS>
hipError_t launch_gs(const MatArgs& a, hipStream_t stream) {
  const int K = (int)a.K;
  // long rows (see row_parts) run the parts kernel, the others the streaming kernel
  const bool parts = row_parts<BITS, GS>(K, weight_rows(a)) > 1;
  // Activation rows the one-tile kernels stage in LDS (x_lds_rows_log2): one row alone, all
  // 16 rows of the tile, or 8 rows for 2-8 rows whose 16-row staging does not fit
  auto lds_at = [&](int xl) {
    return parts ? parts_lds_bytes<1, GS, BITS>(K, xl) : stream_lds_bytes<BITS, 1, GS>(K, xl);
  };
  auto xl_one = [&](int64_t rows) {
    const int xl = x_lds_rows_log2<1>((int)(rows < 16 ? rows : 16));
    return xl == 4 && rows <= 8 && lds_at(4) > kLdsLimit ? 3 : xl;
  };
  const int lds1 = lds_at(xl_one(a.rows_per_batch));
  const int lds2 = parts ? parts_lds_bytes<2, GS, BITS>(K, 5) : stream_lds_bytes<BITS, 2, GS>(K, 5);
  auto run1 = [&](const MatArgs& m) {
    const int xl = xl_one(m.rows_per_batch);
    const int lds = lds_at(xl);
    if (xl == 0)
      return parts ? launch_parts<T, BITS, GS, 1, 0>(m, stream, lds) : launch_stream<T, BITS, GS, 1, 0>(m, stream, lds);
    if (xl == 3)
      return parts ? launch_parts<T, BITS, GS, 1, 3>(m, stream, lds) : launch_stream<T, BITS, GS, 1, 3>(m, stream, lds);
    return parts ? launch_parts<T, BITS, GS, 1, 4>(m, stream, lds) : launch_stream<T, BITS, GS, 1, 4>(m, stream, lds);
  };
  if (a.rows_per_batch <= 16) return lds1 <= kLdsLimit ? run1(a) : launch_chunk<T, BITS, GS, 1>(a, stream);
  if (lds2 <= kLdsLimit)
    return parts ? launch_parts<T, BITS, GS, 2, 5>(a, stream, lds2) : launch_stream<T, BITS, GS, 2, 5>(a, stream, lds2);
  // 17..32 rows whose activations do not fit in LDS at once: when 16 activation rows do,
  // run the one-block kernel on rows 0..15 and on the rest, which keeps every row's
  // arithmetic that of a call of at most 16 rows.  The second block needs the rows to
  // continue one 16-row block further at a fixed offset: one segment, or segments that are
  // whole 16-row blocks; one grid slice.  Both blocks go in one launch, as two grid slices
  // (the second with last_rows rows), so their workgroups run side by side; with a fused
  // argmax (whose completion counts one launch's rows) they run one after the other.
  const int64_t rows = a.rows_per_batch;
  const bool one_seg = a.seg_rows >= rows;
  if (lds1 <= kLdsLimit && a.batches == 1 && (one_seg || a.seg_rows % 16 == 0)) {
    const int64_t x_off = one_seg ? 16 * a.row_stride : (16 / a.seg_rows) * a.seg_stride + (16 % a.seg_rows) * a.row_stride;
    if (a.argmax_keys == nullptr && a.w_index == nullptr) {
      MatArgs two = a;
      two.batches = 2;
      two.batch_stride = x_off;
      two.rows_per_batch = 16;
      two.last_rows = rows - 16;
      if (one_seg) two.seg_rows = 16;
      return run1(two);
    }
    MatArgs lo = a, hi = a;
    lo.rows_per_batch = 16;
    hi.rows_per_batch = rows - 16;
    hi.x = (const uint16_t*)a.x + x_off;
    if (one_seg) {
      lo.seg_rows = 16;
      hi.seg_rows = rows - 16;
    }
    if (a.y) hi.y = (uint16_t*)a.y + 16 * a.N;
    if (a.argmax_keys) {
      hi.argmax_keys = a.argmax_keys + 16;
      hi.argmax_index = a.argmax_index + 16;
      if (a.argmax_value) hi.argmax_value = a.argmax_value + 16;
    }
    hipError_t e = run1(lo);
    if (e != hipSuccess) return e;
    return run1(hi);
  }
  return launch_chunk<T, BITS, GS, 2>(a, stream);
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
