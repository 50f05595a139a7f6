// Decode kernel for long rows: every pair of 16-row weight tiles is cut along K into P equal
// parts, worked on by P waves at once, so that matrices with few rows and long K still give
// every CU several streams of weights.  Included by decode_kernels.hpp.
#pragma once

namespace qmm {
namespace decode {

template <class T, int BITS, int GS, int MT, int D, bool SBB, int XRL>
__global__ __launch_bounds__(kStreamThreads, kStreamWavesPerSimd) void qmv_parts_kernel(const MatArgs a, const int P,
                                                                                    const int spp) {
  // The workgroup's waves form G = 8/P groups of P waves.  Round r: group g works on tile
  // pair wg_p0 + r*G + g of the workgroup's pair range, wave j of the group on slots
  // [j*spp, (j+1)*spp) of it (slots past the row's last are skipped).  Each wave's slots
  // over all rounds form one stream with the ring of the streaming kernel.  At a round's end
  // the parts meet in LDS and the group's wave 0 adds them in part order, then stores.
  using S = Slot<BITS, GS>;
  constexpr int MROWS = 16 * MT;
  constexpr int TN = kPair;
  constexpr int RF = kRingFactor;
  constexpr int R = RF * D;
  constexpr bool kPairBias = GS >= 64 && D >= 2;
  constexpr bool kBuf = BITS == 4 || BITS == 8;
  static_assert(!SBB || kBuf, "block scale/bias loads use the buffer path");
  constexpr int NHB = D * S::kGroups;
  extern __shared__ u32x4 smem[];
  const int K = (int)a.K;
  const int Kp = (K + S::kSpan - 1) / S::kSpan * S::kSpan;
  constexpr int xrl = XRL;   // 2^xrl activation rows in LDS (x_lds_rows_log2)
  u32x4* xs = smem;
  float* sxs = (float*)(smem + (((Kp / 32) * 4) << xrl));
  unsigned long long* kl = (unsigned long long*)(sxs + sx_floats(K / GS, xrl));
  f32x4* hs = (f32x4*)(kl + MROWS);   // part sums handed to the group's wave 0

  const int tid = threadIdx.x;
  const int lane = tid & 63;
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

  const int G = kStreamWaves / P;
  const int grp = wave / P, part = wave - grp * P;
  const int64_t n_tiles = (N + 15) >> 4;
  const int64_t n_pairs = (n_tiles + TN - 1) / TN;
  const int64_t wg_base = n_pairs / gridDim.x, wg_rem = n_pairs % gridDim.x;
  const int64_t wg_p0 = (int64_t)blockIdx.x * wg_base + min((int64_t)blockIdx.x, wg_rem);
  const int64_t wg_pend = wg_p0 + wg_base + ((int64_t)blockIdx.x < wg_rem ? 1 : 0);
  const int64_t rounds = (wg_pend - wg_p0 + G - 1) / G;
  const int nit = Kp / S::kSpan;          // the row's real slots
  const int kb0 = part * spp;             // the part's first slot
  const int sbs = spp / D;                // sub-blocks per round
  const int64_t nsub = rounds * sbs;
  const int row_words = (K * BITS) >> 5;
  const bool do_argmax = a.argmax_keys != nullptr;
  const bool store_y = a.y != nullptr;

  int gword = 0;
  uint32_t gshift = 0;
  if constexpr (!kBuf) generic_lane_offsets<BITS>(lg, gword, gshift);

  // descriptors over the rows of the tile pair starting at tile p (empty past the
  // workgroup's pairs, so the ring's loads past the last round read nothing)
  auto rows_valid = [&](int64_t p) -> uint32_t {
    if (p / TN >= wg_pend) return 0u;
    const int64_t valid = N - p * 16 < 16 * TN ? N - p * 16 : 16 * TN;
    return (uint32_t)valid;
  };
  const WeightBase wb = weight_base(a, z);
  auto w_rsrc = [&](int64_t p) { return make_rsrc(wb.w + p * 16 * a.w_row_stride, rows_valid(p) * w_row_bytes); };
  auto s_rsrc = [&](int64_t p) { return make_rsrc(wb.s + p * 16 * a.sb_row_stride, rows_valid(p) * sb_row_bytes); };
  auto b_rsrc = [&](int64_t p) { return make_rsrc(wb.b + p * 16 * a.sb_row_stride, rows_valid(p) * sb_row_bytes); };
  auto tile_of_round = [&](int64_t r) { return (wg_p0 + r * G + grp) * TN; };

  // ---- weight stream: round w_r, sub-block w_s of the part
  int64_t w_r = 0;
  int w_s = 0;
  int64_t w_p = tile_of_round(0);
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
    const int kit = kb0 + w_s * D + j;
    if (kit >= nit || w_r >= rounds) return;   // past the row's slots or the wave's rounds
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
    if (++w_s == sbs) {
      w_s = 0;
      ++w_r;
      w_p = tile_of_round(w_r);
      if constexpr (kBuf) {
        w_rs = w_rsrc(w_p);
        if constexpr (!SBB) {
          ws_rs = s_rsrc(w_p);
          wb_rs = b_rsrc(w_p);
        }
      }
    }
  };

  // ---- scale/bias stream (SBB), one sub-block ahead of consumption
  int64_t s_r = 0;
  int s_s = 0;
  __amdgpu_buffer_rsrc_t s_rs, b_rs;
  if constexpr (SBB) {
    s_rs = s_rsrc(tile_of_round(0));
    b_rs = b_rsrc(tile_of_round(0));
  }
  SbRegs<NHB> scA[TN], biA[TN], scB[TN], biB[TN];
  auto issue_sb = [&](SbRegs<NHB>(&sc)[TN], SbRegs<NHB>(&bi)[TN]) {
    const int kit = kb0 + s_s * D;
    if (kit < nit && s_r < rounds) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        load_sb_buf<NHB>(sc[t], s_rs, sb_voff[t], kit * S::kGroups * 2);
        load_sb_buf<NHB>(bi[t], b_rs, sb_voff[t], kit * S::kGroups * 2);
      }
    }
    if (++s_s == sbs) {
      s_s = 0;
      ++s_r;
      s_rs = s_rsrc(tile_of_round(s_r));
      b_rs = b_rsrc(tile_of_round(s_r));
    }
  };

  // ---- prologue: activation loads, barrier, weight prefetch, staging waits, sums
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
    XStage<MROWS> st;
    stage_x_issue<T, BITS, MROWS>(st, xr, 0, K, 0, tid, kStreamThreads, rows, xrl);
    lds_barrier();
    prefetch();
    stage_x_commit<T, BITS, MROWS>(st, xs, rows, K, 0, tid, kStreamThreads, xrl);
  } else {
    for (int batch = 0; batch < nbatch; ++batch) {
      XStage<MROWS> st;
      stage_x_issue<T, BITS, MROWS>(st, xr, 0, K, batch, tid, kStreamThreads, rows, xrl);
      stage_x_commit<T, BITS, MROWS>(st, xs, rows, K, batch, tid, kStreamThreads, xrl);
    }
  }
  zero_x_pad<BITS>(xs, K, Kp, tid, kStreamThreads, xrl);
  zero_sx_pad(sxs, K / GS, tid, xrl);
  if (do_argmax && tid < MROWS) kl[tid] = 0ull;
  lds_barrier();
  sum_x<T, GS, MT>(xs, sxs, K, wave, kStreamWaves, lane, xrl);
  lds_barrier();
  if (nbatch != 1) prefetch();

  unsigned long long best[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) best[mt][r] = 0ull;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[TN][MT], partial[TN][MT];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[t][mt] = zero4;
      partial[t][mt] = zero4;
    }

  auto finish_pair = [&](int64_t cp) {
    if (wb.bad) {
#pragma unroll
      for (int t = 0; t < TN; ++t) poison<MT>(acc[t]);
    }
    if (do_argmax) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int64_t n = (cp + t) * 16 + col;
        argmax_update<T, MT>(best, acc[t], n, n < N);
      }
    }
    if (store_y) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
        if (cp + t < n_tiles) store_tile<T, MT>(acc[t], yb, rows, (cp + t) * 16 + col, N, lg);
    }
  };

  // ---- consumption
  int64_t c_r = 0;
  int c_s = 0;
  auto sub_block = [&](int rbase, const SbRegs<NHB>(&sc)[TN], const SbRegs<NHB>(&bi)[TN],
                       SbRegs<NHB>(&sc_next)[TN], SbRegs<NHB>(&bi_next)[TN]) {
    if constexpr (SBB) issue_sb(sc_next, bi_next);
    const int kit0 = kb0 + c_s * D;
    const bool real = kit0 < nit;   // with D = 2 the row's slots are even: both real or both not
    SbRegs<S::kGroups> b_first[TN];
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (real) {
        if constexpr (SBB) {
          consume_slot<T, BITS, GS, MT, TN, NHB, !kPairBias>(ring[rbase + j], sc, bi, j * S::kGroups, xs, sxs,
                                                             (kit0 + j) * S::kSpan, K, acc, partial, lg, col, gshift, xrl);
          if (kPairBias && j % 2 == 1) {
            const int g0 = (kit0 + j - 1) * S::kSpan / GS;
            const bool g_ok = (g0 + lg) * GS < K;
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
                                                                    (kit0 + j) * S::kSpan, K, acc, partial, lg,
                                                                    col, gshift, xrl);
          if (kPairBias && j % 2 == 0) {
#pragma unroll
            for (int t = 0; t < TN; ++t) b_first[t] = b1[t];
          }
          if (kPairBias && j % 2 == 1) {
            const int g0 = (kit0 + j - 1) * S::kSpan / GS;
            const bool g_ok = (g0 + lg) * GS < K;
            uint32_t bh[TN];
#pragma unroll
            for (int t = 0; t < TN; ++t) bh[t] = g_ok ? pair_lane_half<S::kGroups>(b_first[t], b1[t], lg) : 0u;
            bias_mfma<T, MT, TN>(bh, sxs, g0, acc, lg, col, xrl);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      issue_w(j, rbase + j);
      __builtin_amdgcn_sched_barrier(0);
    }
    w_next();
    if (++c_s == sbs) {
      // round end: parts 1.. hand their sums over, wave 0 of the group adds them in order
      if (part != 0) {
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) hs[((wave * TN + t) * MT + mt) * 64 + lane] = acc[t][mt];
      }
      lds_barrier();
      if (part == 0) {
        for (int jj = 1; jj < P; ++jj) {
#pragma unroll
          for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[t][mt] = acc[t][mt] + hs[(((wave + jj) * TN + t) * MT + mt) * 64 + lane];
        }
        const int64_t cp = tile_of_round(c_r);
        if (cp / TN < wg_pend) finish_pair(cp);
      }
      lds_barrier();
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = zero4;
      c_s = 0;
      ++c_r;
    }
  };
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
  if (do_argmax) {
    argmax_merge_wave<MT>(best, kl, lg, col);
    lds_barrier();
    if (tid < rows) argmax_publish(&a.argmax_keys[z * a.rows_per_batch + tid], kl[tid]);
    argmax_complete(a, a.batches * rows, (unsigned*)kl);
  }
}

template <int MT, int GS, int BITS>
constexpr int parts_lds_bytes(int K, int xrl) {
  const int Kp = (K + Slot<BITS, GS>::kSpan - 1) / Slot<BITS, GS>::kSpan * Slot<BITS, GS>::kSpan;
  return ((Kp * 2) << xrl) + sx_floats(K / GS, xrl) * 4 + 16 * MT * 8 + kStreamWaves * kPair * MT * 64 * 16;
}

}  // namespace decode
}  // namespace qmm
