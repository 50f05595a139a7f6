// Decode family: y = x . dequant(W)^T for up to 32 activation rows (qmv, batched decode).
//
// Per output element the kernel computes the factored affine form
//     y[m,n] = sum_g ( s[n,g] * sum_{k in g} x[m,k] q[n,k]  +  b[n,g] * sum_{k in g} x[m,k] )
// (MLX pull request 4516, first commit: the bias term multiplies a sum of the inputs, and
// every input is widened to float before it is added).  The inner sums over a group run on
// the matrix cores with the codes as exact bf16/fp16 integers, so sum x*q is exact whenever
// its partial sums are; the two scale terms are applied with float32 FMAs per group, in
// group order.  Nothing in a row's arithmetic depends on the other rows of the call, which
// makes batched results bitwise equal to single-row results (transformers issue 47331,
// "Fix"/"Expected behavior": every batch row must match the batch-1 output).
//
// Work split (gfx950, wave64):
//   * a workgroup is 4 waves; each wave owns TN tiles of 16 weight rows;
//   * the activation rows (padded to 16*MT with zeros) and their per-group sums are staged
//     in LDS once per K chunk and shared by the 4 waves;
//   * each lane streams 16-byte packed-weight loads (4-bit: 128 codes of a row per 4 lanes),
//     a cross-lane transpose (permlane16/32 swaps) turns them into MFMA operand order;
//   * rows of the last tile beyond N load row N-1 and skip their store, so the K loop has
//     no per-row checks (MLX pull request 4516: affine_qmv_fast_rows, partial last tile).
#include "device_common.hpp"
#include "kernels.hpp"

namespace qmm {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXLdsBytes = 65536;  // activation chunk staged in LDS

// v_permlane32_swap: the upper 32 lanes of the first operand trade places with the lower
// 32 lanes of the second.  v_permlane16_swap: odd 16-lane rows of the first operand trade
// places with even rows of the second.
__device__ inline u32x4 swap_halves(u32x4 u) {
  auto r0 = __builtin_amdgcn_permlane32_swap(u.x, u.z, false, false);
  auto r1 = __builtin_amdgcn_permlane32_swap(u.y, u.w, false, false);
  u32x4 o = {r0[0], r1[0], r0[1], r1[1]};
  return o;
}
// Lane group g holds words (4g .. 4g+3) of a 16-word slice; afterwards register c of lane
// group g holds word 4c + g (a 4x4 transpose across lane groups).
__device__ inline u32x4 transpose_lane_groups(u32x4 u) {
  u = swap_halves(u);
  auto r0 = __builtin_amdgcn_permlane16_swap(u.x, u.y, false, false);
  auto r1 = __builtin_amdgcn_permlane16_swap(u.z, u.w, false, false);
  u32x4 o = {r0[0], r0[1], r1[0], r1[1]};
  return o;
}

// Lane group (16 lanes) that feeds sub-block `sub` (8 consecutive k) of a 32-k MFMA step.
// 4-bit and generic widths use the natural order; 8-bit words arrive pre-shuffled by the
// half-wave swap below, which places sub-blocks 1 and 2 on lane groups 2 and 1.
template <int BITS>
__device__ inline int lane_group_of_sub(int sub) {
  if (BITS == 8) return sub == 1 ? 2 : (sub == 2 ? 1 : sub);
  return sub;
}

template <int BITS>
struct WeightStep {
  // 32-k MFMA steps covered by one packed-weight load
  static constexpr int kSteps = (BITS == 4) ? 4 : (BITS == 8) ? 2 : 1;
};

template <class T, int BITS, int MT, int TN>
__global__ __launch_bounds__(kThreads) void qmv_decode_kernel(const MatArgs a) {
  constexpr int MROWS = 16 * MT;
  constexpr int KC = kXLdsBytes / (MROWS * 2);     // k per LDS chunk
  constexpr int STEPS = WeightStep<BITS>::kSteps;
  constexpr int IT_K = 32 * STEPS;
  __shared__ u32x4 xs[kXLdsBytes / 16];
  __shared__ float sxs[(KC / 32) * MROWS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lg = lane >> 4;   // lane group: k sub-block inside an MFMA step
  const int col = lane & 15;  // weight row inside a 16-row tile
  const int64_t z = blockIdx.z;
  const uint16_t* xb = (const uint16_t*)a.x + z * a.batch_stride;
  const int rows = (int)a.rows_per_batch;
  const int64_t N = a.N;
  const int K = (int)a.K;
  const int gs = a.group_size;
  const int64_t seg_rows = a.seg_rows;

  const uint32_t* wrow[TN];
  const uint16_t* srow[TN];
  const uint16_t* brow[TN];
  int64_t nrow[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int64_t n = ((int64_t)(blockIdx.x * kWaves + wave) * TN + t) * 16 + col;
    const int64_t nl = n < N ? n : N - 1;
    nrow[t] = n;
    wrow[t] = a.w + nl * a.w_row_stride;
    srow[t] = (const uint16_t*)a.scales + nl * a.sb_row_stride;
    brow[t] = (const uint16_t*)a.biases + nl * a.sb_row_stride;
  }

  f32x4 acc[MT][TN];
  f32x4 part[MT][TN];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      acc[mt][t] = zero4;
      part[mt][t] = zero4;
    }

  for (int kc0 = 0; kc0 < K; kc0 += KC) {
    const int kcl = min(KC, K - kc0);
    __syncthreads();
    // ---- stage activations (row m, 8 consecutive k per thread) in MFMA operand order
    const int c8 = kcl >> 3;
    for (int i = tid; i < MROWS * c8; i += kThreads) {
      const int m = i / c8;
      const int j8 = i - m * c8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m < rows) {
        const uint16_t* xr = xb + (m / seg_rows) * a.seg_stride + (m % seg_rows) * a.row_stride;
        v = *(const u32x4*)(xr + kc0 + 8 * j8);
      }
      if (BITS == 4) v = interleave_even_odd(v);
      const int c = j8 >> 2;
      xs[(c * 4 + lane_group_of_sub<BITS>(j8 & 3)) * MROWS + m] = v;
    }
    // ---- per (row, group) sums of x: each element widened to float, added in k order
    const int ngc = kcl / gs;
    for (int i = tid; i < MROWS * ngc; i += kThreads) {
      const int m = i / ngc;
      const int gl = i - m * ngc;
      float sum = 0.f;
      if (m < rows) {
        const uint16_t* xr = xb + (m / seg_rows) * a.seg_stride + (m % seg_rows) * a.row_stride +
                             kc0 + gl * gs;
        for (int k = 0; k < gs; k += 8) {
          const u32x4 v = *(const u32x4*)(xr + k);
          sum += T::to_f32(v.x & 0xFFFFu);
          sum += T::to_f32(v.x >> 16);
          sum += T::to_f32(v.y & 0xFFFFu);
          sum += T::to_f32(v.y >> 16);
          sum += T::to_f32(v.z & 0xFFFFu);
          sum += T::to_f32(v.z >> 16);
          sum += T::to_f32(v.w & 0xFFFFu);
          sum += T::to_f32(v.w >> 16);
        }
      }
      sxs[gl * MROWS + m] = sum;
    }
    __syncthreads();

    // ---- stream the packed weights of this chunk
    const int nit = kcl / IT_K;
    u32x4 cur[TN], nxt[TN];
    uint32_t sbc[TN][STEPS], sbn[TN][STEPS];  // (scale | bias << 16) of groups ending per step

    auto load = [&](u32x4 (&dst)[TN], uint32_t (&sb)[TN][STEPS], int k0) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        if (BITS == 4) {
          dst[t] = *(const u32x4*)(wrow[t] + (k0 >> 3) + 4 * lg);
        } else if (BITS == 8) {
          dst[t] = *(const u32x4*)(wrow[t] + (k0 >> 2) + 4 * lg);
        } else {
          const int row_words = (K * BITS) >> 5;
          const int bit0 = (k0 + 8 * lg) * BITS;
          const int idx = bit0 >> 5;
          dst[t].x = wrow[t][idx];
          dst[t].y = wrow[t][min(idx + 1, row_words - 1)];
          dst[t].z = (uint32_t)(bit0 & 31);
          dst[t].w = 0u;
        }
#pragma unroll
        for (int c = 0; c < STEPS; ++c) {
          const int kend = k0 + 32 * c + 32;
          if (kend % gs == 0) {
            const int gabs = kend / gs - 1;
            sb[t][c] = (uint32_t)srow[t][gabs] | ((uint32_t)brow[t][gabs] << 16);
          } else {
            sb[t][c] = 0u;
          }
        }
      }
    };

    load(cur, sbc, kc0);
    for (int it = 0; it < nit; ++it) {
      const int k0 = kc0 + it * IT_K;
      if (it + 1 < nit) load(nxt, sbn, k0 + IT_K);

      // operand order: transpose 16-byte loads across lane groups
      if (BITS == 4) {
#pragma unroll
        for (int t = 0; t < TN; ++t) cur[t] = transpose_lane_groups(cur[t]);
      } else if (BITS == 8) {
#pragma unroll
        for (int t = 0; t < TN; ++t) cur[t] = swap_halves(cur[t]);
      }

#pragma unroll
      for (int c = 0; c < STEPS; ++c) {
        const int kabs = k0 + 32 * c;
        const bool gstart = (kabs % gs) == 0;
        const int sc = (kabs - kc0) >> 5;
        u32x4 bq[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          if (BITS == 4) {
            const uint32_t word = c == 0 ? cur[t].x : c == 1 ? cur[t].y : c == 2 ? cur[t].z : cur[t].w;
            bq[t] = codes4_to_v8<T>(word);
          } else if (BITS == 8) {
            bq[t] = c == 0 ? codes8_to_v8<T>(cur[t].x, cur[t].y) : codes8_to_v8<T>(cur[t].z, cur[t].w);
          } else {
            bq[t] = codesN_to_v8<T, BITS>(cur[t].x, cur[t].y, cur[t].z);
          }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const typename T::v8 av = as_v8<T>(xs[(sc * 4 + lg) * MROWS + mt * 16 + col]);
#pragma unroll
          for (int t = 0; t < TN; ++t)
            part[mt][t] = T::mfma(av, as_v8<T>(bq[t]), gstart ? zero4 : part[mt][t]);
        }
        if (((kabs + 32) % gs) == 0) {
          const int gl = (kabs - kc0) / gs;
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const float sv = T::to_f32(sbc[t][c] & 0xFFFFu);
            const float bv = T::to_f32(sbc[t][c] >> 16);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const f32x4 sx = *(const f32x4*)&sxs[gl * MROWS + mt * 16 + 4 * lg];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                acc[mt][t][r] = __builtin_fmaf(sv, part[mt][t][r], acc[mt][t][r]);
                acc[mt][t][r] = __builtin_fmaf(bv, sx[r], acc[mt][t][r]);
              }
            }
          }
        }
      }
      if (it + 1 < nit) {
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          cur[t] = nxt[t];
#pragma unroll
          for (int c = 0; c < STEPS; ++c) sbc[t][c] = sbn[t][c];
        }
      }
    }
  }

  // ---- epilogue: round to the storage dtype, store rows < N and activation rows < rows
  uint16_t* yb = (uint16_t*)a.y + z * (int64_t)rows * N;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mt * 16 + 4 * lg + r;
        if (m < rows && nrow[t] < N) yb[(int64_t)m * N + nrow[t]] = T::from_f32(acc[mt][t][r]);
      }
}

template <class T, int BITS, int MT, int TN>
hipError_t launch_typed(const MatArgs& a, hipStream_t stream) {
  const int64_t rows_per_wg = (int64_t)kWaves * TN * 16;
  dim3 grid((unsigned)((a.N + rows_per_wg - 1) / rows_per_wg), 1, (unsigned)a.batches);
  hipLaunchKernelGGL((qmv_decode_kernel<T, BITS, MT, TN>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <class T, int BITS>
hipError_t launch_bits(const MatArgs& a, hipStream_t stream) {
  const bool wide = a.N >= 32768;
  if (a.rows_per_batch <= 16)
    return wide ? launch_typed<T, BITS, 1, 4>(a, stream) : launch_typed<T, BITS, 1, 1>(a, stream);
  return wide ? launch_typed<T, BITS, 2, 4>(a, stream) : launch_typed<T, BITS, 2, 1>(a, stream);
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

hipError_t launch_decode(const MatArgs& a, hipStream_t stream) {
  if (a.rows_per_batch > 32 || a.rows_per_batch <= 0 || a.batches > 65535) return hipErrorInvalidValue;
  return a.dtype == 1 ? launch_dtype<Bf16>(a, stream) : launch_dtype<Fp16>(a, stream);
}

}  // namespace qmm
