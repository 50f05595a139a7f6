// Launch interface between the host dispatcher and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

// One matmul call, already validated and planned.  Row r (0 <= r < rows_per_batch) of grid
// batch z reads x at x + z*batch_stride + (r / seg_rows)*seg_stride + (r % seg_rows)*row_stride
// and writes y + (z*rows_per_batch + r)*N.
struct MatArgs {
  const void* x;
  int64_t batches;
  int64_t batch_stride;
  int64_t rows_per_batch;
  int64_t seg_rows;
  int64_t seg_stride;
  int64_t row_stride;
  const uint32_t* w;
  int64_t w_row_stride;
  const void* scales;
  const void* biases;
  int64_t sb_row_stride;
  void* y;
  int64_t N;
  int64_t K;
  int32_t group_size;
  int32_t bits;
  int32_t dtype;  // 1 = bf16, 2 = fp16
  // Gathered weights (decode family only): when w_index is set, grid batch z (one activation
  // row) uses expert e = w_index[z] of a stack of num_experts weights, i.e. w, scales and
  // biases advanced by e * w_expert_stride words / e * sb_expert_stride elements.  An index
  // outside [0, num_experts) makes the row's outputs NaN.
  const int32_t* w_index = nullptr;
  int64_t num_experts = 0;
  int64_t w_expert_stride = 0;
  int64_t sb_expert_stride = 0;
  // Fused per-row argmax (decode family): when set, argmax_keys[z*rows_per_batch + m] (zero
  // when the kernel starts) receives the atomic maximum of argmax_key(y[m, n], n) over the
  // row; y itself is then optional (nullptr: no logits are stored).  The last workgroup to
  // finish (counted in *argmax_count, zero when the kernel starts) writes argmax_index[m]
  // and, when set, argmax_value[m], and returns the keys and the counter to zero.
  unsigned long long* argmax_keys = nullptr;
  unsigned int* argmax_count = nullptr;
  int32_t* argmax_index = nullptr;
  float* argmax_value = nullptr;
  // Rows of the last grid slice when it has fewer than rows_per_batch (0: every slice has
  // rows_per_batch).  The decode family's 16-row blocks of a 17..32-row call use it; slice
  // z's outputs still start at row z * rows_per_batch of y.
  int64_t last_rows = 0;
};

struct QuantArgs {
  const float* w;
  int64_t N;
  int64_t K;
  int64_t w_row_stride;
  int32_t group_size;
  int32_t bits;
  int32_t dtype;
  uint32_t* w_packed;
  void* scales;
  void* biases;
};

// Dequantization of whole weight rows: out row r = dequant(W[src(r)]), src(r) = index[r] when
// index is set (an embedding-row gather; out-of-range -> NaN row), else r.
struct DequantArgs {
  const uint32_t* w;
  int64_t w_row_stride;
  const void* scales;
  const void* biases;
  int64_t sb_row_stride;
  int64_t N;          // weight rows
  int64_t K;
  int32_t group_size;
  int32_t bits;
  int32_t dtype;
  const int32_t* index;
  int64_t rows;       // output rows
  void* out;
  int64_t out_row_stride;
};

// Decode family: rows_per_batch <= 32.
hipError_t launch_decode(const MatArgs& a, hipStream_t stream);
// MFMA prefill: any rows_per_batch.
hipError_t launch_prefill(const MatArgs& a, hipStream_t stream);
// Standalone dequantize / embedding gather.
hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream);
// Min/max group quantizer.
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);

}  // namespace qmm
