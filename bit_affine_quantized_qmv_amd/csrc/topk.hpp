// Launch interface of the per-row top-k over stored logits.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qmm {

// Largest k the top-k kernel takes.
constexpr int kTopkMax = 1024;
// Workspace layout: per row 4096 candidate words of 8 bytes (32768 bytes; the ABI's 32776
// bytes per row leave 8 spare).  Every word the merge reads is written by the select kernel
// of the same call, so the workspace needs no initial content.
constexpr int64_t kTopkWsRowWords = 4096;   // candidate words per row

struct TopkArgs {
  const void* logits;   // [rows, row_stride] of dtype (1 = bf16, 2 = fp16)
  int64_t rows;
  int64_t n;            // columns per row
  int64_t row_stride;   // elements
  int32_t k;
  int32_t dtype;
  int32_t* out_index;   // [rows, k]
  float* out_value;     // [rows, k] or null
  void* workspace;      // null (one workgroup per row) or the row-split workspace
};

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

}  // namespace qmm
