// extern "C" entry points of libqmm.so: validate, plan, launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>

#include "../../include/qmm.h"
#include "capi_internal.hpp"
#include "dispatch.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace {

thread_local std::string g_error;

int32_t finish(int32_t rc, const std::string& msg) {
  g_error = rc == QMM_OK ? std::string() : msg;
  return rc;
}

int32_t launch_status(hipError_t e) {
  if (e == hipSuccess) return finish(QMM_OK, "");
  return finish(QMM_ERR_HIP, std::string("HIP launch failed: ") + hipGetErrorString(e));
}

qmm::MatArgs make_args(const void* x, const qmm_plan_t& p, const qmm_weight_desc_t* w, void* y) {
  qmm::MatArgs a{};
  a.x = x;
  a.batches = p.batches;
  a.batch_stride = p.batch_stride;
  a.rows_per_batch = p.rows_per_batch;
  a.seg_rows = p.seg_rows;
  a.seg_stride = p.seg_stride;
  a.row_stride = p.row_stride;
  a.w = w->w_packed;
  a.w_row_stride = w->w_row_stride;
  a.scales = w->scales;
  a.biases = w->biases;
  a.sb_row_stride = w->sb_row_stride;
  a.y = y;
  a.N = w->N;
  a.K = w->K;
  a.group_size = w->group_size;
  a.bits = w->bits;
  a.dtype = w->dtype;
  return a;
}

int32_t run_matmul(const void* x, const qmm_tensor_desc_t* xd, const qmm_weight_desc_t* w, void* y,
                   const qmm_tensor_desc_t* yd, uint32_t flags, void* stream, int entry) {
  std::string err;
  qmm_plan_t p;
  const int rc = qmm::plan_matmul(x, xd, w, y, yd, flags, entry, true, &p, &err);
  if (rc != QMM_OK) return finish(rc, err);
  if (p.rows == 0 || w->N == 0) return finish(QMM_OK, "");
  const qmm::MatArgs a = make_args(x, p, w, y);
  hipStream_t s = (hipStream_t)stream;
  return launch_status(p.family == 0 ? qmm::launch_decode(a, s) : qmm::launch_prefill(a, s));
}

// Validation of a top-k call over logits rows (shared by the two top-k entry points).
int32_t check_topk(int32_t dtype, int64_t n, int64_t row_stride, int32_t k) {
  if (dtype != QMM_BF16 && dtype != QMM_FP16) return finish(QMM_ERR_UNSUPPORTED, "topk: dtype must be QMM_BF16 or QMM_FP16");
  if (n <= 0 || n >= (1ll << 31)) return finish(QMM_ERR_SHAPE, "topk: need 0 < n < 2^31");
  if (row_stride < n) return finish(QMM_ERR_SHAPE, "topk: row_stride < n");
  if (k < 1 || k > QMM_TOPK_MAX || k > n) return finish(QMM_ERR_SHAPE, "topk: need 1 <= k <= min(n, QMM_TOPK_MAX)");
  return QMM_OK;
}

}  // namespace

namespace qmm {

int32_t report(int32_t rc, const std::string& msg) { return finish(rc, msg); }

int32_t report_launch(hipError_t e) { return launch_status(e); }

int32_t prepare_qmv_argmax(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w, void* y,
                           const qmm_tensor_desc_t* y_desc, int32_t* out_index, float* out_value, MatArgs* out,
                           int64_t* rows) {
  std::string err;
  qmm_plan_t p;
  *rows = 0;
  // y may be NULL (no logits stored); validate the call with a stand-in output pointer
  static char y_stand_in alignas(16);
  int rc = plan_matmul(x, x_desc, w, y ? y : (void*)&y_stand_in, y_desc, 0, 0, true, &p, &err);
  if (rc != QMM_OK) return finish(rc, err);
  if (p.rows == 0) return finish(QMM_OK, "");
  if (w->w_row_stride % 4)
    return finish(QMM_ERR_ALIGN, "qmv_argmax: needs w_row_stride a multiple of 4 words");
  if (!out_index) return finish(QMM_ERR_NULL, "qmv_argmax: out_index must be non-NULL");
  if ((uintptr_t)out_index % 4 || (uintptr_t)out_value % 4)
    return finish(QMM_ERR_ALIGN, "qmv_argmax: out_index/out_value must be 4-byte aligned");
  if (w->N == 0 || w->N >= (1ll << 31)) return finish(QMM_ERR_SHAPE, "qmv_argmax: need 0 < N < 2^31");
  *out = make_args(x, p, w, y);
  out->argmax_index = out_index;
  out->argmax_value = out_value;
  *rows = p.rows;
  return finish(QMM_OK, "");
}

}  // namespace qmm

extern "C" {

int32_t qmm_topk(const void* logits, int32_t dtype, int64_t rows, int64_t n, int64_t row_stride, int32_t k,
                 int32_t* out_index, float* out_value, void* workspace, void* stream) {
  if (rows < 0) return finish(QMM_ERR_SHAPE, "topk: rows must be >= 0");
  const int32_t rc = check_topk(dtype, n, row_stride, k);
  if (rc != QMM_OK) return rc;
  if (rows == 0) return finish(QMM_OK, "");
  if (rows >= (1ll << 31)) return finish(QMM_ERR_SHAPE, "topk: rows must be < 2^31");
  if (!logits || !out_index) return finish(QMM_ERR_NULL, "topk: logits and out_index must be non-NULL");
  if ((uintptr_t)logits % 2 || (uintptr_t)out_index % 4 || (uintptr_t)out_value % 4 || (uintptr_t)workspace % 8)
    return finish(QMM_ERR_ALIGN, "topk: logits must be 2-byte, out_index/out_value 4-byte, workspace 8-byte aligned");
  const qmm::TopkArgs a{logits, rows, n, row_stride, k, dtype, out_index, out_value, workspace};
  return launch_status(qmm::launch_topk(a, (hipStream_t)stream));
}

int32_t qmm_qmv_topk(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w, void* y,
                     const qmm_tensor_desc_t* y_desc, int32_t k, int32_t* out_index, float* out_value,
                     void* workspace, void* stream) {
  std::string err;
  qmm_plan_t p;
  int rc = qmm::plan_matmul(x, x_desc, w, y, y_desc, 0, 0, true, &p, &err);
  if (rc != QMM_OK) return finish(rc, err);
  if (p.rows == 0) return finish(QMM_OK, "");
  rc = check_topk(w->dtype, w->N, w->N, k);
  if (rc != QMM_OK) return rc;
  if (!out_index) return finish(QMM_ERR_NULL, "qmv_topk: out_index must be non-NULL");
  if ((uintptr_t)out_index % 4 || (uintptr_t)out_value % 4 || (uintptr_t)workspace % 8)
    return finish(QMM_ERR_ALIGN, "qmv_topk: out_index/out_value must be 4-byte, workspace 8-byte aligned");
  const qmm::MatArgs a = make_args(x, p, w, y);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = p.family == 0 ? qmm::launch_decode(a, s) : qmm::launch_prefill(a, s);
  if (e != hipSuccess) return launch_status(e);
  const qmm::TopkArgs t{y, p.rows, w->N, w->N, k, w->dtype, out_index, out_value, workspace};
  return launch_status(qmm::launch_topk(t, s));
}

int32_t qmm_abi_version(void) { return QMM_ABI_VERSION; }

const char* qmm_last_error(void) { return g_error.c_str(); }

int32_t qmm_gather_qmv(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w,
                       int64_t num_experts, int64_t w_expert_stride, int64_t sb_expert_stride,
                       const int32_t* expert_index, void* y, const qmm_tensor_desc_t* y_desc, void* stream) {
  std::string err;
  qmm_plan_t p;
  // one grid slice per activation row: the forced per-row plan of the row layout
  int rc = qmm::plan_matmul(x, x_desc, w, y, y_desc, QMM_FLAG_FORCE_STRIDED, 1, true, &p, &err);
  if (rc != QMM_OK) return finish(rc, err);
  if (p.rows == 0 || w->N == 0) return finish(QMM_OK, "");
  if (p.rows_per_batch != 1)
    return finish(QMM_ERR_LAYOUT, "gather_qmv: x rows must fold into one strided level");
  if (w->w_row_stride % 4)
    return finish(QMM_ERR_ALIGN, "gather_qmv: needs w_row_stride a multiple of 4 words");
  if (num_experts < 1) return finish(QMM_ERR_SHAPE, "gather_qmv: num_experts must be >= 1");
  if (!expert_index) return finish(QMM_ERR_NULL, "gather_qmv: expert_index must be non-NULL");
  if ((uintptr_t)expert_index % 4) return finish(QMM_ERR_ALIGN, "gather_qmv: expert_index must be 4-byte aligned");
  if (w_expert_stride < w->N * w->w_row_stride || sb_expert_stride < w->N * w->sb_row_stride)
    return finish(QMM_ERR_SHAPE, "gather_qmv: expert strides smaller than one expert's weight");
  if (w_expert_stride % 4) return finish(QMM_ERR_ALIGN, "gather_qmv: w_expert_stride must be a multiple of 4 words");
  qmm::MatArgs a = make_args(x, p, w, y);
  a.w_index = expert_index;
  a.num_experts = num_experts;
  a.w_expert_stride = w_expert_stride;
  a.sb_expert_stride = sb_expert_stride;
  return launch_status(qmm::launch_decode(a, (hipStream_t)stream));
}

int32_t qmm_qmv_argmax(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w, void* y,
                       const qmm_tensor_desc_t* y_desc, int32_t* out_index, float* out_value, void* workspace,
                       void* stream) {
  qmm::MatArgs a;
  int64_t rows = 0;
  const int32_t rc = qmm::prepare_qmv_argmax(x, x_desc, w, y, y_desc, out_index, out_value, &a, &rows);
  if (rc != QMM_OK || rows == 0) return rc;
  if (!workspace) return finish(QMM_ERR_NULL, "qmv_argmax: workspace must be non-NULL");
  if ((uintptr_t)workspace % 8) return finish(QMM_ERR_ALIGN, "qmv_argmax: workspace must be 8-byte aligned");
  a.argmax_keys = (unsigned long long*)workspace;
  a.argmax_count = (unsigned int*)(a.argmax_keys + rows);
  return launch_status(qmm::launch_decode(a, (hipStream_t)stream));
}

// Shared validation of the whole-row dequantization entry points.
static int32_t run_dequant(const qmm_weight_desc_t* w, const int32_t* index, int64_t rows, void* out,
                           int64_t out_row_stride, void* stream) {
  if (!w) return finish(QMM_ERR_NULL, "w must be non-NULL");
  std::string err;
  int rc = qmm::check_codec(w->group_size, w->bits, w->dtype, &err);
  if (rc) return finish(rc, err);
  if (w->K <= 0 || w->N < 0 || rows < 0) return finish(QMM_ERR_SHAPE, "need K > 0, N >= 0 and rows >= 0");
  if (w->K % w->group_size) return finish(QMM_ERR_SHAPE, "K is not a multiple of group_size");
  if (w->w_row_stride < w->K * w->bits / 32 || w->sb_row_stride < w->K / w->group_size)
    return finish(QMM_ERR_SHAPE, "w_row_stride or sb_row_stride smaller than a row");
  if (out_row_stride < w->K) return finish(QMM_ERR_SHAPE, "out_row_stride < K");
  if (rows == 0 || (!index && w->N == 0)) return finish(QMM_OK, "");
  if (!w->w_packed || !w->scales || !w->biases || !out)
    return finish(QMM_ERR_NULL, "w_packed, scales, biases and out must be non-NULL");
  // a 32-code run is loaded with one access of its own size: 4 words for 4/8-bit codes,
  // 2 words for 2/6-bit codes, single words otherwise
  const int run_align = w->bits % 4 == 0 ? 4 : (w->bits % 2 == 0 ? 2 : 1);
  if ((uintptr_t)w->w_packed % (4 * run_align) || w->w_row_stride % run_align)
    return finish(QMM_ERR_ALIGN, "w_packed / w_row_stride not aligned to the code runs");
  if ((uintptr_t)w->scales % 2 || (uintptr_t)w->biases % 2) return finish(QMM_ERR_ALIGN, "scales/biases alignment");
  if ((uintptr_t)out % 16 || out_row_stride % 8)
    return finish(QMM_ERR_ALIGN, "out must be 16-byte aligned with a row stride that is a multiple of 8");
  if (index && (uintptr_t)index % 4) return finish(QMM_ERR_ALIGN, "indices must be 4-byte aligned");
  qmm::DequantArgs a{};
  a.w = w->w_packed;
  a.w_row_stride = w->w_row_stride;
  a.scales = w->scales;
  a.biases = w->biases;
  a.sb_row_stride = w->sb_row_stride;
  a.N = w->N;
  a.K = w->K;
  a.group_size = w->group_size;
  a.bits = w->bits;
  a.dtype = w->dtype;
  a.index = index;
  a.rows = rows;
  a.out = out;
  a.out_row_stride = out_row_stride;
  return launch_status(qmm::launch_dequant(a, (hipStream_t)stream));
}

int32_t qmm_dequantize(const qmm_weight_desc_t* w, void* out, int64_t out_row_stride, void* stream) {
  return run_dequant(w, nullptr, w ? w->N : 0, out, out_row_stride, stream);
}

int32_t qmm_embedding(const qmm_weight_desc_t* w, const int32_t* indices, int64_t count, void* out,
                      int64_t out_row_stride, void* stream) {
  if (count > 0 && !indices) return finish(QMM_ERR_NULL, "indices must be non-NULL");
  return run_dequant(w, indices, count, out, out_row_stride, stream);
}

int32_t qmm_quantize(const float* w, int64_t N, int64_t K, int64_t w_row_stride, int32_t group_size,
                     int32_t bits, int32_t dtype, uint32_t* w_packed, void* scales, void* biases,
                     void* stream) {
  std::string err;
  int rc = qmm::check_codec(group_size, bits, dtype, &err);
  if (rc) return finish(rc, err);
  if (N < 0 || K <= 0) return finish(QMM_ERR_SHAPE, "need N >= 0 and K > 0");
  if (K % group_size) return finish(QMM_ERR_SHAPE, "K is not a multiple of group_size");
  if (w_row_stride < K) return finish(QMM_ERR_SHAPE, "w_row_stride < K");
  if (N == 0) return finish(QMM_OK, "");
  if (!w || !w_packed || !scales || !biases)
    return finish(QMM_ERR_NULL, "w, w_packed, scales and biases must be non-NULL");
  if ((uintptr_t)w % 4 || (uintptr_t)w_packed % 4 || (uintptr_t)scales % 2 || (uintptr_t)biases % 2)
    return finish(QMM_ERR_ALIGN, "w/w_packed must be 4-byte and scales/biases 2-byte aligned");
  qmm::QuantArgs a{w, N, K, w_row_stride, group_size, bits, dtype, w_packed, scales, biases};
  return launch_status(qmm::launch_quantize(a, (hipStream_t)stream));
}

int32_t qmv(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w, void* y,
            const qmm_tensor_desc_t* y_desc, uint32_t flags, void* stream) {
  return run_matmul(x, x_desc, w, y, y_desc, flags, stream, 0);
}

int32_t qmm_t(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w, void* y,
              const qmm_tensor_desc_t* y_desc, uint32_t flags, void* stream) {
  return run_matmul(x, x_desc, w, y, y_desc, flags, stream, 1);
}

int32_t qmm_plan(const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w,
                 const qmm_tensor_desc_t* y_desc, uint32_t flags, int32_t entry, qmm_plan_t* out) {
  std::string err;
  if (entry != 0 && entry != 1) return finish(QMM_ERR_UNSUPPORTED, "entry must be 0 (qmv) or 1 (qmm_t)");
  const int rc = qmm::plan_matmul(nullptr, x_desc, w, nullptr, y_desc, flags, entry, false, out, &err);
  return finish(rc, err);
}

}  // extern "C"
