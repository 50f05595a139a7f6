// Host-side validation and batch-collapse planning (no GPU calls).
//
// Folding rule (candle pitfall page "Metal 上批量 matmul 结果不对", sections 出处 and
// 怎么确认没中招): two adjacent batch dims merge when stride[i] == stride[i+1] * shape[i+1];
// size-1 dims always merge.  The rule is applied to every leading dim of x (the rows dim
// included), at any rank.  A single remaining level is one 2D matrix (the flattening that
// fixes transformers issue 47331, "Fix"); two remaining levels are served by per-row
// addressing; more than two are rejected with a message that names the layout, instead
// of reading rows at the wrong offsets.
#include "dispatch.hpp"

#include <cstdarg>
#include <cstdio>
#include <string>

namespace qmm {

static int fail(std::string* err, int code, const char* fmt, ...) {
  if (err) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    *err = buf;
  }
  return code;
}

static std::string describe(const qmm_tensor_desc_t* d) {
  std::string s = "shape [";
  for (int i = 0; i < d->ndim; ++i) s += (i ? ", " : "") + std::to_string(d->shape[i]);
  s += "] stride [";
  for (int i = 0; i < d->ndim; ++i) s += (i ? ", " : "") + std::to_string(d->stride[i]);
  return s + "]";
}

static bool supported_bits(int32_t b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8; }
static bool supported_gs(int32_t g) { return g == 32 || g == 64 || g == 128; }

int check_codec(int32_t group_size, int32_t bits, int32_t dtype, std::string* err) {
  if (!supported_bits(bits)) return fail(err, QMM_ERR_UNSUPPORTED, "bits=%d not in {2,3,4,5,6,8}", bits);
  if (!supported_gs(group_size))
    return fail(err, QMM_ERR_UNSUPPORTED, "group_size=%d not in {32,64,128}", group_size);
  if (dtype != QMM_BF16 && dtype != QMM_FP16)
    return fail(err, QMM_ERR_UNSUPPORTED, "dtype=%d not QMM_BF16 (1) or QMM_FP16 (2)", dtype);
  return QMM_OK;
}

int plan_matmul(const void* x, const qmm_tensor_desc_t* xd, const qmm_weight_desc_t* w,
                const void* y, const qmm_tensor_desc_t* yd, uint32_t flags, int entry,
                bool require_pointers, qmm_plan_t* out, std::string* err) {
  if (!xd || !w || !yd) return fail(err, QMM_ERR_NULL, "x_desc, w and y_desc must be non-NULL");
  int rc = check_codec(w->group_size, w->bits, w->dtype, err);
  if (rc) return rc;
  if (flags & ~(uint32_t)QMM_FLAG_FORCE_STRIDED)
    return fail(err, QMM_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  const int64_t K = w->K, N = w->N;
  if (K <= 0 || N < 0) return fail(err, QMM_ERR_SHAPE, "need K > 0 and N >= 0 (K=%lld, N=%lld)",
                                   (long long)K, (long long)N);
  if (K % w->group_size) return fail(err, QMM_ERR_SHAPE, "K=%lld is not a multiple of group_size=%d",
                                     (long long)K, w->group_size);
  if (K > (1ll << 30) || N > (1ll << 40))
    return fail(err, QMM_ERR_SHAPE, "K=%lld or N=%lld too large", (long long)K, (long long)N);
  if (xd->ndim < 1 || xd->ndim > QMM_MAX_DIMS)
    return fail(err, QMM_ERR_SHAPE, "x ndim=%d not in [1, %d]", xd->ndim, QMM_MAX_DIMS);
  const int nd = xd->ndim;
  for (int i = 0; i < nd; ++i)
    if (xd->shape[i] < 0) return fail(err, QMM_ERR_SHAPE, "x has a negative size: %s", describe(xd).c_str());
  if (xd->shape[nd - 1] != K)
    return fail(err, QMM_ERR_SHAPE, "x last dim %lld != K=%lld", (long long)xd->shape[nd - 1], (long long)K);
  for (int i = 0; i < nd; ++i)
    if (xd->stride[i] < 0)
      return fail(err, QMM_ERR_LAYOUT, "x has a negative stride: %s", describe(xd).c_str());
  if (xd->stride[nd - 1] != 1)
    return fail(err, QMM_ERR_LAYOUT, "x last-dim stride must be 1: %s", describe(xd).c_str());
  // y: dense row-major x.shape[:-1] + [N]
  if (yd->ndim != nd) return fail(err, QMM_ERR_SHAPE, "y ndim=%d != x ndim=%d", yd->ndim, nd);
  for (int i = 0; i + 1 < nd; ++i)
    if (yd->shape[i] != xd->shape[i])
      return fail(err, QMM_ERR_SHAPE, "y %s does not match x %s", describe(yd).c_str(), describe(xd).c_str());
  if (yd->shape[nd - 1] != N)
    return fail(err, QMM_ERR_SHAPE, "y last dim %lld != N=%lld", (long long)yd->shape[nd - 1], (long long)N);
  {
    int64_t expect = 1;
    for (int i = nd - 1; i >= 0; --i) {
      if (yd->shape[i] > 1 && yd->stride[i] != expect)
        return fail(err, QMM_ERR_LAYOUT, "y must be dense row-major: %s", describe(yd).c_str());
      expect *= yd->shape[i];
    }
  }
  const int64_t row_words = K * w->bits / 32;
  const int64_t n_groups = K / w->group_size;
  if (w->w_row_stride < row_words)
    return fail(err, QMM_ERR_SHAPE, "w_row_stride=%lld < K*bits/32=%lld", (long long)w->w_row_stride,
                (long long)row_words);
  // rows are read in 32-code runs: 4 words (16 bytes) for 4/8-bit codes, 2 words for
  // 2/6-bit codes, single words otherwise
  const int run_align = w->bits % 4 == 0 ? 4 : (w->bits % 2 == 0 ? 2 : 1);
  if (w->w_row_stride % run_align)
    return fail(err, QMM_ERR_ALIGN, "w_row_stride=%lld must be a multiple of %d words for %d-bit codes",
                (long long)w->w_row_stride, run_align, w->bits);
  if (w->sb_row_stride < n_groups)
    return fail(err, QMM_ERR_SHAPE, "sb_row_stride=%lld < K/group_size=%lld", (long long)w->sb_row_stride,
                (long long)n_groups);

  int64_t M = 1;
  for (int i = 0; i + 1 < nd; ++i) M *= xd->shape[i];

  qmm_plan_t p = {};
  p.rows = M;
  p.batches = 1;
  p.rows_per_batch = M;
  p.seg_rows = M > 0 ? M : 1;
  // The decode kernels take rows that start on 16-byte boundaries (any K that is a multiple
  // of the group size: a last slot that ends past K is masked); weights padded to other row
  // strides go through the MFMA kernel at every row count, whose per-row arithmetic does not
  // depend on the row count either.
  p.family = (M <= QMM_DECODE_MAX_ROWS && w->w_row_stride % 4 == 0) ? 0 : 1;
  if (entry == 0 && M > QMM_DECODE_MAX_ROWS)
    return fail(err, QMM_ERR_SHAPE, "qmv takes at most %d activation rows, got %lld; use qmm_t",
                QMM_DECODE_MAX_ROWS, (long long)M);
  if (M == 0 || N == 0) {
    if (out) *out = p;
    return QMM_OK;
  }

  if (require_pointers || x || y || w->w_packed || w->scales || w->biases) {
    if (!x || !y || !w->w_packed || !w->scales || !w->biases)
      return fail(err, QMM_ERR_NULL, "x, y, w_packed, scales and biases must be non-NULL");
    if ((uintptr_t)x % 16) return fail(err, QMM_ERR_ALIGN, "x must be 16-byte aligned");
    if ((uintptr_t)w->w_packed % 16) return fail(err, QMM_ERR_ALIGN, "w_packed must be 16-byte aligned");
    if ((uintptr_t)w->scales % 2 || (uintptr_t)w->biases % 2 || (uintptr_t)y % 2)
      return fail(err, QMM_ERR_ALIGN, "scales, biases and y must be 2-byte aligned");
  }
  for (int i = 0; i + 1 < nd; ++i)
    if (xd->shape[i] > 1 && xd->stride[i] % 8)
      return fail(err, QMM_ERR_ALIGN, "x strides must be multiples of 8 elements: %s", describe(xd).c_str());

  // fold the leading dims, innermost first
  int64_t sz[QMM_MAX_DIMS], st[QMM_MAX_DIMS];
  int lv = 0;  // levels, outermost first after the loop (stored reversed)
  for (int i = nd - 2; i >= 0; --i) {
    if (xd->shape[i] == 1) continue;
    if (lv > 0 && xd->stride[i] == st[lv - 1] * sz[lv - 1]) {
      sz[lv - 1] *= xd->shape[i];
      continue;
    }
    sz[lv] = xd->shape[i];
    st[lv] = xd->stride[i];
    ++lv;
  }
  if (lv > 2)
    return fail(err, QMM_ERR_LAYOUT,
                "x batch dims do not fold into at most two strided levels (%d remain): %s", lv,
                describe(xd).c_str());
  const bool force = (flags & QMM_FLAG_FORCE_STRIDED) != 0;
  if (lv == 1) {
    // one level: sz[0] rows at stride st[0]
    if (force) {
      p.kind = 2;
      p.batches = sz[0];
      p.batch_stride = st[0];
      p.rows_per_batch = 1;
      p.seg_rows = 1;
    } else {
      p.kind = 0;
      p.seg_rows = sz[0];
      p.row_stride = st[0];
    }
  } else if (lv == 2) {
    // outer level sz[1] at st[1], inner level sz[0] at st[0]
    if (force) {
      p.kind = 2;
      p.batches = sz[1];
      p.batch_stride = st[1];
      p.rows_per_batch = sz[0];
      p.seg_rows = sz[0];
      p.row_stride = st[0];
    } else {
      p.kind = 1;
      p.seg_rows = sz[0];
      p.row_stride = st[0];
      p.seg_stride = st[1];
    }
  }
  if (p.batches > 65535)
    return fail(err, QMM_ERR_UNSUPPORTED, "forced strided launch supports at most 65535 batch slices");
  if (out) *out = p;
  return QMM_OK;
}

}  // namespace qmm
