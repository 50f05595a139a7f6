/*
 * qmm.h -- C ABI of the affine group-quantized matmul library (libqmm.so, gfx950).
 *
 * Operation:  y = x . dequant(W)^T with w[n,k] = s[n,g] * q[n,k] + b[n,g], g = k / group_size.
 * (huggingface/transformers issue 47331, section "Root cause": the kernel call
 *  affine_qmm_t(x, w_packed, scales, biases, group_size, bits) returns y of shape
 *  x.shape[:-1] + [N]; "Fix": a batched input must give the same rows as the same input
 *  flattened to 2D.)
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers.  Descriptors are HOST pointers, read during the
 *     call only.  The caller owns all memory; the library allocates no device memory.  Its
 *     host state is a thread-local error message and, per device, cached launch settings
 *     (kernel LDS limits, occupancies) and the address of its one static device array (the
 *     workspace of qmm_qmv_argmax_noalloc), guarded so that calls from several threads are
 *     safe.
 *   - Strides are in elements.  A tensor pointer points at the view's first element (a view's
 *     storage offset is already applied).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued asynchronously;
 *     the library never synchronizes.
 *   - Every argument is validated before anything is launched; on error nothing is written,
 *     the call returns a negative QMM_ERR_* code and qmm_last_error() describes it
 *     (candle pitfall page "Metal 上批量 matmul 结果不对", section 现象: a structured error that
 *     names the layout is preferred over a silently wrong result).
 *   - dtype of x, scales, biases and y is one and the same: QMM_BF16 or QMM_FP16.
 *   - bits in {2,3,4,5,6,8}; group_size in {32,64,128}; K % group_size == 0.
 *   - Codes are a little-endian bitstream per weight row: code k of row n sits at bit k*bits
 *     of the row's stream of uint32 words, continuing into the next word when it straddles
 *     one (Metal Kernel Bits=8 final report, section 3.1, gives the 4- and 8-bit cases).
 */
#ifndef QMM_H
#define QMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMM_ABI_VERSION 1
#define QMM_MAX_DIMS 8
/* Collapsed activation rows up to this count use the decode (qmv) kernels. */
#define QMM_DECODE_MAX_ROWS 32

typedef enum { QMM_BF16 = 1, QMM_FP16 = 2 } qmm_dtype_t;

/* Return codes. */
enum {
  QMM_OK = 0,
  QMM_ERR_NULL = -1,        /* a required pointer is NULL                                  */
  QMM_ERR_UNSUPPORTED = -2, /* bits / group_size / dtype / flag not supported              */
  QMM_ERR_SHAPE = -3,       /* shapes disagree (K, N, y shape, K % group_size, qmv rows)    */
  QMM_ERR_LAYOUT = -4,      /* x batch dims cannot be expressed as <= 2 strided levels, a   */
                            /* negative stride, x last-dim stride != 1, or y not dense      */
  QMM_ERR_ALIGN = -5,       /* pointer / stride / K alignment that the kernels require      */
  QMM_ERR_HIP = -6          /* the HIP runtime reported an error at launch                  */
};

/* Flags for qmv / qmm_t. */
enum {
  /* Do not fold the batch dims: launch one grid slice per batch element, each of which
   * re-reads the whole weight.  Results are bitwise identical to the folded launch; it
   * exists to time the per-batch-element path against the folded one
   * (transformers issue 47331 summary page, 原因分析: 60 ms vs 2.2 ms for [32,1,K]). */
  QMM_FLAG_FORCE_STRIDED = 1u << 0
};

typedef struct {
  int32_t ndim;                   /* 1 .. QMM_MAX_DIMS                                    */
  int64_t shape[QMM_MAX_DIMS];
  int64_t stride[QMM_MAX_DIMS];   /* elements, >= 0                                        */
} qmm_tensor_desc_t;

typedef struct {
  const uint32_t* w_packed; /* device, row n at w_packed + n * w_row_stride                 */
  int64_t w_row_stride;     /* uint32 words, >= K*bits/32; the matmul needs a multiple of 4 */
  const void* scales;       /* device, [N, sb_row_stride] of dtype                          */
  const void* biases;       /* device, [N, sb_row_stride] of dtype                          */
  int64_t sb_row_stride;    /* elements, >= K / group_size                                  */
  int64_t N;                /* output features (weight rows)                                */
  int64_t K;                /* input features                                               */
  int32_t group_size;
  int32_t bits;
  int32_t dtype;            /* qmm_dtype_t                                                  */
} qmm_weight_desc_t;

/* How a call is executed; filled by qmm_plan (host only, no GPU needed).
 * Row r (0 <= r < rows_per_batch) of grid batch z reads x at
 *   x + z*batch_stride + (r / seg_rows)*seg_stride + (r % seg_rows)*row_stride
 * and writes y at y + (z*rows_per_batch + r)*N. */
typedef struct {
  int64_t rows;            /* total collapsed activation rows M                          */
  int64_t batches;         /* grid batch slices (1 unless QMM_FLAG_FORCE_STRIDED)         */
  int64_t batch_stride;
  int64_t rows_per_batch;
  int64_t seg_rows;        /* rows per contiguous-stride segment                          */
  int64_t seg_stride;
  int64_t row_stride;
  int32_t family;          /* 0: decode kernels (rows <= QMM_DECODE_MAX_ROWS), 1: prefill */
  int32_t kind;            /* 0: folded to one 2D matrix, 1: two strided levels,          */
                           /* 2: one grid slice per batch element (forced)                */
} qmm_plan_t;

/* Version of this ABI (QMM_ABI_VERSION). */
int32_t qmm_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  Valid until the next call
 * into the library on the same thread. */
const char* qmm_last_error(void);

/* Quantize W [N, K] (float32, row n at w + n*w_row_stride) per row and per group of
 * group_size columns with min/max affine parameters (transformers issue 47331, "Root
 * cause": quantize, then cast scales and biases to the storage dtype):
 *   s = fl32(fl32(max - min) / (2^bits - 1)),  b = min,
 *   q = clamp(round_half_even(fl32(fl32(w - b) / s)), 0, 2^bits - 1)   (q = 0 when s == 0),
 * scales/biases stored as s, b rounded to nearest-even in dtype.
 * Outputs are dense: w_packed [N, K*bits/32] words, scales and biases [N, K/group_size].
 * Requires K % group_size == 0 and finite inputs.  N == 0 is a no-op. */
int32_t qmm_quantize(const float* w, int64_t N, int64_t K, int64_t w_row_stride,
                     int32_t group_size, int32_t bits, int32_t dtype,
                     uint32_t* w_packed, void* scales, void* biases, void* stream);

/* Matrix-vector form for decode: y = x . dequant(W)^T where the collapsed activation rows
 * number at most QMM_DECODE_MAX_ROWS (otherwise QMM_ERR_SHAPE: use qmm_t).
 * x: shape [..., K] (any rank 1..8), last-dim stride 1, other strides >= 0.  Batch dims
 *    are folded when their strides allow (candle pitfall page, 怎么确认没中招: dims i, i+1
 *    merge iff stride[i] == stride[i+1]*shape[i+1]; size-1 dims always merge); at most two
 *    strided levels may remain, otherwise QMM_ERR_LAYOUT.
 * y: dense row-major, shape x.shape[:-1] + [N].
 * Every row's arithmetic is independent of how many rows share the call, so row i of a
 * batched call is bit-identical to a call on row i alone (MLX pull request 4516,
 * "Correctness": bitwise-identical outputs over decode steps).
 * Sums of x are taken in float32 after widening each element (MLX pull request 4516,
 * first commit: widen each input before adding it to the bias * sum(x) term).
 * Alignment: x, w_packed 16-byte aligned; x strides (except the last) multiples of 8;
 * w_row_stride a multiple of the 32-code run: 4 words for 4- and 8-bit codes, 2 words for
 * 2- and 6-bit codes, 1 word otherwise.
 * Any K that is a multiple of group_size is accepted (e.g. K = 96 with group_size 32): the
 * decode kernels mask a last 128-code slot that ends past K (MLX pull request 4516, second
 * commit text: inputs that are not aligned for the fast qmv kernel need a guarded tail).
 * When w_row_stride is not a multiple of 4 words (rows padded to an odd word count) the
 * call runs the MFMA kernel that qmm_t uses for many rows.
 * M == 0 or N == 0 is a no-op returning QMM_OK. */
int32_t qmv(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w,
            void* y, const qmm_tensor_desc_t* y_desc, uint32_t flags, void* stream);

/* Transposed matrix-matrix form (prefill and batched decode): same operation and contract
 * as qmv, any number of rows.  Up to QMM_DECODE_MAX_ROWS collapsed rows it runs the same
 * kernels as qmv (so the results agree bitwise); beyond that, and at every row count for the
 * shapes the decode kernels do not take, it runs the MFMA prefill kernel, which dequantizes
 * weight tiles to dtype in LDS before the products. */
int32_t qmm_t(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w,
              void* y, const qmm_tensor_desc_t* y_desc, uint32_t flags, void* stream);

/* Gathered-weight decode form (mixture-of-experts decode): a stack of num_experts
 * quantized weights that share N, K, group_size, bits and dtype, expert e's codes at
 * w->w_packed + e*w_expert_stride words and its scales/biases at w->scales / w->biases +
 * e*sb_expert_stride elements; activation row r uses expert e = expert_index[r]:
 *   y[r, :] = x[r, :] . dequant(W_e)^T.
 * (MLX pull request 4516, pull request text: "Gathered QMV" is the expert-indexed variant of
 * the affine qmv; "Correctness": covered with batched weights.  The Bits=8 final report,
 * section 4.3, shows such expert stacks.)
 * x: rows folding to ONE strided level (e.g. [M, K] or [M, 1, K]); y dense [..., N].
 * expert_index: DEVICE array of x's row count int32 values.  Indices are read on the GPU; a
 * row whose index is outside [0, num_experts) gets NaN outputs (nothing is read outside the
 * stack).  Each row runs the decode kernels on its own (at most 65535 rows), and its result
 * is bit-identical to qmv on that row with expert e's weight.
 * Strides: w_expert_stride >= N * w_row_stride (a multiple of 4), sb_expert_stride >=
 * N * sb_row_stride.  w_row_stride must be a multiple of 4 words (the decode kernels' row
 * alignment; QMM_ERR_ALIGN otherwise).  Other requirements as for qmv.  Zero rows or
 * N == 0 is a no-op. */
int32_t qmm_gather_qmv(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w,
                       int64_t num_experts, int64_t w_expert_stride, int64_t sb_expert_stride,
                       const int32_t* expert_index, void* y, const qmm_tensor_desc_t* y_desc, void* stream);

/* Decode form with a fused per-row argmax (e.g. greedy next-token choice on lm_head logits;
 * the failure the transformers issue 47331 report shows is this argmax collapsing to
 * token 0 for every row after the first, section "Reproduction"):
 *   y = x . dequant(W)^T as in qmv, and for every activation row m
 *   out_index[m] = the first n with y[m, n] == max_n y[m, n], out_value[m] = that value
 *   (as float32; NaN counts as larger than any number).
 * The comparison uses the values y holds (rounded to dtype), so out_index equals an argmax
 * over the returned logits.  y may be NULL: the logits are then not written at all.
 * workspace: DEVICE, 8-byte aligned, 8 * (rows + 1) bytes (QMM_ARGMAX_WORKSPACE_BYTES), ALL
 * ZERO when the call's kernel starts: zero-fill it once when it is allocated.  The kernel
 * leaves it all-zero again when it ends (its last workgroup reads the per-row keys out and
 * clears them), so one workspace serves any number of calls in stream order; calls that may
 * run at the same time (different streams) need workspaces of their own.  out_value may be
 * NULL.  Contract otherwise as for qmv (at most QMM_DECODE_MAX_ROWS rows), but w_row_stride
 * must be a multiple of 4 words (QMM_ERR_ALIGN otherwise); 0 < N < 2^31.
 * One kernel is enqueued. */
#define QMM_ARGMAX_WORKSPACE_BYTES(rows) (8 * ((rows) + 1))
int32_t qmm_qmv_argmax(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w, void* y,
                       const qmm_tensor_desc_t* y_desc, int32_t* out_index, float* out_value, void* workspace,
                       void* stream);

/* The same call as qmm_qmv_argmax without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The workspace is a library-owned device array of
 * QMM_NOALLOC_MAX_ROWS + 1 eight-byte words per GPU (512 bytes), kept until the process ends;
 * its device address is looked up once per device, on the first call made there.  Each call
 * enqueues a small kernel that zeroes the words it uses, then the decode kernel; nothing is
 * allocated or freed.  Calls on one GPU share that array: calls in stream order are fine,
 * calls that may run at the same time (different streams) race and give wrong results.
 * More than QMM_NOALLOC_MAX_ROWS collapsed activation rows -> QMM_ERR_SHAPE (the decode
 * family takes at most QMM_DECODE_MAX_ROWS anyway).  Results are bitwise those of
 * qmm_qmv_argmax; contract otherwise as for it. */
#define QMM_NOALLOC_MAX_ROWS 32
int32_t qmm_qmv_argmax_noalloc(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w, void* y,
                               const qmm_tensor_desc_t* y_desc, int32_t* out_index, float* out_value, void* stream);

/* Per-row top-k of stored logits (the top-k form of the decode epilogue on lm_head logits;
 * transformers issue 47331, "Reproduction": the next-token choice that collapses to token
 * 0): for every row m and j < k, out_index[m * k + j] and out_value[m * k + j] are the
 * column and value of the j-th largest entry of logits row m.  Order: larger value first;
 * NaN counts as larger than any number and +0 as larger than -0; equal values by lower
 * column, so k = 1 gives the column qmm_qmv_argmax returns.  A NaN entry is reported as a
 * quiet NaN.
 * logits: DEVICE [rows, row_stride] of dtype (QMM_BF16 or QMM_FP16), 2-byte aligned,
 * row_stride >= n.  out_index: DEVICE int32 [rows, k], 4-byte aligned; out_value: DEVICE
 * float32 [rows, k] or NULL.  Need 0 < n < 2^31, 0 <= rows < 2^31 and
 * 1 <= k <= min(n, QMM_TOPK_MAX) (QMM_ERR_SHAPE otherwise); rows == 0 is a no-op.
 * workspace: NULL, or DEVICE, 8-byte aligned, QMM_TOPK_WORKSPACE_BYTES(rows) bytes of any
 * content (the call writes every word it reads back; one workspace serves any number of
 * calls in stream order; calls that may overlap need workspaces of their own).  With a
 * workspace, long rows are split into column chunks of at least 2048 (about one chunk
 * workgroup per compute unit in all, at most 1024 / k chunks per row): one kernel writes
 * each chunk's k best candidates to the workspace and a second merges them per row.
 * Without one, or when a row is not split, each row is one workgroup and one kernel.  The
 * results are the same either way.
 * One or two kernels are enqueued; nothing is allocated. */
#define QMM_TOPK_MAX 1024
#define QMM_TOPK_WORKSPACE_BYTES(rows) (32776 * (rows))
int32_t qmm_topk(const void* logits, int32_t dtype, int64_t rows, int64_t n, int64_t row_stride, int32_t k,
                 int32_t* out_index, float* out_value, void* workspace, void* stream);

/* Decode with a per-row top-k: y = x . dequant(W)^T exactly as qmv (y is required and
 * dense, contract as for qmv), then qmm_topk over the rows of y (n = N, row_stride = N)
 * into out_index / out_value [rows, k], with `workspace` as for qmm_topk.  k is checked
 * before anything is enqueued.  The decode kernel and the top-k's one or two kernels are
 * enqueued. */
int32_t qmm_qmv_topk(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w, void* y,
                     const qmm_tensor_desc_t* y_desc, int32_t k, int32_t* out_index, float* out_value,
                     void* workspace, void* stream);

/* Dequantize a whole quantized weight to a dense matrix: out[n, k] = RNE_dtype(fl32(fma(s, q, b)))
 * with s, b the (n, k / group_size) scale and bias and q the code (transformers issue 47331,
 * "Root cause": the probe dequantizes the packed weight back to a dense tensor; the
 * float32 multiply-add followed by one rounding to dtype is this library's reading).
 * out: DEVICE [N, out_row_stride] of dtype, 16-byte aligned, out_row_stride >= K and a
 * multiple of 8.  w_packed and w_row_stride aligned to a 32-code run: 4 words (16 bytes)
 * for 4- and 8-bit codes, 2 words for 2- and 6-bit codes, 1 word otherwise.
 * N == 0 is a no-op. */
int32_t qmm_dequantize(const qmm_weight_desc_t* w, void* out, int64_t out_row_stride, void* stream);

/* Quantized embedding lookup: out[r, :] = dequantized row indices[r] of W (same rounding as
 * qmm_dequantize; Metal Kernel Bits=8 final report, section 3.2, dequantizes single rows of
 * a quantized table).  indices: DEVICE int32 [count]; an index outside [0, N) yields a NaN
 * row (nothing is read outside the table).  out as for qmm_dequantize with count rows.
 * count == 0 is a no-op. */
int32_t qmm_embedding(const qmm_weight_desc_t* w, const int32_t* indices, int64_t count, void* out,
                      int64_t out_row_stride, void* stream);

/* Host-only: validate a qmv (entry = 0) or qmm_t (entry = 1) call and report its plan
 * without touching the GPU.  Pointers inside `w` are only checked for NULL/alignment when
 * they are non-NULL (pass NULLs to test layouts alone).  Returns QMM_OK or the same error
 * code the call itself would return. */
int32_t qmm_plan(const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w,
                 const qmm_tensor_desc_t* y_desc, uint32_t flags, int32_t entry,
                 qmm_plan_t* out);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
