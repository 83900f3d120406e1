// C ABI of the MXFP4 library (and its MXFP8 comparator): argument validation
// and launch dispatch.
// Every check runs on the host before anything is enqueued, so an invalid
// call launches nothing and writes nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxfp4.h"
#include "mx_kernels.h"

namespace {

// HIP error behind the most recent MX_ERR_HIP returned on this thread.
thread_local hipError_t g_last_hip_error = hipSuccess;

mx_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MX_OK;
  g_last_hip_error = e;
  return MX_ERR_HIP;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_rotate(int32_t r) {
  return r == MX_ROT_NONE || r == MX_ROT_HADAMARD || r == MX_ROT_RAND_SIGN_HADAMARD ||
         r == MX_ROT_HADAMARD16;
}
bool valid_round(int32_t r) { return r == MX_ROUND_RNE || r == MX_ROUND_SR; }
bool valid_format(int32_t f) { return f == MX_FMT_FP4_E2M1 || f == MX_FMT_FP8_E4M3; }

// Code bytes per element, times two (E2M1: half a byte; E4M3: one byte).
int64_t code_bytes_x2(int32_t format) { return format == MX_FMT_FP8_E4M3 ? 2 : 1; }

// Reduction (K) and non-reduction (MN) extents of a quantized operand.
void operand_extents(const mx_qtensor *q, int64_t *mn, int64_t *k) {
  if (q->axis == 1) {
    *mn = q->rows;
    *k = q->cols;
  } else {
    *mn = q->cols;
    *k = q->rows;
  }
}

// Tiled-layout extents: MN up to a multiple of 256, K up to a multiple of 128
// (empty operands stay empty).
void padded_extents(int64_t rows, int64_t cols, int32_t axis, int64_t *mnp, int64_t *kp) {
  const int64_t mn = axis == 1 ? rows : cols;
  const int64_t k = axis == 1 ? cols : rows;
  const bool empty = rows == 0 || cols == 0;
  *mnp = empty ? 0 : (mn + 255) / 256 * 256;
  *kp = empty ? 0 : (k + 127) / 128 * 128;
}

// The GEMM addresses each operand's codes with 32-bit signed offsets (one
// 256-row block tile past the end must still be representable).
constexpr int64_t kMaxCodeBytes = (int64_t)1 << 30;

// Larger extents are unsupported: with at least 32 elements along the other
// axis their codes would pass the limit above anyway, and below it the
// product of two padded extents cannot overflow int64.
constexpr int64_t kMaxExtent = (int64_t)1 << 31;

bool extents_too_large(int64_t rows, int64_t cols) {
  return rows > kMaxExtent || cols > kMaxExtent;
}

// True when `rows` rows of `ld` elements of `elem_bytes` bytes each span more
// than 2^62 bytes, which no addressing in the kernels is built for
// (rows <= kMaxExtent).
bool span_too_large(int64_t rows, int64_t ld, int64_t elem_bytes) {
  return rows > 0 && ld > (((int64_t)1 << 62) / elem_bytes) / rows;
}

mx_status check_qtensor(const mx_qtensor *q) {
  if (q == nullptr) return MX_ERR_NULL;
  if (q->axis != 0 && q->axis != 1) return MX_ERR_ARG;
  if (q->block != 32) return MX_ERR_ARG;
  if (!valid_rotate(q->rotate) || !valid_round(q->round)) return MX_ERR_ARG;
  if (!valid_format(q->format)) return MX_ERR_ARG;
  if (q->format == MX_FMT_FP8_E4M3 && q->round != MX_ROUND_RNE) return MX_ERR_ARG;
  if (q->rows < 0 || q->cols < 0) return MX_ERR_SHAPE;
  const int64_t k = q->axis == 1 ? q->cols : q->rows;
  if (k % 32 != 0) return MX_ERR_SHAPE;
  if (q->rows > 0 && q->cols > 0) {
    if (q->codes == nullptr || q->scales == nullptr) return MX_ERR_NULL;
    if (!aligned(q->codes, 16) || !aligned(q->scales, 4)) return MX_ERR_ALIGN;
    if (extents_too_large(q->rows, q->cols)) return MX_ERR_UNSUPPORTED;
    int64_t mnp, kp;
    padded_extents(q->rows, q->cols, q->axis, &mnp, &kp);
    if (mnp * kp * code_bytes_x2(q->format) / 2 >= kMaxCodeBytes) return MX_ERR_UNSUPPORTED;
  }
  return MX_OK;
}

void fill_desc(mx_qtensor *d, void *codes, void *scales, int64_t rows, int64_t cols,
               int32_t axis, int32_t block, int32_t rotate, int32_t round, uint64_t seed,
               int32_t format) {
  if (d == nullptr) return;
  d->codes = codes;
  d->scales = scales;
  d->rows = rows;
  d->cols = cols;
  d->axis = axis;
  d->block = block;
  d->rotate = rotate;
  d->round = round;
  d->seed = seed;
  d->format = format;
}

// Validation shared by the single-orientation quantize calls.
mx_status check_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld,
                         int32_t axis, int32_t block, int32_t rotate, int32_t round,
                         const void *codes, const void *scales, int32_t format) {
  if (axis != 0 && axis != 1) return MX_ERR_ARG;
  if (block != 32) return MX_ERR_ARG;
  if (!valid_rotate(rotate) || !valid_round(round)) return MX_ERR_ARG;
  if (rows < 0 || cols < 0) return MX_ERR_SHAPE;
  const int64_t k = axis == 1 ? cols : rows;
  if (k % 32 != 0) return MX_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MX_OK;
  if (x_bf16 == nullptr || codes == nullptr || scales == nullptr) return MX_ERR_NULL;
  if (ld < cols) return MX_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(scales, 4)) return MX_ERR_ALIGN;
  if (extents_too_large(rows, cols) || span_too_large(rows, ld, 2)) return MX_ERR_UNSUPPORTED;
  int64_t mnp, kp;
  padded_extents(rows, cols, axis, &mnp, &kp);
  if (mnp * kp * code_bytes_x2(format) / 2 >= kMaxCodeBytes) return MX_ERR_UNSUPPORTED;
  if (axis == 1) {
    if (ld % 8 != 0 || !aligned(x_bf16, 16)) return MX_ERR_ALIGN;
  } else {
    if (!aligned(x_bf16, 2)) return MX_ERR_ALIGN;
  }
  return MX_OK;
}

mx_status sizes(int64_t rows, int64_t cols, int32_t axis, int32_t block, int32_t format,
                size_t *codes_bytes, size_t *scales_bytes) {
  if (codes_bytes == nullptr || scales_bytes == nullptr) return MX_ERR_NULL;
  if (axis != 0 && axis != 1) return MX_ERR_ARG;
  if (block != 32) return MX_ERR_ARG;
  if (rows < 0 || cols < 0) return MX_ERR_SHAPE;
  const int64_t k = axis == 1 ? cols : rows;
  if (k % 32 != 0) return MX_ERR_SHAPE;
  if (rows > 0 && cols > 0 && extents_too_large(rows, cols)) return MX_ERR_UNSUPPORTED;
  int64_t mnp, kp;
  padded_extents(rows, cols, axis, &mnp, &kp);
  *codes_bytes = (size_t)(mnp * kp * code_bytes_x2(format) / 2);
  *scales_bytes = (size_t)mnp * (size_t)kp / 32;
  return MX_OK;
}

mx_status quantize_any(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld, int32_t axis,
                       int32_t block, int32_t rotate, int32_t round, uint64_t seed, void *codes,
                       void *scales, mx_qtensor *out_desc, void *stream, int32_t format) {
  const mx_status st =
      check_quantize(x_bf16, rows, cols, ld, axis, block, rotate, round, codes, scales, format);
  if (st != MX_OK) return st;
  fill_desc(out_desc, codes, scales, rows, cols, axis, block, rotate, round, seed, format);
  if (rows == 0 || cols == 0) return MX_OK;
  mx::QuantArgs a;
  a.x = static_cast<const uint16_t *>(x_bf16);
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.axis = axis;
  a.rotate = rotate;
  a.round = round;
  a.seed_lo = (uint32_t)(seed & 0xFFFFFFFFull);
  a.seed_hi = (uint32_t)(seed >> 32);
  a.codes = static_cast<uint8_t *>(codes);
  a.scales = static_cast<uint8_t *>(scales);
  a.rb = 0;
  a.fmt = format == MX_FMT_FP8_E4M3 ? 1 : 0;
  return hip_status(mx::quantize_launch(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

mx_status mx_quantize_sizes(int64_t rows, int64_t cols, int32_t axis, int32_t block,
                            size_t *codes_bytes, size_t *scales_bytes) {
  return sizes(rows, cols, axis, block, MX_FMT_FP4_E2M1, codes_bytes, scales_bytes);
}

mx_status mx_quantize_fp8_sizes(int64_t rows, int64_t cols, int32_t axis, int32_t block,
                                size_t *codes_bytes, size_t *scales_bytes) {
  return sizes(rows, cols, axis, block, MX_FMT_FP8_E4M3, codes_bytes, scales_bytes);
}

mx_status mx_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld, int32_t axis,
                      int32_t block, int32_t rotate, int32_t round, uint64_t seed, void *codes,
                      void *scales, mx_qtensor *out_desc, void *stream) {
  return quantize_any(x_bf16, rows, cols, ld, axis, block, rotate, round, seed, codes, scales,
                      out_desc, stream, MX_FMT_FP4_E2M1);
}

mx_status mx_quantize_fp8(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld,
                          int32_t axis, int32_t block, int32_t rotate, uint64_t seed,
                          void *codes, void *scales, mx_qtensor *out_desc, void *stream) {
  return quantize_any(x_bf16, rows, cols, ld, axis, block, rotate, MX_ROUND_RNE, seed, codes,
                      scales, out_desc, stream, MX_FMT_FP8_E4M3);
}

mx_status mx_quantize_pair(const void *xa_bf16, int64_t rows_a, int64_t lda,
                           const void *xb_bf16, int64_t rows_b, int64_t ldb, int64_t cols,
                           int32_t block, int32_t rotate, int32_t round, uint64_t seed_a,
                           uint64_t seed_b, void *codes_a, void *scales_a, void *codes_b,
                           void *scales_b, mx_qtensor *desc_a, mx_qtensor *desc_b,
                           void *stream) {
  mx_status st = check_quantize(xa_bf16, rows_a, cols, lda, 1, block, rotate, round, codes_a,
                                scales_a, MX_FMT_FP4_E2M1);
  if (st != MX_OK) return st;
  st = check_quantize(xb_bf16, rows_b, cols, ldb, 1, block, rotate, round, codes_b, scales_b,
                      MX_FMT_FP4_E2M1);
  if (st != MX_OK) return st;
  fill_desc(desc_a, codes_a, scales_a, rows_a, cols, 1, block, rotate, round, seed_a,
            MX_FMT_FP4_E2M1);
  fill_desc(desc_b, codes_b, scales_b, rows_b, cols, 1, block, rotate, round, seed_b,
            MX_FMT_FP4_E2M1);
  const bool live_a = rows_a > 0 && cols > 0, live_b = rows_b > 0 && cols > 0;
  if (!live_a && !live_b) return MX_OK;
  mx::QuantArgs q[2];
  const void *xs[2] = {xa_bf16, xb_bf16};
  const int64_t rs[2] = {rows_a, rows_b}, lds[2] = {lda, ldb};
  const uint64_t seeds[2] = {seed_a, seed_b};
  void *cs[2] = {codes_a, codes_b}, *ss[2] = {scales_a, scales_b};
  for (int i = 0; i < 2; ++i) {
    q[i].x = static_cast<const uint16_t *>(xs[i]);
    q[i].rows = rs[i];
    q[i].cols = cols;
    q[i].ld = lds[i];
    q[i].axis = 1;
    q[i].rotate = rotate;
    q[i].round = round;
    q[i].seed_lo = (uint32_t)(seeds[i] & 0xFFFFFFFFull);
    q[i].seed_hi = (uint32_t)(seeds[i] >> 32);
    q[i].codes = static_cast<uint8_t *>(cs[i]);
    q[i].scales = static_cast<uint8_t *>(ss[i]);
    q[i].rb = 0;
    q[i].fmt = 0;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!live_b) return hip_status(mx::quantize_launch(q[0], s));
  if (!live_a) return hip_status(mx::quantize_launch(q[1], s));
  return hip_status(mx::quantize_pair_launch(q[0], q[1], s));
}

mx_status mx_quantize_dual(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld,
                           int32_t block, int32_t rotate, int32_t round, uint64_t seed1,
                           uint64_t seed0, void *codes1, void *scales1, void *codes0,
                           void *scales0, mx_qtensor *desc1, mx_qtensor *desc0, void *stream) {
  if (block != 32) return MX_ERR_ARG;
  if (!valid_rotate(rotate) || !valid_round(round)) return MX_ERR_ARG;
  if (rows < 0 || cols < 0) return MX_ERR_SHAPE;
  if (rows % 32 != 0 || cols % 32 != 0) return MX_ERR_SHAPE;
  const bool empty = rows == 0 || cols == 0;
  if (!empty) {
    if (x_bf16 == nullptr || codes1 == nullptr || scales1 == nullptr || codes0 == nullptr ||
        scales0 == nullptr)
      return MX_ERR_NULL;
    if (ld < cols) return MX_ERR_SHAPE;
    if (ld % 8 != 0 || !aligned(x_bf16, 16)) return MX_ERR_ALIGN;
    if (!aligned(codes1, 16) || !aligned(scales1, 4) || !aligned(codes0, 16) ||
        !aligned(scales0, 4))
      return MX_ERR_ALIGN;
    if (extents_too_large(rows, cols) || span_too_large(rows, ld, 2)) return MX_ERR_UNSUPPORTED;
    for (int axis = 0; axis < 2; ++axis) {
      int64_t mnp, kp;
      padded_extents(rows, cols, axis, &mnp, &kp);
      if (mnp * kp / 2 >= kMaxCodeBytes) return MX_ERR_UNSUPPORTED;
    }
  }
  fill_desc(desc0, codes0, scales0, rows, cols, 0, block, rotate, round, seed0, MX_FMT_FP4_E2M1);
  fill_desc(desc1, codes1, scales1, rows, cols, 1, block, rotate, round, seed1, MX_FMT_FP4_E2M1);
  if (empty) return MX_OK;

  mx::DualArgs a;
  a.x = static_cast<const uint16_t *>(x_bf16);
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.rotate = rotate;
  a.round = round;
  a.seed1_lo = (uint32_t)(seed1 & 0xFFFFFFFFull);
  a.seed1_hi = (uint32_t)(seed1 >> 32);
  a.seed0_lo = (uint32_t)(seed0 & 0xFFFFFFFFull);
  a.seed0_hi = (uint32_t)(seed0 >> 32);
  a.codes1 = static_cast<uint8_t *>(codes1);
  a.scales1 = static_cast<uint8_t *>(scales1);
  a.codes0 = static_cast<uint8_t *>(codes0);
  a.scales0 = static_cast<uint8_t *>(scales0);
  return hip_status(mx::quantize_dual_launch(a, static_cast<hipStream_t>(stream)));
}

namespace {

// mx_linear's checks of one (A, B, C) entry; fills the GEMM's extents and the
// entry's pointers. *empty is set when M or N is 0 (nothing to launch).
mx_status linear_entry(int32_t op, const mx_qtensor *A, const mx_qtensor *B, void *C, int64_t ldc,
                       int32_t out_dtype, mx::GemmArgs *g, bool *empty) {
  if (op != MX_OP_FPROP && op != MX_OP_DGRAD && op != MX_OP_WGRAD) return MX_ERR_ARG;
  if (out_dtype != MX_OUT_F32 && out_dtype != MX_OUT_BF16) return MX_ERR_ARG;
  mx_status st = check_qtensor(A);
  if (st != MX_OK) return st;
  st = check_qtensor(B);
  if (st != MX_OK) return st;
  // Which axis each operand must be quantized along, per op.
  static const int32_t need_axis[3][2] = {{1, 1}, {1, 0}, {0, 0}};
  if (A->axis != need_axis[op][0] || B->axis != need_axis[op][1]) return MX_ERR_ARG;
  if (A->rotate != B->rotate || A->format != B->format) return MX_ERR_MISMATCH;
  if (A->rotate == MX_ROT_RAND_SIGN_HADAMARD &&
      (uint32_t)(A->seed & 0xFFFFFFFFull) != (uint32_t)(B->seed & 0xFFFFFFFFull))
    return MX_ERR_MISMATCH;
  int64_t M, Ka, N, Kb;
  operand_extents(A, &M, &Ka);
  operand_extents(B, &N, &Kb);
  if (Ka != Kb) return MX_ERR_SHAPE;
  if (ldc < N) return MX_ERR_SHAPE;
  *empty = M == 0 || N == 0;
  if (!*empty) {
    if (C == nullptr) return MX_ERR_NULL;
    if (!aligned(C, out_dtype == MX_OUT_F32 ? 4 : 2)) return MX_ERR_ALIGN;
    if (span_too_large(M, ldc, out_dtype == MX_OUT_F32 ? 4 : 2)) return MX_ERR_UNSUPPORTED;
  }
  g->a_codes = static_cast<const uint8_t *>(A->codes);
  g->a_scales = static_cast<const uint8_t *>(A->scales);
  g->b_codes = static_cast<const uint8_t *>(B->codes);
  g->b_scales = static_cast<const uint8_t *>(B->scales);
  g->c = C;
  g->M = M;
  g->N = N;
  g->K = Ka;
  g->ldc = ldc;
  g->out_bf16 = out_dtype == MX_OUT_BF16 ? 1 : 0;
  return MX_OK;
}

}  // namespace

mx_status mx_linear(int32_t op, const mx_qtensor *A, const mx_qtensor *B, void *C, int64_t ldc,
                    int32_t out_dtype, void *stream) {
  mx::GemmArgs g;
  bool empty = false;
  const mx_status st = linear_entry(op, A, B, C, ldc, out_dtype, &g, &empty);
  if (st != MX_OK || empty) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(A->format == MX_FMT_FP8_E4M3 ? mx::gemm_e4m3_launch(g, s)
                                                 : mx::gemm_launch(g, s));
}

mx_status mx_linear_batched(int32_t op, int32_t count, const mx_qtensor *A, const mx_qtensor *B,
                            void *const *C, int64_t ldc, int32_t out_dtype, void *stream) {
  if (count < 1 || count > mx::kMaxGemmBatch) return MX_ERR_ARG;
  if (A == nullptr || B == nullptr || C == nullptr) return MX_ERR_NULL;
  mx::GemmArgs g;
  bool empty = false;
  for (int32_t i = 0; i < count; ++i) {
    if (A[i].rows != A[0].rows || A[i].cols != A[0].cols || A[i].axis != A[0].axis ||
        B[i].rows != B[0].rows || B[i].cols != B[0].cols || B[i].axis != B[0].axis)
      return MX_ERR_SHAPE;
    mx::GemmArgs gi;
    const mx_status st = linear_entry(op, &A[i], &B[i], C[i], ldc, out_dtype, &gi, &empty);
    if (st != MX_OK) return st;
    if (A[i].format != MX_FMT_FP4_E2M1) return MX_ERR_UNSUPPORTED;
    if (i == 0)
      g = gi;
    else
      g.more[i - 1] = mx::GemmEntry{gi.a_codes, gi.a_scales, gi.b_codes, gi.b_scales, gi.c};
  }
  if (empty) return MX_OK;
  g.batch = count;
  return hip_status(mx::gemm_launch(g, static_cast<hipStream_t>(stream)));
}

mx_status mx_dequantize(const mx_qtensor *q, float *out, int64_t ld, void *stream) {
  const mx_status st = check_qtensor(q);
  if (st != MX_OK) return st;
  if (ld < q->cols) return MX_ERR_SHAPE;
  if (q->rows == 0 || q->cols == 0) return MX_OK;
  if (out == nullptr) return MX_ERR_NULL;
  if (!aligned(out, 4)) return MX_ERR_ALIGN;
  if (span_too_large(q->rows, ld, 4)) return MX_ERR_UNSUPPORTED;
  mx::DequantArgs a;
  a.codes = static_cast<const uint8_t *>(q->codes);
  a.scales = static_cast<const uint8_t *>(q->scales);
  operand_extents(q, &a.mn, &a.k);
  padded_extents(q->rows, q->cols, q->axis, &a.mnp, &a.kp);
  a.axis = q->axis;
  a.fmt = q->format == MX_FMT_FP8_E4M3 ? 1 : 0;
  a.out = out;
  a.ld = ld;
  return hip_status(mx::dequantize_launch(a, static_cast<hipStream_t>(stream)));
}

const char *mx_status_string(int32_t status) {
  switch (status) {
    case MX_OK: return "MX_OK";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: bad extents";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN: misaligned pointer or leading dimension";
    case MX_ERR_ARG: return "MX_ERR_ARG: bad argument value";
    case MX_ERR_MISMATCH: return "MX_ERR_MISMATCH: operands quantized inconsistently";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED: not implemented";
    case MX_ERR_HIP: return "MX_ERR_HIP: HIP runtime error";
    default: return "unknown mx_status";
  }
}

const char *mx_version(void) { return "mxfp4-gfx950 0.1.0"; }

const char *mx_last_hip_error(void) {
  return g_last_hip_error == hipSuccess ? "hipSuccess" : hipGetErrorName(g_last_hip_error);
}

}  // extern "C"
