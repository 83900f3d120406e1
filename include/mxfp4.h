/*
 * mxfp4.h -- C ABI of the MI355X (gfx950) MXFP4 linear-layer library.
 *
 * The library computes the three GEMMs of a transformer linear layer with
 * both operands in MXFP4 (36Kr article "Neue Studie von AMD durchbricht die
 * bestehende Erkenntnis: Die Instabilitaet von FP4-Training liegt nicht an
 * unzureichender Zufaelligkeit", section "Fehlerdiagnoseexperiment"):
 *   Fprop  Y  = X  W^T     X [T, in],  W [out, in]  -> Y  [T, out]
 *   Dgrad  dX = dY W       dY [T, out], W [out, in] -> dX [T, in]
 *   Wgrad  dW = dY^T X     dY [T, out], X [T, in]   -> dW [out, in]
 * Every operand is first rotated along the GEMM reduction axis (none, the
 * deterministic 32-point Hadamard, or the random-sign Hadamard -- same page,
 * same section) and then quantized to MXFP4: blocks of 32 elements sharing
 * one E8M0 exponent, each element an E2M1 4-bit float (same page, section
 * "Was ist MXFP4?"), rounded to nearest-even or stochastically.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory)
 *    on the current HIP device. The caller allocates and owns every buffer;
 *    the library allocates nothing and keeps no per-call state.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work and return; results are ready when the stream
 *    reaches them.
 *  - Arguments are validated before anything is enqueued; on any error
 *    nothing is launched and no output byte is written. Nothing throws.
 *  - Results are bitwise deterministic for identical inputs (no atomics).
 *  - Calls that write the same buffers concurrently on different streams race.
 */
#ifndef MXFP4_H_
#define MXFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (returned by every call). */
typedef enum mx_status {
  MX_OK = 0,
  MX_ERR_NULL = -1,        /* a required pointer is NULL                         */
  MX_ERR_SHAPE = -2,       /* bad extents: reduction extent % 32, ld < cols, K mismatch */
  MX_ERR_ALIGN = -3,       /* a device pointer or leading dimension is misaligned */
  MX_ERR_ARG = -4,         /* bad enum value, block != 32, axis wrong for the op  */
  MX_ERR_MISMATCH = -5,    /* A and B quantized with different rotations / sign seeds / formats */
  MX_ERR_UNSUPPORTED = -6, /* valid request the library does not implement       */
  MX_ERR_HIP = -7          /* the HIP runtime reported a launch error            */
} mx_status;

/* Pre-quantization rotation along the reduction axis (36Kr, section
 * "Fehlerdiagnoseexperiment": randomized vs deterministic Hadamard; section
 * "Ende-zu-Ende-Effizienz": the stabilised run is labelled H16). */
typedef enum mx_rotate {
  MX_ROT_NONE = 0,
  MX_ROT_HADAMARD = 1,            /* y = (H32 x) * fp32(1/sqrt 32), H32 Sylvester */
  MX_ROT_RAND_SIGN_HADAMARD = 2,  /* x_k <- s_k x_k first, s_k = +-1 from Philox */
  MX_ROT_HADAMARD16 = 3           /* y = block-diag(H16, H16) x / 4 inside each
                                     32-element block (two 16-point butterflies) */
} mx_rotate;

/* Element rounding (36Kr, "Was ist MXFP4?": nearest; "Fehlerdiagnoseexperiment":
 * stochastic rounding with zero expected error). */
typedef enum mx_round {
  MX_ROUND_RNE = 0,   /* nearest E2M1 value, ties to even mantissa, saturate at 6 */
  MX_ROUND_SR = 1     /* upper neighbour with probability (a-lo)/(hi-lo), 24-bit uniform */
} mx_round;

/* Element format of a quantized operand. MXFP4 is the method; MXFP8 with
 * E4M3 elements is the baseline it is measured against (36Kr, opening
 * section: FP4 has in theory twice FP8's compute; "Ende-zu-Ende-Effizienz":
 * throughput against the FP8 baseline; ShowAPI page
 * "AMD颠覆认知：FP4不稳定性的真正原因", section 2.2: E4M3 as an FP8 format). */
typedef enum mx_format {
  MX_FMT_FP4_E2M1 = 0,  /* written by mx_quantize / _dual / _pair             */
  MX_FMT_FP8_E4M3 = 1   /* written by mx_quantize_fp8                         */
} mx_format;

typedef enum mx_op { MX_OP_FPROP = 0, MX_OP_DGRAD = 1, MX_OP_WGRAD = 2 } mx_op;

typedef enum mx_out_dtype { MX_OUT_F32 = 0, MX_OUT_BF16 = 1 } mx_out_dtype;

/*
 * A quantized operand, filled by mx_quantize (and mx_quantize_dual,
 * mx_quantize_fp8). Its pointers are BORROWED from the caller (the buffers
 * passed to the quantize call). The layout below is MXFP4's; the MXFP8
 * comparator's codes are described at mx_quantize_fp8.
 *
 * The operand is always stored reduction-major ("K-major"), whatever the axis:
 *   MN = rows, K = cols   when axis == 1 (blocks run along a row);
 *   MN = cols, K = rows   when axis == 0 (blocks run down a column; the
 *                         source is written out transposed).
 * It is zero-padded to MNp = MN rounded up to 256 (whole 256-row panels, the
 * GEMM's block height) and Kp = K rounded up to 128, and stored in 16 x 128
 * tiles, the fragment shape of the gfx950 FP4 matrix instruction, so the GEMM
 * streams every tile as one contiguous 1 KB:
 *   codes : MNp * Kp / 2 bytes. Tile (g, q) -- rows 16g..16g+15, K elements
 *           128q..128q+127 -- is the 1 KB at byte (g * Kp/128 + q) * 1024;
 *           inside it, 32-element block c (0..3) of row r (0..15) is the 16
 *           bytes at c * 256 + r * 16, two codes per byte, the even K index in
 *           the low nibble. Code = sign << 3 | E2M1 magnitude code (0..7 for
 *           0, 0.5, 1, 1.5, 2, 3, 4, 6).
 *   scales: MNp * Kp / 32 bytes, [Kp/128][MNp/256][4][4][16][4]: the E8M0
 *           code s (value 2^(s-127)) of block kb = 4q + c of row
 *           mn = 256T + 16h + r is at byte
 *           (q * MNp/256 + T) * 1024 + (h / 4) * 256 + c * 64 + r * 4 + h % 4.
 *           One 1 KB block per K slice and 256-row panel; inside it, the
 *           256-byte quarter h / 4 holds, for every (r, c), the scales of
 *           four consecutive row groups as four consecutive bytes at
 *           (16c + r) * 4, so a matrix-instruction lane reads the scales of
 *           its row groups with one linear 4-byte-per-lane read and picks
 *           each with the instruction's byte select. 0xFF marks a block that
 *           held a NaN or
 *           Inf (its codes are 0).
 * Padding rows and blocks hold the encoding of zeros (codes 0, scale code 0).
 * Element value = (-1)^sign * E2M1(mag) * 2^(s - 127).
 */
typedef struct mx_qtensor {
  void *codes;
  void *scales;
  int64_t rows, cols;   /* logical bf16 source shape [rows, cols]             */
  int32_t axis;         /* 0 or 1: the dimension the 32-blocks run along (= K) */
  int32_t block;        /* always 32                                          */
  int32_t rotate;       /* mx_rotate used                                     */
  int32_t round;        /* mx_round used                                      */
  uint64_t seed;        /* seed used (see mx_quantize)                        */
  int32_t format;       /* mx_format of the codes (layout: see mx_quantize_fp8) */
} mx_qtensor;

/*
 * Byte sizes of the tiled codes and scales of a [rows, cols] source quantized
 * along `axis`, padding included (see mx_qtensor). Host-only; launches nothing.
 * Errors: MX_ERR_NULL (null out-pointer), MX_ERR_ARG (axis, block != 32),
 * MX_ERR_SHAPE (negative extents, or the axis extent not a multiple of 32),
 * MX_ERR_UNSUPPORTED (a non-empty source with rows or cols above 2^31).
 */
mx_status mx_quantize_sizes(int64_t rows, int64_t cols, int32_t axis, int32_t block,
                            size_t *codes_bytes, size_t *scales_bytes);

/*
 * Rotate + quantize a bf16 tensor into MXFP4 (36Kr, "Was ist MXFP4?": shared
 * E8M0 exponent per 32-element block from the block maximum, 4-bit elements;
 * "Fehlerdiagnoseexperiment": Hadamard rotation before quantization).
 *
 *  x_bf16  device, bf16 [rows, cols] row-major with leading dimension `ld`
 *          (elements). Read only.
 *  axis    1: blocks of 32 along each row (needs cols % 32 == 0);
 *          0: blocks of 32 down each column (needs rows % 32 == 0).
 *  block   must be 32.
 *  rotate  mx_rotate; applied per 32-block along `axis`, before the scale.
 *  round   mx_round.
 *  seed    64-bit. Random signs use key (seed_lo, 0) with counter
 *          (k >> 2, 0, 1, 0), word k & 3, bit 31, for reduction index k, so
 *          two operands quantized with the same low 32 bits share the signs
 *          and the rotation cancels in the product. Stochastic rounding uses
 *          key (seed_lo, seed_hi) with counter (L >> 2 mod 2^32, L >> 34, 0, 0),
 *          word L & 3, top 24 bits, for the row-major source index
 *          L = row * cols + col. Generator: Philox4x32-10 (Salmon et al., SC'11).
 *          Ignored when neither random option is selected.
 *  codes   device, >= codes_bytes of mx_quantize_sizes, 16-byte aligned. Written
 *          in full (padding included).
 *  scales  device, >= scales_bytes of mx_quantize_sizes, 4-byte aligned. Written
 *          in full.
 *  out_desc  host, may be NULL; filled with the operand's description.
 * Requirements: ld >= cols; axis 1: x_bf16 16-byte aligned and ld % 8 == 0;
 * axis 0: x_bf16 2-byte aligned (any ld; 4-byte-aligned rows load faster).
 * rows == 0 or cols == 0 is valid and launches nothing.
 * Limit: the padded codes (MNp * Kp / 2 bytes) must stay below 1 GiB, rows
 * and cols at most 2^31, and rows * ld * 2 bytes at most 2^62, else
 * MX_ERR_UNSUPPORTED.
 * Errors: MX_ERR_NULL, MX_ERR_ARG, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_UNSUPPORTED,
 * MX_ERR_HIP.
 */
mx_status mx_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld,
                      int32_t axis, int32_t block, int32_t rotate, int32_t round,
                      uint64_t seed, void *codes, void *scales, mx_qtensor *out_desc,
                      void *stream);

/*
 * Both packed orientations of one bf16 tensor from a single read of it: the
 * axis-1 and the axis-0 operand that mx_quantize would write for this
 * source, with seeds seed1 and seed0. Each linear layer uses every source
 * tensor twice, once per orientation (36Kr, section
 * "Fehlerdiagnoseexperiment": X enters Fprop and Wgrad, W Fprop and Dgrad,
 * dY Dgrad and Wgrad), so the tensor is read once instead of twice.
 *
 *   x_bf16, rows, cols, ld, block, rotate, round : as for mx_quantize, with
 *       rows % 32 == 0 and cols % 32 == 0 (both are reduction extents here),
 *       ld % 8 == 0 and x_bf16 16-byte aligned.
 *   codes1 / scales1 / desc1 : the axis-1 operand (mx_quantize_sizes with
 *       axis 1 gives the sizes), quantized with seed1.
 *   codes0 / scales0 / desc0 : the axis-0 operand, quantized with seed0.
 *   Ownership, alignment of the outputs, the descriptors (may be NULL), the
 *   limits and the error codes are as for mx_quantize. The results are
 *   byte-identical to the two mx_quantize calls.
 */
mx_status mx_quantize_dual(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld,
                           int32_t block, int32_t rotate, int32_t round, uint64_t seed1,
                           uint64_t seed0, void *codes1, void *scales1, void *codes0,
                           void *scales0, mx_qtensor *desc1, mx_qtensor *desc0, void *stream);

/*
 * Two axis-1 quantizations in one launch: the Fprop pair X [T, in] and
 * W [out, in], which share their reduction extent (36Kr, section
 * "Fehlerdiagnoseexperiment": Fprop takes X and W, both quantized along
 * `in`). One launch covers the row groups of A and then those of B, which
 * saves one launch's ramp and drain.
 *
 *   xa_bf16, rows_a, lda / xb_bf16, rows_b, ldb : the two sources
 *       [rows_a, cols] and [rows_b, cols], each as x_bf16, rows, ld of
 *       mx_quantize with axis 1 (ld % 8 == 0, 16-byte aligned).
 *   cols, block, rotate, round : shared; cols % 32 == 0, block == 32.
 *   seed_a / seed_b : as seed of mx_quantize for each operand (for an Fprop,
 *       s and s | 1 << 32: shared random signs, independent SR noise).
 *   codes_a, scales_a, desc_a / codes_b, scales_b, desc_b : as codes,
 *       scales, out_desc of mx_quantize with axis 1, one set per operand.
 *   Either operand may be empty (rows 0). Ownership, alignment, the
 *   descriptors (may be NULL), the limits and the error codes are as for
 *   mx_quantize, checked for A and then for B before anything is launched.
 *   The results are byte-identical to the two mx_quantize calls.
 */
mx_status mx_quantize_pair(const void *xa_bf16, int64_t rows_a, int64_t lda,
                           const void *xb_bf16, int64_t rows_b, int64_t ldb, int64_t cols,
                           int32_t block, int32_t rotate, int32_t round, uint64_t seed_a,
                           uint64_t seed_b, void *codes_a, void *scales_a, void *codes_b,
                           void *scales_b, mx_qtensor *desc_a, mx_qtensor *desc_b,
                           void *stream);

/*
 * Byte sizes of the tiled codes and scales of mx_quantize_fp8 (codes: one
 * byte per element, MNp * Kp; scales as for MXFP4, MNp * Kp / 32). Host-only.
 * Errors as for mx_quantize_sizes.
 */
mx_status mx_quantize_fp8_sizes(int64_t rows, int64_t cols, int32_t axis, int32_t block,
                                size_t *codes_bytes, size_t *scales_bytes);

/*
 * Rotate + quantize a bf16 tensor into MXFP8 with E4M3 elements: the FP8
 * comparator of the MXFP4 path (see mx_format). Same blocks, rotations and
 * E8M0 scales as mx_quantize; the block exponent is floor(log2 amax) - 8
 * (E4M3's largest exponent), clamped to [-127, 127], and each element
 * t = y * 2^-e is rounded to the nearest E4M3 value, ties to even, values
 * above 448 saturating to 448. Only nearest rounding: the pages compare
 * stochastic rounding within MXFP4, not within FP8.
 *
 *  x_bf16, rows, cols, ld, axis, block, rotate, seed, out_desc, stream:
 *          as for mx_quantize (seed only feeds the random signs).
 *  codes   device, >= codes_bytes of mx_quantize_fp8_sizes, 16-byte aligned.
 *          Same zero-padded [MNp, Kp] extent and 16 x 128 tiles as MXFP4, but
 *          a tile is 2 KB, at byte (g * Kp/128 + q) * 2048, holding
 *          [16-element chunk j][row r][16 B]: K element k of the slice, row
 *          r, at (k / 16) * 256 + r * 16 + k % 16. (The matrix instruction
 *          takes lane (r, g)'s 32 bytes as chunks g and g + 4 of row r, i.e.
 *          the 16 bytes at 16 l and at 1024 + 16 l for lane l = 16 g + r.)
 *          Code = sign << 7 | E4M3 magnitude (exponent bias 7, 0x7E = 448;
 *          0x7F is never written).
 *  scales  as for mx_quantize.
 * Limit: the padded codes (MNp * Kp bytes) must stay below 1 GiB; the other
 * limits are mx_quantize's.
 * Errors: MX_ERR_NULL, MX_ERR_ARG, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_UNSUPPORTED,
 * MX_ERR_HIP.
 */
mx_status mx_quantize_fp8(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld,
                          int32_t axis, int32_t block, int32_t rotate, uint64_t seed,
                          void *codes, void *scales, mx_qtensor *out_desc, void *stream);

/*
 * One GEMM of the triple over two quantized operands, fp32 accumulation on
 * the gfx950 block-scaled matrix cores:
 *     C[m][n] = sum_k A(m, k) * B(n, k)
 * with A, B in their tiled K-major form (36Kr, "Fehlerdiagnoseexperiment").
 *
 *  op = MX_OP_FPROP: A = q(X [T,in], axis 1),  B = q(W [out,in], axis 1); C [T][out]
 *  op = MX_OP_DGRAD: A = q(dY [T,out], axis 1), B = q(W [out,in], axis 0); C [T][in]
 *  op = MX_OP_WGRAD: A = q(dY [T,out], axis 0), B = q(X [T,in], axis 0);  C [out][in]
 *  C        device, row-major [M][N] with leading dimension ldc >= N (elements),
 *           fp32 or bf16 (round to nearest even of the fp32 accumulator).
 *           Written; must not overlap A or B.
 *  stream   hipStream_t as void*.
 * Both operands must use the same rotation and, for the random-sign rotation,
 * the same low 32 bits of the seed (else MX_ERR_MISMATCH): that is what makes
 * the rotation cancel in the product. Their reduction extents must match.
 * Both must have the same format (else MX_ERR_MISMATCH): two MXFP8 operands
 * run the E4M3 comparator GEMM (same call, same C), two MXFP4 operands the
 * MXFP4 GEMM.
 * A block with the NaN scale code 0xFF (a NaN or Inf in its source block)
 * makes every element of C that reduces over it NaN.
 * Requirements: C aligned to its element size (4 bytes for fp32, 2 for bf16),
 * ldc >= N. M or N == 0 launches nothing; K == 0 with M, N > 0 writes zeros.
 * Limits: each operand's as for mx_quantize (MX_ERR_UNSUPPORTED beyond them,
 * also for a descriptor not filled by a quantize call), and M * ldc elements
 * of C at most 2^62 bytes (else MX_ERR_UNSUPPORTED).
 * Errors: MX_ERR_NULL, MX_ERR_ARG, MX_ERR_SHAPE, MX_ERR_ALIGN,
 * MX_ERR_MISMATCH, MX_ERR_UNSUPPORTED, MX_ERR_HIP.
 */
mx_status mx_linear(int32_t op, const mx_qtensor *A, const mx_qtensor *B, void *C,
                    int64_t ldc, int32_t out_dtype, void *stream);

/*
 * count GEMMs of one op and one shape in a single launch (a grouped GEMM):
 *     C[i] = mx_linear(op, &A[i], &B[i])    for i < count
 * The Fprop, Dgrad or Wgrad of several linears that see their inputs at the
 * same time (the k and v projections of an attention block, which read the
 * same activations; the gate and up projections of its feed-forward layer),
 * as in mx_linear (36Kr, "Fehlerdiagnoseexperiment": the three GEMMs of every
 * linear). Small GEMMs fill the compute units together where each alone
 * would leave some idle. Each C[i] is bitwise identical to what mx_linear
 * writes for the same pair.
 *  A, B     host arrays of count descriptors, MXFP4 (E2M1) operands only.
 *           Every A[i] must have A[0]'s rows, cols and axis, every B[i]
 *           B[0]'s (else MX_ERR_SHAPE); each pair must satisfy mx_linear's
 *           rules for op.
 *  C        host array of count device pointers, each row-major [M][N] with
 *           the shared leading dimension ldc; written; no C[i] may overlap
 *           another C[j] or any operand.
 *  count    1 .. 4 (else MX_ERR_ARG).
 * Requirements and errors otherwise as for mx_linear; an MXFP8 operand gives
 * MX_ERR_UNSUPPORTED. Nothing is launched unless every entry is valid.
 */
mx_status mx_linear_batched(int32_t op, int32_t count, const mx_qtensor *A, const mx_qtensor *B,
                            void *const *C, int64_t ldc, int32_t out_dtype, void *stream);

/*
 * Dequantize a packed operand to fp32 in its source's shape [rows, cols]:
 *     out[i][j] = (-1)^sign * E(code) * 2^(s - 127)
 * with E the E2M1 value of the element's 4-bit code (E4M3 for an MXFP8
 * operand) and s the E8M0 scale of its 32-element block (36Kr, "Was ist
 * MXFP4?": one shared exponent per block; the reconstruction formula is
 * OCP MX's, the standard the pages name in "Fazit"). An axis-0 operand is
 * written back transposed into [rows, cols], so the output has the source's
 * orientation either way: the inverse of mx_quantize's encoding, up to its
 * rounding.
 *
 *  q        a descriptor filled by a quantize call; its buffers are read.
 *  out      device fp32 [rows][ld], ld >= cols (elements), 4-byte aligned;
 *           written (only the rows x cols elements). Must not overlap q's
 *           buffers. Caller-owned.
 *  stream   hipStream_t as void*.
 * A block with scale 0xFF (a NaN or Inf in the source block) gives NaN in
 * every element. Every other value is exact in fp32 while finite; values of
 * magnitude 2^128 or more (scale codes 126 and 127 only, which the
 * quantizers never write) become +-Inf. Empty operands launch nothing.
 * Errors: MX_ERR_NULL, MX_ERR_ARG, MX_ERR_SHAPE (ld < cols, or q's extents),
 * MX_ERR_ALIGN, MX_ERR_UNSUPPORTED (q's limits, or rows * ld * 4 bytes above
 * 2^62), MX_ERR_HIP.
 */
mx_status mx_dequantize(const mx_qtensor *q, float *out, int64_t ld, void *stream);

/* Static, NUL-terminated name of a status code. Never NULL. */
const char *mx_status_string(int32_t status);

/* Static, NUL-terminated library version string. */
const char *mx_version(void);

/* Name of the HIP error behind the most recent MX_ERR_HIP returned to the
 * calling thread ("hipSuccess" if there was none). Static string; never NULL. */
const char *mx_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H_ */
