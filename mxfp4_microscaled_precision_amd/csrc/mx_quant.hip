// Fused rotate + amax + E8M0 / E2M1 pack quantizer for gfx950.
//
// Per 32-element block along the reduction axis (36Kr article "Neue Studie
// von AMD durchbricht die bestehende Erkenntnis ...", sections "Was ist
// MXFP4?" and "Fehlerdiagnoseexperiment"):
//   1. widen bf16 to fp32 (exact);
//   2. random-sign option: negate x_k where Philox bit 31 of index k is set;
//   3. rotation: fp32 radix-2 butterfly, strides 1, 2, 4, 8, 16 (lower index
//      a+b, upper a-b), then one multiply by fp32(1/sqrt 32);
//   4. amax over |y| (on the fp32 bit patterns, so NaN/Inf are seen);
//   5. E8M0 exponent e = clamp(floor(log2 amax) - 2, -127, 127);
//   6. t = fp32(y * 2^-e); E2M1 magnitude by nearest-even or stochastic
//      rounding; sign bit of y;
//   7. pack two codes per byte (even index in the low nibble) and one scale
//      byte per block.
// The whole block lives in one lane's registers, so every butterfly stage is
// in-lane and the stage order above is the instruction order.
//
// Output layout is reduction-major for both axes: axis 1 writes [rows][cols/2]
// codes and [rows][cols/32] scales; axis 0 writes the transposed tensor,
// [cols][rows/2] codes and [cols][rows/32] scales, which is the operand order
// the FP4 matrix cores consume.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void fwht32(float (&y)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = y[i];
        const float b = y[i + h];
        y[i] = __fadd_rn(a, b);
        y[i + h] = __fsub_rn(a, b);
      }
    }
  }
  const float c = bits_f(kInvSqrt32Bits);
#pragma unroll
  for (int i = 0; i < 32; ++i) y[i] = __fmul_rn(y[i], c);
}

// Quantize one 32-element block held in y. For stochastic rounding the 24-bit
// uniform of element i is produced by u24_of(i). Writes 16 code bytes (as 4
// dwords) and returns the scale byte.
template <int RND, typename U24Fn>
__device__ __forceinline__ uint32_t quantize_block(const float (&y)[32], uint32_t (&out)[4],
                                                   U24Fn u24_of) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = max(amax, f_bits(y[i]) & 0x7FFFFFFFu);
  if (amax >= 0x7F800000u) {  // a NaN or Inf in the block
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = 0u;
    return 0xFFu;
  }
  const int e = block_exponent(amax);
  const float p = pow2_neg(e);
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t yb = f_bits(y[i]);
    const uint32_t ab = f_bits(__fmul_rn(y[i], p)) & 0x7FFFFFFFu;
    uint32_t mag;
    if (RND == MX_K_ROUND_SR)
      mag = e2m1_sr_mag(ab, u24_of(i));
    else
      mag = e2m1_rne_mag(ab);
    const uint32_t code = mag | ((yb >> 28) & 8u);
    out[i >> 3] |= code << (4 * (i & 7));
  }
  return (uint32_t)(e + 127);
}

__device__ __forceinline__ void apply_signs(float (&y)[32], uint32_t k0, uint32_t seed_lo) {
  // k0 is a multiple of 32: indices k0 + i, counters (k0 >> 2) + i / 4
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const U4 s = sign_words((k0 >> 2) + q, seed_lo);
    y[4 * q + 0] = bits_f(f_bits(y[4 * q + 0]) ^ (s.x & 0x80000000u));
    y[4 * q + 1] = bits_f(f_bits(y[4 * q + 1]) ^ (s.y & 0x80000000u));
    y[4 * q + 2] = bits_f(f_bits(y[4 * q + 2]) ^ (s.z & 0x80000000u));
    y[4 * q + 3] = bits_f(f_bits(y[4 * q + 3]) ^ (s.w & 0x80000000u));
  }
}

// ---------------------------------------------------------------------------
// axis = 1: blocks run along a row; one lane per block, 64 contiguous bf16
// bytes in, 16 code bytes + 1 scale byte out.
// ---------------------------------------------------------------------------
template <int ROT, int RND>
__global__ __launch_bounds__(256) void quant_axis1_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint32_t seed_lo,
    uint32_t seed_hi) {
  const int64_t nblk = cols >> 5;
  const int64_t total = rows * nblk;
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= total) return;
  const int64_t r = b / nblk;
  const int64_t kb = b - r * nblk;

  const u32x4 *src = reinterpret_cast<const u32x4 *>(x + r * ld + (kb << 5));
  u32x4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(src + j);
  float y[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t d[4] = {v[j][0], v[j][1], v[j][2], v[j][3]};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      y[8 * j + 2 * t] = bits_f(d[t] << 16);
      y[8 * j + 2 * t + 1] = bits_f(d[t] & 0xFFFF0000u);
    }
  }
  if (ROT == MX_K_ROT_RAND_SIGN) apply_signs(y, (uint32_t)(kb << 5), seed_lo);
  if (ROT != MX_K_ROT_NONE) fwht32(y);

  // stochastic rounding index L = r * cols + kb * 32 + i (cols % 32 == 0)
  const uint64_t q0 = (uint64_t)(r * cols + (kb << 5)) >> 2;
  U4 w{0u, 0u, 0u, 0u};
  auto u24_of = [&](int i) -> uint32_t {
    if ((i & 3) == 0) w = sr_words(q0 + (uint64_t)(i >> 2), seed_lo, seed_hi);
    return pick_word(w, (uint32_t)(i & 3)) >> 8;
  };
  uint32_t out[4];
  const uint32_t s = quantize_block<RND>(y, out, u24_of);
  *reinterpret_cast<uint4 *>(codes + r * (cols >> 1) + (kb << 4)) =
      make_uint4(out[0], out[1], out[2], out[3]);
  scales[r * nblk + kb] = (uint8_t)s;
}

// ---------------------------------------------------------------------------
// axis = 0: blocks run down a column. A lane owns a column pair (c0, c0 + 1)
// and walks `rb` consecutive 32-row blocks; each row is one coalesced 4-byte
// load per lane (256 contiguous bytes per wave). Output is transposed:
// codes [cols][rows/2], scales [cols][rows/32].
// ---------------------------------------------------------------------------
template <int ROT, int RND>
__global__ __launch_bounds__(256) void quant_axis0_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint32_t seed_lo,
    uint32_t seed_hi, int rb, int pair_loads) {
  const int64_t cp = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t c0 = cp * 2;
  if (c0 >= cols) return;
  const bool two = (c0 + 1) < cols;
  const int64_t nkb = rows >> 5;
  const int64_t kb_begin = (int64_t)blockIdx.y * rb;
  const int64_t kb_end = min(nkb, kb_begin + rb);
  const int64_t code_ld = rows >> 1;

  for (int64_t kb = kb_begin; kb < kb_end; ++kb) {
    float ya[32], yb[32];
    const uint16_t *src = x + (kb << 5) * ld + c0;
    if (two && pair_loads) {   // rows 4-byte aligned: one load per column pair
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t d = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t *>(src + (int64_t)i * ld));
        ya[i] = bits_f(d << 16);
        yb[i] = bits_f(d & 0xFFFF0000u);
      }
    } else if (two) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        ya[i] = bits_f((uint32_t)src[(int64_t)i * ld] << 16);
        yb[i] = bits_f((uint32_t)src[(int64_t)i * ld + 1] << 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        ya[i] = bits_f((uint32_t)src[(int64_t)i * ld] << 16);
        yb[i] = 0.0f;
      }
    }
    if (ROT == MX_K_ROT_RAND_SIGN) {
      apply_signs(ya, (uint32_t)(kb << 5), seed_lo);
      apply_signs(yb, (uint32_t)(kb << 5), seed_lo);
    }
    if (ROT != MX_K_ROT_NONE) {
      fwht32(ya);
      fwht32(yb);
    }
    // stochastic rounding: element (row, c) has L = row * cols + c
    const int64_t row0 = kb << 5;
    auto u24_a = [&](int i) -> uint32_t {
      const uint64_t L = (uint64_t)((row0 + i) * cols + c0);
      const U4 w = sr_words(L >> 2, seed_lo, seed_hi);
      return pick_word(w, (uint32_t)(L & 3)) >> 8;
    };
    auto u24_b = [&](int i) -> uint32_t {
      const uint64_t L = (uint64_t)((row0 + i) * cols + c0 + 1);
      const U4 w = sr_words(L >> 2, seed_lo, seed_hi);
      return pick_word(w, (uint32_t)(L & 3)) >> 8;
    };
    uint32_t oa[4], ob[4];
    const uint32_t sa = quantize_block<RND>(ya, oa, u24_a);
    *reinterpret_cast<uint4 *>(codes + c0 * code_ld + (kb << 4)) =
        make_uint4(oa[0], oa[1], oa[2], oa[3]);
    scales[c0 * nkb + kb] = (uint8_t)sa;
    if (two) {
      const uint32_t sb = quantize_block<RND>(yb, ob, u24_b);
      *reinterpret_cast<uint4 *>(codes + (c0 + 1) * code_ld + (kb << 4)) =
          make_uint4(ob[0], ob[1], ob[2], ob[3]);
      scales[(c0 + 1) * nkb + kb] = (uint8_t)sb;
    }
  }
}

template <int ROT, int RND>
hipError_t launch_quant(const QuantArgs &a, hipStream_t stream) {
  if (a.axis == 1) {
    const int64_t total = a.rows * (a.cols >> 5);
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    return launch(quant_axis1_kernel<ROT, RND>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                  a.x, a.rows, a.cols, a.ld, a.codes, a.scales, a.seed_lo, a.seed_hi);
  } else {
    const int threads = 256;
    const int64_t pairs = (a.cols + 1) >> 1;
    const int64_t gx = (pairs + threads - 1) / threads;
    const int64_t nkb = a.rows >> 5;
    const int rb = a.rb > 0 ? a.rb : 4;
    const int64_t gy = (nkb + rb - 1) / rb;
    const int pair_loads =
        (a.ld % 2 == 0) && (reinterpret_cast<uintptr_t>(a.x) % 4 == 0) ? 1 : 0;
    return launch(quant_axis0_kernel<ROT, RND>, dim3((unsigned)gx, (unsigned)gy), dim3(threads),
                  0, stream, a.x, a.rows, a.cols, a.ld, a.codes, a.scales, a.seed_lo, a.seed_hi,
                  rb, pair_loads);
  }
}

}  // namespace

hipError_t quantize_launch(const QuantArgs &a, hipStream_t stream) {
  switch (a.rotate * 2 + a.round) {
    case 0: return launch_quant<0, 0>(a, stream);
    case 1: return launch_quant<0, 1>(a, stream);
    case 2: return launch_quant<1, 0>(a, stream);
    case 3: return launch_quant<1, 1>(a, stream);
    case 4: return launch_quant<2, 0>(a, stream);
    case 5: return launch_quant<2, 1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mx
