// Fused rotate + amax + E8M0 / E2M1 pack quantizer for gfx950.
//
// Per 32-element block along the reduction axis (36Kr article "Neue Studie
// von AMD durchbricht die bestehende Erkenntnis ...", sections "Was ist
// MXFP4?" and "Fehlerdiagnoseexperiment"):
//   1. widen bf16 to fp32 (exact);
//   2. random-sign option: negate x_k where Philox bit 31 of index k is set;
//   3. rotation: fp32 radix-2 butterfly, strides 1, 2, 4, 8, 16 (lower index
//      a+b, upper a-b), then one multiply by fp32(1/sqrt 32) (folded into
//      the scale multiply where that is bit-identical, see quantize_block);
//   4. amax over |y| (on the fp32 bit patterns, so NaN/Inf are seen);
//   5. E8M0 exponent e = clamp(floor(log2 amax) - 2, -127, 127);
//   6. t = fp32(y * 2^-e); E2M1 magnitude by nearest-even or stochastic
//      rounding; sign bit of y;
//   7. pack two codes per byte (even index in the low nibble) and one scale
//      byte per block.
// The whole block lives in one lane's registers, so every butterfly stage is
// in-lane and the stage order above is the instruction order.
//
// Output layout is the tiled, reduction-major operand layout the GEMM streams
// (see below); axis 0 writes the transposed tensor, so both GEMM operands are
// always reduction-major.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Unnormalised butterfly: h = H32 x in fp32, strides 1, 2, 4, 8, 16, lower
// index a + b, upper a - b. The normalisation y = fl32(h * c) is folded into
// the scale multiply of quantize_block.
__device__ __forceinline__ void butterfly32(float (&y)[32]) {
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
}

// The 16-point variant: two independent butterflies (strides 1, 2, 4, 8) on
// elements 0..15 and 16..31; its normalisation 1/4 is applied like c below.
__device__ __forceinline__ void butterfly16x2(float (&y)[32]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
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
}

typedef short v2i16 __attribute__((ext_vector_type(2)));

// |t| clamped to 448, E4M3's largest finite value (one v_med3_f32).
__device__ __forceinline__ float sat448(float t) {
  return __builtin_amdgcn_fmed3f(t, -448.0f, 448.0f);
}

// Element formats: the E2M1 elements of MXFP4, and the E4M3 elements of the
// MXFP8 comparator (same 32-element blocks and E8M0 scales; one code byte per
// element; nearest-even rounding only).
constexpr int kFmtE2M1 = 0;
constexpr int kFmtE4M3 = 1;

// Rotation kind of the encoder: 0 none, 1 the 32-point Hadamard (with or
// without random signs), 2 the 16-point variant.
template <int ROT>
struct RotKind {
  static constexpr int value = ROT == MX_K_ROT_NONE ? 0 : (ROT == MX_K_ROT_HADAMARD16 ? 2 : 1);
};

template <int ROT>
__device__ __forceinline__ void rotate_block(float (&y)[32]) {
  if (ROT == MX_K_ROT_HADAMARD16)
    butterfly16x2(y);
  else if (ROT != MX_K_ROT_NONE)
    butterfly32(y);
}

// Normalisation of the rotation: fp32(1/sqrt 32), or 1/4 for the 16-point
// variant.
template <int RK>
__device__ __forceinline__ float rot_norm() {
  return RK == 2 ? 0.25f : bits_f(kInvSqrt32Bits);
}

// Quantize one 32-element block. v holds the butterfly output h (RK != 0) or
// the input x (RK == 0). The rotated value is y = fl32(h * c) with c the
// normalisation (rot_norm).
//
//  * amax: max |y| = fl32(max |h| * c), since rounding is monotonic; a NaN
//    or Inf anywhere in the block marks it (see the amax comment below).
//  * scale: e from amax; t = fl32(y * 2^-e). Stochastic rounding reads
//    every bit of t, so it takes the two multiplies as written. For nearest
//    rounding with e <= 123, c_e = c * 2^-e is an exact normal fp32 number
//    and t = fl32(h * c_e) gives the same code as fl32(y * 2^-e): a
//    power-of-two scaling commutes with rounding unless y or t is subnormal.
//    A subnormal t encodes as a signed zero either way. A subnormal y needs
//    |h| < 2^-123.5, and h is then n * 2^-133 with n < 724 (bf16's finest
//    step; butterfly sums of such values are exact); no such n * c comes
//    within fp32 rounding distance of a decision threshold times 2^e (the
//    thresholds are multiples of 2^-10: it would need |16 c n - j| < 2^-13
//    for an integer j, and over n < 724 the closest approach is 8.8e-4, at
//    n = 204).
//    For e > 123 the two multiplies are done as written.
//  * RNE: v_cvt_scalef32_pk_fp4_f32 at scale 1.0, which rounds to nearest
//    even and saturates at +-6 exactly like the threshold rule (checked over
//    every fp32 pattern); two elements per instruction, element 2j in the low
//    nibble. SR: integer rule of e2m1_sr_mag with the Philox uniform. E4M3
//    (nearest only): the hardware fp8 convert behind a clamp to +-448, one
//    code byte per element.
template <int RK, int RND, int FMT, typename U24Fn>
__device__ __forceinline__ uint32_t quantize_block(const float (&v)[32],
                                                   uint32_t (&out)[FMT == kFmtE4M3 ? 8 : 4],
                                                   U24Fn u24_of) {
  constexpr int kWords = FMT == kFmtE4M3 ? 8 : 4;
  // amax as bits of |v| (a NaN or Inf compares above 0x7f800000). Without
  // the 32-point rotation: integer max of |bits|, which sees a lone NaN (the
  // 16-point variant leaves one half finite when the other holds a NaN).
  // With it every output of a block holding a NaN or Inf is itself NaN or
  // Inf, so the float max of |v| (which skips NaN operands) still lands above
  // 0x7f800000 for such blocks and equals the integer max for the others.
  uint32_t amax = 0;
  if (RK != 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = max(amax, f_bits(v[i]) & 0x7FFFFFFFu);
  } else {
    float m = fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 31; i += 2) m = fmaxf(fmaxf(m, fabsf(v[i])), fabsf(v[i + 1]));
    amax = f_bits(fmaxf(m, fabsf(v[31])));
  }
  const bool nonfinite = amax >= 0x7F800000u;
  const float c = rot_norm<RK>();
  if (RK) amax = f_bits(__fmul_rn(bits_f(amax), c));
  // E4M3's largest exponent is 8 where E2M1's is 2: six more below the amax
  const int e = FMT == kFmtE4M3 ? max(block_exponent(amax) - 6, -127) : block_exponent(amax);
  float t[32];
  if (!RK) {
    const float p = pow2_neg(e);
#pragma unroll
    for (int i = 0; i < 32; ++i) t[i] = __fmul_rn(v[i], p);
  } else if (RND == MX_K_ROUND_SR) {
    const float p = pow2_neg(e);
#pragma unroll
    for (int i = 0; i < 32; ++i) t[i] = __fmul_rn(__fmul_rn(v[i], c), p);
  } else {
    // c * 2^-e is an exact normal number for e <= 123: one multiply gives
    // the bits of fl32(fl32(h * c) * 2^-e). If some lane of the wave has
    // |y| >= 2^126 (e > 123), the wave multiplies twice: such a lane by c,
    // then by 2^-e, as written; the other lanes by c_e, then by 1, which
    // changes nothing. The first multiply overwrites a copy of v in place,
    // so only one array of 32 is live (a separate array for each case cost
    // 26 more registers in the dual kernel and one wave per SIMD).
    const float ce = __fmul_rn(c, pow2_neg(min(e, 123)));
    float h[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) h[i] = v[i];
    float mult = ce;
    if (__builtin_expect(__any(e > 123), 0)) {
      const float m1 = e > 123 ? c : ce;
      mult = e > 123 ? pow2_neg(e) : 1.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) h[i] = __fmul_rn(h[i], m1);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) t[i] = __fmul_rn(h[i], mult);
  }
  if constexpr (FMT == kFmtE4M3) {
    // v_cvt_scalef32_pk_fp8_f32 at scale 1.0 rounds to the nearest E4M3
    // value, ties to even, exactly like the integer rule below 464 (checked
    // over every fp32 value of magnitude below 512) but turns larger
    // magnitudes into NaN; the med3 clamp to +-448 makes it saturate.
    // Element 4j + i goes to byte i of word j.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v2i16 w = {0, 0};
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, sat448(t[4 * j]), sat448(t[4 * j + 1]),
                                                   1.0f, false);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, sat448(t[4 * j + 2]),
                                                   sat448(t[4 * j + 3]), 1.0f, true);
      out[j] = (uint32_t)(uint16_t)w[0] | ((uint32_t)(uint16_t)w[1] << 16);
    }
  } else if (RND == MX_K_ROUND_SR) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t tb = f_bits(t[i]);
      const uint32_t code = e2m1_sr_mag(tb & 0x7FFFFFFFu, u24_of(i)) | ((tb >> 28) & 8u);
      out[i >> 3] |= code << (4 * (i & 7));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0u;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[8 * j + 0], t[8 * j + 1], 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[8 * j + 2], t[8 * j + 3], 1.0f, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[8 * j + 4], t[8 * j + 5], 1.0f, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[8 * j + 6], t[8 * j + 7], 1.0f, 3);
      out[j] = w;
    }
  }
  if (nonfinite) {
#pragma unroll
    for (int j = 0; j < kWords; ++j) out[j] = 0u;
    return 0xFFu;
  }
  return (uint32_t)(e + 127);
}

// Scale of one block for stochastic rounding, t = fl32(fl32(v * m1) * m2):
// m1 = c, m2 = 2^-e with rotation (the two roundings as defined, see
// quantize_block); m1 = 2^-e, m2 = 1 without. Returns the scale code (0xFF
// for a block holding a NaN or Inf, detected as in quantize_block).
template <int RK>
__device__ __forceinline__ uint32_t block_scale(const float (&v)[32], float &m1, float &m2) {
  uint32_t amax = 0;
  if (RK != 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = max(amax, f_bits(v[i]) & 0x7FFFFFFFu);
  } else {
    float m = fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 31; i += 2) m = fmaxf(fmaxf(m, fabsf(v[i])), fabsf(v[i + 1]));
    amax = f_bits(fmaxf(m, fabsf(v[31])));
  }
  const bool nonfinite = amax >= 0x7F800000u;
  const float c = rot_norm<RK>();
  if (RK) amax = f_bits(__fmul_rn(bits_f(amax), c));
  const int e = block_exponent(amax);
  if (!RK) {
    m1 = pow2_neg(e);
    m2 = 1.0f;
  } else {
    m1 = c;
    m2 = pow2_neg(e);
  }
  return nonfinite ? 0xFFu : (uint32_t)(e + 127);
}

// Stochastic rounding of a column pair (c0, c0 + 1) of the axis-0 path. The
// elements of row i have source indices L = L0 + i * cols and L + 1, which
// one Philox call covers unless L % 4 == 3.
template <int RK>
__device__ __forceinline__ void quantize_pair_sr(const float (&va)[32], const float (&vb)[32],
                                                 uint32_t (&oa)[4], uint32_t (&ob)[4],
                                                 uint32_t &sa, uint32_t &sb, uint64_t L0,
                                                 int64_t cols, uint32_t seed_lo,
                                                 uint32_t seed_hi) {
  float m1a, m2a, m1b, m2b;
  sa = block_scale<RK>(va, m1a, m2a);
  sb = block_scale<RK>(vb, m1b, m2b);
#pragma unroll
  for (int j = 0; j < 4; ++j) oa[j] = ob[j] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint64_t L = L0 + (uint64_t)i * (uint64_t)cols;
    const U4 w = sr_words(L >> 2, seed_lo, seed_hi);
    const uint32_t j = (uint32_t)(L & 3);
    const uint32_t ua = pick_word(w, j) >> 8;
    uint32_t ub;
    if (j == 3) {
      ub = sr_words((L >> 2) + 1, seed_lo, seed_hi).x >> 8;
    } else {
      ub = pick_word(w, j + 1) >> 8;
    }
    const uint32_t ta = f_bits(__fmul_rn(__fmul_rn(va[i], m1a), m2a));
    const uint32_t tb = f_bits(__fmul_rn(__fmul_rn(vb[i], m1b), m2b));
    oa[i >> 3] |= (e2m1_sr_mag(ta & 0x7FFFFFFFu, ua) | ((ta >> 28) & 8u)) << (4 * (i & 7));
    ob[i >> 3] |= (e2m1_sr_mag(tb & 0x7FFFFFFFu, ub) | ((tb >> 28) & 8u)) << (4 * (i & 7));
  }
  if (sa == 0xFFu) {
#pragma unroll
    for (int j = 0; j < 4; ++j) oa[j] = 0u;
  }
  if (sb == 0xFFu) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ob[j] = 0u;
  }
}

// Sign bits of K indices 4 ctr .. 4 ctr + 3 as a nibble (bit j for index
// 4 ctr + j), from one Philox call of the sign stream.
__device__ __forceinline__ uint32_t sign_nibble(uint32_t ctr, uint32_t seed_lo) {
  const U4 sw = sign_words(ctr, seed_lo);
  return (sw.x >> 31) | ((sw.y >> 31) << 1) | ((sw.z >> 31) << 2) | ((sw.w >> 31) << 3);
}

// The 32 sign bits whose nibbles lanes base .. base + 7 of the wave hold
// (bit i for element i of the block).
__device__ __forceinline__ uint32_t gather_sign_mask(uint32_t nib, int base) {
  uint32_t mask = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) mask |= (uint32_t)__builtin_amdgcn_readlane((int)nib, base + j) << (4 * j);
  return mask;
}

__device__ __forceinline__ void apply_sign_mask(float (&y)[32], uint32_t mask) {
#pragma unroll
  for (int i = 0; i < 32; ++i) y[i] = bits_f(f_bits(y[i]) ^ ((mask << (31 - i)) & 0x80000000u));
}

// ---------------------------------------------------------------------------
// Output layout (tiled, see mx_qtensor in mxfp4.h): the operand is viewed
// reduction-major, [MN, K], zero-padded to [MNp, Kp] (MNp multiple of 256, Kp
// of 128). Codes: tile (g, q) = rows 16g.., K elements 128q.. is 1 KB at
// (g * Kp/128 + q) * 1024, block c of row r at c * 256 + r * 16 inside it.
// Scales: [Kp/128][MNp/256][4][4][16][4], the scale of row 256T + 16h + r,
// block 4q + c at (q * MNp/256 + T) * 1024 + (h / 4) * 256 + c * 64 + r * 4 +
// h % 4. Padding positions hold the encoding of zeros (codes 0, scale code 0).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t code_offset(int64_t mn, int64_t kb, int64_t nslices) {
  return ((mn >> 4) * nslices + (kb >> 2)) * 1024 + (kb & 3) * 256 + (mn & 15) * 16;
}
// E4M3 codes (one byte per element): tile (g, q) is 2 KB at
// (g * Kp/128 + q) * 2048; inside it the 16-element chunk j of row r is the
// 16 bytes at j * 256 + r * 16. Block kb of row mn is chunks 2 (kb % 4) and
// 2 (kb % 4) + 1; this returns the first one's address (the second is 256
// bytes on).
__device__ __forceinline__ int64_t code_offset_e4m3(int64_t mn, int64_t kb, int64_t nslices) {
  return ((mn >> 4) * nslices + (kb >> 2)) * 2048 + (kb & 3) * 512 + (mn & 15) * 16;
}
__device__ __forceinline__ int64_t scale_offset(int64_t mn, int64_t kb, int64_t mnp) {
  const int64_t h = (mn >> 4) & 15;
  return ((kb >> 2) * (mnp >> 8) + (mn >> 8)) * 1024 + (h >> 2) * 256 + (kb & 3) * 64 +
         (mn & 15) * 4 + (h & 3);
}

// ---------------------------------------------------------------------------
// axis = 1 (blocks run along a source row): each wave encodes one output tile
// (16 rows x 128 K elements), four tiles per workgroup, one launch covering
// every tile. The tile's 4 KB of bf16 is read with each load instruction
// covering four whole 256-byte row pieces (all four in flight at once),
// staged in LDS, and lane l then takes row (l & 15), block (l >> 4): 64
// bytes in, 16 code bytes out at tile + 16 l (the wave writes its 1 KB tile
// in one go). LDS holds row r's 16-byte chunk ch at r * 256 + (ch ^ r) * 16,
// so both the staging writes and the per-lane reads hit 16 distinct chunk
// positions per 16 lanes.
// At most 85 registers (6 waves per SIMD); the nearest-rounding instances
// need 53-55, so up to 8 waves per SIMD cover each other's loads. This was
// 3-9% faster than a persistent grid of 12 waves per compute unit that kept
// the next tile's loads in flight in registers (88 registers), and 5-9%
// faster with stochastic rounding than a bound of 8 waves (bitwise
// identical).
// ---------------------------------------------------------------------------

// The second operand of a two-operand launch (PAIR): a source with the same
// column count whose row groups follow the first operand's in one sequence
// of tiles.
struct Axis1Second {
  const uint16_t *x;
  int64_t rows, ld;
  uint8_t *codes, *scales;
  uint32_t seed_lo, seed_hi;
};

template <int ROT, int RND, int FMT, bool PAIR>
__global__ __launch_bounds__(256, 6) void quant_axis1_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint32_t seed_lo,
    uint32_t seed_hi, Axis1Second sec) {
  static_assert(!PAIR || FMT == kFmtE2M1, "two-operand launches are MXFP4 only");
  __shared__ __attribute__((aligned(16))) uint8_t stage[4][4096];
  __shared__ __attribute__((aligned(16))) uint8_t signs_lds[ROT == MX_K_ROT_RAND_SIGN ? 4 : 1][128];
  const int64_t mnp = (rows + 255) & ~(int64_t)255;
  const int64_t mnp2 = PAIR ? (sec.rows + 255) & ~(int64_t)255 : 0;
  const uint32_t gsplit = (uint32_t)(mnp >> 4);   // row groups of the first operand
  // Tile counts fit 32 bits: the host refuses operands of 1 GiB of codes.
  const uint32_t nslices = (uint32_t)((cols + 127) >> 7);
  const uint32_t ntiles = (gsplit + (uint32_t)(mnp2 >> 4)) * nslices;
  const int wv = threadIdx.x >> 6;
  const uint32_t tile = blockIdx.x * 4u + (uint32_t)wv;
  if (tile >= ntiles) return;
  const int lane = threadIdx.x & 63;
  uint8_t *st = stage[wv];
  const int ch = lane & 15;
  const uint32_t g = tile / nslices, q = tile - g * nslices;   // (row group, K slice)
  const bool two = PAIR && g >= gsplit;                         // the second operand's tile
  const uint32_t gl = two ? g - gsplit : g;
  {
    // instruction j reads rows 4j .. 4j + 3, 16 lanes per row. Rows and
    // columns past the source are read from its last row / last chunk: only
    // padding blocks use them (cols % 32 == 0, so a 32-block is all inside or
    // all padding) and those are written as zeros below. Unconditional loads
    // keep all four in flight; with a branch around each, the compiler
    // waited for the first two before issuing the other two.
    const uint16_t *xs = two ? sec.x : x;
    const int64_t rs = two ? sec.rows : rows, ls = two ? sec.ld : ld;
    const int64_t k = min((int64_t)q * 128 + ch * 8, cols - 8);   // first element of the chunk
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = j * 4 + (lane >> 4);
      const int64_t r = min((int64_t)gl * 16 + rr, rs - 1);
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xs + r * ls + k));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = j * 4 + (lane >> 4);
      *reinterpret_cast<u32x4 *>(st + rr * 256 + ((ch ^ rr) << 4)) = v[j];
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int rr = lane & 15, cb = lane >> 4;
  const uint32_t s_lo = two ? sec.seed_lo : seed_lo, s_hi = two ? sec.seed_hi : seed_hi;
  const int64_t r = (int64_t)gl * 16 + rr;
  const int64_t kb = (int64_t)q * 4 + cb;
  const bool valid = r < (two ? sec.rows : rows) && (kb << 5) < cols;
  float y[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 d = *reinterpret_cast<const u32x4 *>(st + rr * 256 + (((cb * 4 + j) ^ rr) << 4));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      y[8 * j + 2 * t] = bits_f(d[t] << 16);
      y[8 * j + 2 * t + 1] = bits_f(d[t] & 0xFFFF0000u);
    }
  }
  if (ROT == MX_K_ROT_RAND_SIGN) {
    // the tile's 128 reduction indices need 32 Philox calls: lanes 0..31
    // make one each, the sign bits meet in LDS as one nibble per call
    uint32_t *sg = reinterpret_cast<uint32_t *>(signs_lds[wv]);
    if (lane < 32) {
      const U4 sw = sign_words((uint32_t)(q * 32 + lane), s_lo);
      sg[lane] = (sw.x >> 31) | ((sw.y >> 31) << 1) | ((sw.z >> 31) << 2) | ((sw.w >> 31) << 3);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t mask = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) mask |= sg[cb * 8 + j] << (4 * j);
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = bits_f(f_bits(y[i]) ^ ((mask << (31 - i)) & 0x80000000u));
  }
  rotate_block<ROT>(y);
  // stochastic rounding index L = r * cols + kb * 32 + i (cols % 32 == 0)
  const uint64_t q0 = (uint64_t)(r * cols + (kb << 5)) >> 2;
  U4 w{0u, 0u, 0u, 0u};
  auto u24_of = [&](int i) -> uint32_t {
    if ((i & 3) == 0) w = sr_words(q0 + (uint64_t)(i >> 2), s_lo, s_hi);
    return pick_word(w, (uint32_t)(i & 3)) >> 8;
  };
  constexpr int kWords = FMT == kFmtE4M3 ? 8 : 4;
  uint32_t out[kWords];
  uint32_t s = quantize_block<RotKind<ROT>::value, RND, FMT>(y, out, u24_of);
  if (!valid) {                                           // padding: zero codes, scale code 0
#pragma unroll
    for (int j = 0; j < kWords; ++j) out[j] = 0u;
    s = 0u;
  }
  if constexpr (FMT == kFmtE4M3) {  // block cb of row rr: chunks 2 cb and 2 cb + 1
    uint8_t *tp = codes + (size_t)tile * 2048 + cb * 512 + rr * 16;
    *reinterpret_cast<uint4 *>(tp) = make_uint4(out[0], out[1], out[2], out[3]);
    *reinterpret_cast<uint4 *>(tp + 256) = make_uint4(out[4], out[5], out[6], out[7]);
  } else {
    const uint32_t lt = PAIR ? gl * nslices + q : tile;     // tile within its operand
    *reinterpret_cast<uint4 *>((two ? sec.codes : codes) + (size_t)lt * 1024 + lane * 16) =
        make_uint4(out[0], out[1], out[2], out[3]);
  }
  (two ? sec.scales : scales)[scale_offset(r, kb, two ? mnp2 : mnp)] = (uint8_t)s;
}

// ---------------------------------------------------------------------------
// axis = 0 with nearest rounding: one source column (one operand row) per
// lane and one 32-row block per workgroup row. Each source row is a 2-byte
// load per lane, 128 contiguous bytes per wave, all 32 in flight; sixteen
// lanes cover the 16 operand rows of one tile, so each store instruction
// writes whole 256-byte block rows of four tiles. At most 64 registers (8
// waves per SIMD; the instances need 46-56): against the column-pair kernel
// below (a lane encoding two blocks, 81-99 registers, 5 waves per SIMD) it
// was 3-12% faster with H32 and 16-18% with random signs, bitwise identical.
// ---------------------------------------------------------------------------
template <int ROT, int FMT>
__global__ __launch_bounds__(256, 8) void quant_axis0_rne_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint32_t seed_lo) {
  const int64_t mnp = (cols + 255) & ~(int64_t)255;
  const int64_t nslices = (rows + 127) >> 7;
  const int64_t nkb = rows >> 5;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;   // < mnp (grid)
  const int64_t kb = blockIdx.y;                                // < 4 nslices (grid)
  constexpr int kWords = FMT == kFmtE4M3 ? 8 : 4;
  uint32_t o[kWords];
#pragma unroll
  for (int j = 0; j < kWords; ++j) o[j] = 0u;
  uint32_t s = 0u;                                  // padding: zero codes, scale code 0
  // random signs: the block's 32 rows need the 8 sign calls at counters
  // 8 kb + j, the same for every column; lane j makes call j and the bits
  // are gathered with readlane, before any lane of the wave branches off
  uint32_t smask = 0u;
  if (ROT == MX_K_ROT_RAND_SIGN)
    smask = gather_sign_mask(sign_nibble((uint32_t)((kb << 3) + (threadIdx.x & 7)), seed_lo), 0);
  if (kb < nkb && c < cols) {
    float y[32];
    const uint16_t *src = x + (kb << 5) * ld + c;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      y[i] = bits_f((uint32_t)__builtin_nontemporal_load(src + (int64_t)i * ld) << 16);
    if (ROT == MX_K_ROT_RAND_SIGN) apply_sign_mask(y, smask);
    rotate_block<ROT>(y);
    auto u24_of = [](int) -> uint32_t { return 0u; };   // nearest rounding draws nothing
    s = quantize_block<RotKind<ROT>::value, MX_K_ROUND_RNE, FMT>(y, o, u24_of);
  }
  if constexpr (FMT == kFmtE4M3) {
    uint8_t *p = codes + code_offset_e4m3(c, kb, nslices);
    *reinterpret_cast<uint4 *>(p) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4 *>(p + 256) = make_uint4(o[4], o[5], o[6], o[7]);
  } else {
    *reinterpret_cast<uint4 *>(codes + code_offset(c, kb, nslices)) =
        make_uint4(o[0], o[1], o[2], o[3]);
  }
  scales[scale_offset(c, kb, mnp)] = (uint8_t)s;
}

// ---------------------------------------------------------------------------
// axis = 0 (blocks run down a source column; the output is the transposed
// operand), stochastic rounding with cols % 4 != 0 (nearest rounding takes
// quant_axis0_rne_kernel above): a lane owns a column pair (c0, c0 + 1) = operand rows, and walks
// `rb` consecutive 32-row blocks; each source row is one coalesced 4-byte
// load per lane (256 contiguous bytes per wave). Eight lanes cover the 16
// operand rows of one tile, so each store instruction writes whole 256-byte
// block rows of eight tiles.
// ---------------------------------------------------------------------------
template <int ROT, int RND, int FMT>
__global__ __launch_bounds__(256) void quant_axis0_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint32_t seed_lo,
    uint32_t seed_hi, int rb, int pair_loads) {
  const int64_t mnp = (cols + 255) & ~(int64_t)255;
  const int64_t nslices = (rows + 127) >> 7;
  const int64_t nkb_pad = nslices * 4;
  const int64_t nkb = rows >> 5;
  const int64_t cp = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t c0 = cp * 2;
  if (c0 >= mnp) return;
  const bool has_a = c0 < cols;
  const bool has_b = (c0 + 1) < cols;
  const int64_t kb_begin = (int64_t)blockIdx.y * rb;
  const int64_t kb_end = min(nkb_pad, kb_begin + rb);

  constexpr int kWords = FMT == kFmtE4M3 ? 8 : 4;
  for (int64_t kb = kb_begin; kb < kb_end; ++kb) {
    uint32_t oa[kWords], ob[kWords];
#pragma unroll
    for (int j = 0; j < kWords; ++j) oa[j] = ob[j] = 0u;
    uint32_t sa = 0u, sb = 0u;                     // padding: zero codes, scale code 0
    // random signs: the block's 32 rows need the 8 sign calls at counters
    // 8 kb + j, the same for every column; lane j makes call j and the bits
    // are gathered with readlane, before any lane of the wave branches off
    uint32_t smask = 0u;
    if (ROT == MX_K_ROT_RAND_SIGN)
      smask = gather_sign_mask(sign_nibble((uint32_t)((kb << 3) + (threadIdx.x & 7)), seed_lo), 0);
    if (kb < nkb && has_a) {
      float ya[32], yb[32];
      const uint16_t *src = x + (kb << 5) * ld + c0;
      if (has_b && pair_loads) {   // rows 4-byte aligned: one load per column pair
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t d = __builtin_nontemporal_load(
              reinterpret_cast<const uint32_t *>(src + (int64_t)i * ld));
          ya[i] = bits_f(d << 16);
          yb[i] = bits_f(d & 0xFFFF0000u);
        }
      } else if (has_b) {
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
        apply_sign_mask(ya, smask);
        apply_sign_mask(yb, smask);
      }
      rotate_block<ROT>(ya);
      rotate_block<ROT>(yb);
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
      if constexpr (RND == MX_K_ROUND_SR && FMT == kFmtE2M1) {
        quantize_pair_sr<RotKind<ROT>::value>(ya, yb, oa, ob, sa, sb,
                                               (uint64_t)(row0 * cols + c0), cols, seed_lo,
                                               seed_hi);
        if (!has_b) {
#pragma unroll
          for (int j = 0; j < 4; ++j) ob[j] = 0u;
          sb = 0u;
        }
      } else {
        sa = quantize_block<RotKind<ROT>::value, RND, FMT>(ya, oa, u24_a);
        if (has_b) sb = quantize_block<RotKind<ROT>::value, RND, FMT>(yb, ob, u24_b);
      }
    }
    if constexpr (FMT == kFmtE4M3) {
      uint8_t *pa = codes + code_offset_e4m3(c0, kb, nslices);
      uint8_t *pb = codes + code_offset_e4m3(c0 + 1, kb, nslices);
      *reinterpret_cast<uint4 *>(pa) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
      *reinterpret_cast<uint4 *>(pa + 256) = make_uint4(oa[4], oa[5], oa[6], oa[7]);
      *reinterpret_cast<uint4 *>(pb) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
      *reinterpret_cast<uint4 *>(pb + 256) = make_uint4(ob[4], ob[5], ob[6], ob[7]);
    } else {
      *reinterpret_cast<uint4 *>(codes + code_offset(c0, kb, nslices)) =
          make_uint4(oa[0], oa[1], oa[2], oa[3]);
      *reinterpret_cast<uint4 *>(codes + code_offset(c0 + 1, kb, nslices)) =
          make_uint4(ob[0], ob[1], ob[2], ob[3]);
    }
    scales[scale_offset(c0, kb, mnp)] = (uint8_t)sa;
    scales[scale_offset(c0 + 1, kb, mnp)] = (uint8_t)sb;
  }
}

// ---------------------------------------------------------------------------
// axis = 0 with stochastic rounding and cols % 4 == 0: a lane owns one source
// column (one operand row) and walks `rb` 32-row blocks. Element (row, c)
// draws word L % 4 of Philox call L / 4, L = row * cols + c, so the four
// words of a call are columns 4m .. 4m + 3 of one row: the four lanes of a
// quad. Each lane of a quad makes the call for one row of every group of four
// rows, and three DPP exchanges (a 4 x 4 transpose) hand every lane the words
// of its own column: 8 calls per lane per block instead of 32. Random signs
// (one per row, the same for every column) come from one call per lane,
// lanes 0..7 covering the block's 32 rows, read back with readlane. The grid
// covers MNp exactly, so every lane of a wave is live for the exchanges.
// ---------------------------------------------------------------------------
template <int ROT>
__global__ __launch_bounds__(256) void quant_axis0_sr_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint32_t seed_lo,
    uint32_t seed_hi, int rb) {
  constexpr int RK = RotKind<ROT>::value;
  const int64_t mnp = (cols + 255) & ~(int64_t)255;
  const int64_t nslices = (rows + 127) >> 7;
  const int64_t nkb_pad = nslices * 4;
  const int64_t nkb = rows >> 5;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool present = c < cols;                    // quads are all present or all padding
  const int lane = threadIdx.x & 63;
  const uint32_t q = threadIdx.x & 3;               // lane within its quad
  const int64_t kb_begin = (int64_t)blockIdx.y * rb;
  const int64_t kb_end = min(nkb_pad, kb_begin + rb);
  for (int64_t kb = kb_begin; kb < kb_end; ++kb) {
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    uint32_t s = 0u;                                // padding: zero codes, scale code 0
    if (kb < nkb) {
      const int64_t row0 = kb << 5;
      float y[32];
      if (present) {
        const uint16_t *src = x + row0 * ld + c;
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] = bits_f((uint32_t)src[(int64_t)i * ld] << 16);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] = 0.0f;
      }
      if (ROT == MX_K_ROT_RAND_SIGN) {
        const U4 sw = sign_words((uint32_t)((row0 >> 2) + (lane & 7)), seed_lo);
        const uint32_t nib =
            (sw.x >> 31) | ((sw.y >> 31) << 1) | ((sw.z >> 31) << 2) | ((sw.w >> 31) << 3);
        uint32_t mask = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          mask |= (uint32_t)__builtin_amdgcn_readlane((int)nib, j) << (4 * j);
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] = bits_f(f_bits(y[i]) ^ ((mask << (31 - i)) & 0x80000000u));
      }
      rotate_block<ROT>(y);
      float m1, m2;
      s = block_scale<RK>(y, m1, m2);
      const uint64_t lq0 = (uint64_t)row0 * (uint64_t)cols + (uint64_t)(c & ~(int64_t)3);
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        // this lane's call: row row0 + i + q, columns 4m .. 4m + 3; partner
        // q ^ d sends the word of this lane's column from its row i + (q ^ d)
        const U4 w = sr_words((lq0 + (uint64_t)(i + (int)q) * (uint64_t)cols) >> 2, seed_lo,
                              seed_hi);
        const uint32_t own = pick_word(w, q);
        const uint32_t g1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pick_word(w, q ^ 1u),
                                                                  0xB1, 0xF, 0xF, false);
        const uint32_t g2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pick_word(w, q ^ 2u),
                                                                  0x4E, 0xF, 0xF, false);
        const uint32_t g3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pick_word(w, q ^ 3u),
                                                                  0x1B, 0xF, 0xF, false);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t d = (uint32_t)r ^ q;       // row i + r came from lane q ^ d
          uint32_t u = own;
          u = d == 1u ? g1 : u;
          u = d == 2u ? g2 : u;
          u = d == 3u ? g3 : u;
          const uint32_t t = f_bits(__fmul_rn(__fmul_rn(y[i + r], m1), m2));
          o[(i + r) >> 3] |= (e2m1_sr_mag(t & 0x7FFFFFFFu, u >> 8) | ((t >> 28) & 8u))
                             << (4 * ((i + r) & 7));
        }
      }
      if (s == 0xFFu || !present) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = 0u;
      }
      if (!present) s = 0u;
    }
    *reinterpret_cast<uint4 *>(codes + code_offset(c, kb, nslices)) = make_uint4(o[0], o[1], o[2], o[3]);
    scales[scale_offset(c, kb, mnp)] = (uint8_t)s;
  }
}

// ---------------------------------------------------------------------------
// Both orientations from one read. A workgroup stages a 32-row x 128-column
// piece of the source in LDS, widened to fp32 (row stride 132 floats: one
// 16-byte chunk of padding, so that the staging writes, the row reads and
// the column reads below all spread over distinct banks, and every LDS
// access is a base address plus immediate offsets); threads 0..127 then
// encode its 128 row blocks into the
// axis-1 operand (source rows, K along the columns) and threads 128..255 its
// 128 column blocks into the axis-0 operand (source columns, K along the
// rows), each exactly as quant_axis1_kernel / quant_axis0_kernel would.
// Workgroups past the last source row only write the axis-0 operand's K
// padding (encoded zeros).
// ---------------------------------------------------------------------------
// At most 64 registers (8 waves per SIMD): the nearest-rounding instances
// need 48 anyway; the stochastic-rounding ones, at 59-75 unbounded, ran
// 0.5-3% faster bounded (a few registers spilled; bitwise identical).
template <int ROT, int RND>
__global__ __launch_bounds__(256, 8) void quant_dual_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t *__restrict__ codes1, uint8_t *__restrict__ scales1, uint32_t s1_lo, uint32_t s1_hi,
    uint8_t *__restrict__ codes0, uint8_t *__restrict__ scales0, uint32_t s0_lo, uint32_t s0_hi,
    int64_t gx) {
  __shared__ __attribute__((aligned(16))) float st[32 * 132];
  const int tid = threadIdx.x;
  const int64_t bx = (int64_t)blockIdx.x % gx, by = (int64_t)blockIdx.x / gx;
  const int64_t C0 = bx * 128, R0 = by * 32;
  const int64_t nsl1 = (cols + 127) >> 7;   // axis-1 operand: MN = rows, K = cols
  const int64_t nsl0 = (rows + 127) >> 7;   // axis-0 operand: MN = cols, K = rows
  const int64_t mnp1 = (rows + 255) & ~(int64_t)255, mnp0 = (cols + 255) & ~(int64_t)255;
  const bool rows_live = R0 < rows;

  if (rows_live) {
    // lane (r0, q) loads columns 4q .. 4q + 3 and 64 + 4q .. 64 + 4q + 3 of
    // rows r0 and r0 + 16, 8 bytes each and all four in flight at once (a
    // wait between them cost 5-12%), and writes them widened. cols % 32 == 0:
    // a group of four columns is all inside or all padding (zeros).
    const int q = tid & 15, r0 = tid >> 4;
    const int64_t c = C0 + 4 * q;
    u32x2 v[4] = {{0u, 0u}, {0u, 0u}, {0u, 0u}, {0u, 0u}};
    const uint16_t *p = x + R0 * ld + c + (int64_t)r0 * ld;
    if (c < cols) {
      v[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
      v[2] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p + 16 * ld));
    }
    if (c + 64 < cols) {
      v[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p + 64));
      v[3] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p + 16 * ld + 64));
    }
    float *d = st + r0 * 132 + 4 * q;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<float4 *>(d + (k >> 1) * 16 * 132 + (k & 1) * 64) =
          make_float4(bits_f(v[k].x << 16), bits_f(v[k].x & 0xFFFF0000u),
                      bits_f(v[k].y << 16), bits_f(v[k].y & 0xFFFF0000u));
  }
  __syncthreads();

  float y[32];
  uint32_t out[4];
  uint32_t s;
  const int lane = tid & 63;
  if (tid < 128) {
    // axis 1: row R0 + rr (< mnp1), 32-block kb along the columns
    const int rr = tid & 31, b = tid >> 5;
    const int64_t r = R0 + rr;
    const int64_t kb = (C0 >> 5) + b;
    // random signs: this wave's two blocks need the 16 sign calls at
    // counters ((C0 / 32) + 2 wave) * 8 + m, m < 16; lane m makes call m
    // (before any lane leaves, so that every source lane is active)
    uint32_t mask = 0u;
    if (ROT == MX_K_ROT_RAND_SIGN) {
      const uint32_t nib =
          sign_nibble((uint32_t)(((C0 >> 5) + 2 * (tid >> 6)) * 8 + (lane & 15)), s1_lo);
      const uint32_t m0 = gather_sign_mask(nib, 0), m1 = gather_sign_mask(nib, 8);
      mask = (lane >> 5) ? m1 : m0;
    }
    if (kb >= nsl1 * 4) return;                           // past the operand's K extent
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 f = *reinterpret_cast<const float4 *>(st + rr * 132 + b * 32 + 4 * j);
      y[4 * j] = f.x;
      y[4 * j + 1] = f.y;
      y[4 * j + 2] = f.z;
      y[4 * j + 3] = f.w;
    }
    if (ROT == MX_K_ROT_RAND_SIGN) apply_sign_mask(y, mask);
    rotate_block<ROT>(y);
    const uint64_t q0 = (uint64_t)(r * cols + (kb << 5)) >> 2;   // L % 4 == 0
    U4 w{0u, 0u, 0u, 0u};
    auto u24_of = [&](int i) -> uint32_t {
      if ((i & 3) == 0) w = sr_words(q0 + (uint64_t)(i >> 2), s1_lo, s1_hi);
      return pick_word(w, (uint32_t)(i & 3)) >> 8;
    };
    s = quantize_block<RotKind<ROT>::value, RND, kFmtE2M1>(y, out, u24_of);
    if ((kb << 5) >= cols || !rows_live) {                // padding of the operand
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = 0u;
      s = 0u;
    }
    // code_offset(r, kb, nsl1) and scale_offset(r, kb, mnp1) split into a
    // uniform part and a 32-bit lane part (R0 % 32 == 0, C0 % 128 == 0: row
    // group R0 / 16 + rr / 16, one K slice C0 / 128 for the four blocks,
    // scale group R0 / 256; codes < 1 GiB)
    {
      const int64_t cu = ((R0 >> 4) * nsl1 + (C0 >> 7)) * 1024;
      const uint32_t cl = ((rr >> 4) ? (uint32_t)nsl1 * 1024u : 0u) + (uint32_t)(b * 256 + (rr & 15) * 16);
      const int64_t hR = (R0 >> 4) & 15;                  // even: + rr / 16 carries into no other field
      const int64_t su = ((C0 >> 7) * (mnp1 >> 8) + (R0 >> 8)) * 1024 + (hR >> 2) * 256 + (hR & 3);
      const uint32_t sl = (uint32_t)(b * 64 + (rr & 15) * 4 + (rr >> 4));
      *reinterpret_cast<uint4 *>(codes1 + cu + cl) = make_uint4(out[0], out[1], out[2], out[3]);
      scales1[su + sl] = (uint8_t)s;
    }
  } else {
    // axis 0: column C0 + cc, 32-block R0 / 32 along the rows
    const int cc = tid - 128;
    const int64_t c = C0 + cc;                            // < mnp0
    const int64_t kb = R0 >> 5;
    if (kb >= nsl0 * 4) return;                           // past the operand's K extent (uniform)
    // random signs: the block's 32 rows need the 8 sign calls at counters
    // R0 / 4 + j; lane j makes call j
    uint32_t mask = 0u;
    if (ROT == MX_K_ROT_RAND_SIGN)
      mask = gather_sign_mask(sign_nibble((uint32_t)((R0 >> 2) + (lane & 7)), s0_lo), 0);
    if (rows_live && c < cols) {                          // uniform over each quad (cols % 32 == 0)
#pragma unroll
      for (int j = 0; j < 32; ++j) y[j] = st[j * 132 + cc];
      if (ROT == MX_K_ROT_RAND_SIGN) apply_sign_mask(y, mask);
      rotate_block<ROT>(y);
      if (RND == MX_K_ROUND_SR) {
        // element (R0 + i, c) draws word c % 4 of the call at
        // ((R0 + i) cols + c - c % 4) / 4 (cols % 4 == 0): the four lanes of
        // a quad (columns 4m .. 4m + 3) share each call. Lane q makes the
        // calls of rows i + q and a 4 x 4 transpose over DPP hands each lane
        // its column's words, as in quant_axis0_sr_kernel.
        float m1, m2;
        s = block_scale<RotKind<ROT>::value>(y, m1, m2);
        const uint32_t q = (uint32_t)(cc & 3);
        const uint64_t lq0 = (uint64_t)R0 * (uint64_t)cols + (uint64_t)(c & ~(int64_t)3);
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = 0u;
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
          const U4 w = sr_words((lq0 + (uint64_t)(i + (int)q) * (uint64_t)cols) >> 2, s0_lo,
                                s0_hi);
          const uint32_t own = pick_word(w, q);
          const uint32_t g1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pick_word(w, q ^ 1u),
                                                                    0xB1, 0xF, 0xF, false);
          const uint32_t g2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pick_word(w, q ^ 2u),
                                                                    0x4E, 0xF, 0xF, false);
          const uint32_t g3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pick_word(w, q ^ 3u),
                                                                    0x1B, 0xF, 0xF, false);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t d = (uint32_t)r ^ q;           // row i + r came from lane q ^ d
            uint32_t u = own;
            u = d == 1u ? g1 : u;
            u = d == 2u ? g2 : u;
            u = d == 3u ? g3 : u;
            const uint32_t t = f_bits(__fmul_rn(__fmul_rn(y[i + r], m1), m2));
            out[(i + r) >> 3] |= (e2m1_sr_mag(t & 0x7FFFFFFFu, u >> 8) | ((t >> 28) & 8u))
                                 << (4 * ((i + r) & 7));
          }
        }
        if (s == 0xFFu) {
#pragma unroll
          for (int j = 0; j < 4; ++j) out[j] = 0u;
        }
      } else {
        auto u24_of = [](int) -> uint32_t { return 0u; };   // nearest rounding draws nothing
        s = quantize_block<RotKind<ROT>::value, RND, kFmtE2M1>(y, out, u24_of);
      }
    } else {                                              // K padding of the operand
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = 0u;
      s = 0u;
    }
    // code_offset(c, kb, nsl0) and scale_offset(c, kb, mnp0) split the same
    // way (C0 % 128 == 0: row group C0 / 16 + cc / 16, scale group C0 / 256)
    {
      const int64_t cu = ((C0 >> 4) * nsl0 + (kb >> 2)) * 1024 + (kb & 3) * 256;
      const uint32_t cl = (uint32_t)(cc >> 4) * ((uint32_t)nsl0 * 1024u) + (uint32_t)((cc & 15) * 16);
      const int h = (int)((C0 >> 4) & 15) + (cc >> 4);  // 0 or 8, plus 0..7
      const int64_t su = ((kb >> 2) * (mnp0 >> 8) + (C0 >> 8)) * 1024 + (kb & 3) * 64;
      const uint32_t sl = (uint32_t)((h >> 2) * 256 + (cc & 15) * 4 + (h & 3));
      *reinterpret_cast<uint4 *>(codes0 + cu + cl) = make_uint4(out[0], out[1], out[2], out[3]);
      scales0[su + sl] = (uint8_t)s;
    }
  }
}

template <int ROT, int RND>
hipError_t launch_dual(const DualArgs &a, hipStream_t stream) {
  // columns up to the axis-0 operand's padded MN extent (which covers the
  // axis-1 operand's K extent), rows up to the axis-1 operand's padded MN
  // extent (which covers the axis-0 operand's K extent)
  const int64_t gx = ((a.cols + 255) & ~(int64_t)255) / 128;
  const int64_t gy = ((a.rows + 255) & ~(int64_t)255) / 32;
  return launch(quant_dual_kernel<ROT, RND>, dim3((unsigned)(gx * gy)), dim3(256), 0, stream,
                a.x, a.rows, a.cols, a.ld, a.codes1, a.scales1, a.seed1_lo, a.seed1_hi,
                a.codes0, a.scales0, a.seed0_lo, a.seed0_hi, gx);
}

template <int ROT, int RND, int FMT>
hipError_t launch_quant(const QuantArgs &a, hipStream_t stream) {
  if (a.axis == 1) {
    const int64_t mnp = (a.rows + 255) & ~(int64_t)255;
    const int64_t ntiles = (mnp >> 4) * ((a.cols + 127) >> 7);
    const int64_t blocks = (ntiles + 3) / 4;                  // one tile per wave
    return launch(quant_axis1_kernel<ROT, RND, FMT, false>, dim3((unsigned)blocks), dim3(256), 0,
                  stream, a.x, a.rows, a.cols, a.ld, a.codes, a.scales, a.seed_lo, a.seed_hi,
                  Axis1Second{});
  }
  const int threads = 256;
  const int64_t mnp = (a.cols + 255) & ~(int64_t)255;
  const int64_t nkb_pad = ((a.rows + 127) >> 7) * 4;
  // 32-row blocks per lane of the stochastic-rounding kernels: measured best 2
  const int rb = a.rb > 0 ? a.rb : (RND == MX_K_ROUND_SR ? 2 : 1);
  const int64_t gy = (nkb_pad + rb - 1) / rb;
  // one column per lane, quads sharing Philox: measured 15-18% faster with a
  // rotation and 21-23% faster without one than the column-pair kernel
  if constexpr (RND == MX_K_ROUND_SR && FMT == kFmtE2M1) {
    if ((a.cols & 3) == 0)
      return launch(quant_axis0_sr_kernel<ROT>, dim3((unsigned)(mnp / threads), (unsigned)gy),
                    dim3(threads), 0, stream, a.x, a.rows, a.cols, a.ld, a.codes, a.scales,
                    a.seed_lo, a.seed_hi, rb);
  }
  if constexpr (RND == MX_K_ROUND_RNE) {   // one column per lane, one block per workgroup row
    return launch(quant_axis0_rne_kernel<ROT, FMT>, dim3((unsigned)(mnp / 256), (unsigned)nkb_pad),
                  dim3(256), 0, stream, a.x, a.rows, a.cols, a.ld, a.codes, a.scales, a.seed_lo);
  } else {
    const int64_t gx = (mnp / 2 + threads - 1) / threads;
    const int pair_loads = (a.ld % 2 == 0) && (reinterpret_cast<uintptr_t>(a.x) % 4 == 0) ? 1 : 0;
    return launch(quant_axis0_kernel<ROT, RND, FMT>, dim3((unsigned)gx, (unsigned)gy), dim3(threads),
                  0, stream, a.x, a.rows, a.cols, a.ld, a.codes, a.scales, a.seed_lo, a.seed_hi, rb,
                  pair_loads);
  }
}

// Two axis-1 MXFP4 operands with the same column count in one launch: the
// grid walks the first operand's row groups and then the second's, saving
// one launch's ramp and drain.
template <int ROT, int RND>
hipError_t launch_pair(const QuantArgs &a, const QuantArgs &b, hipStream_t stream) {
  const int64_t mnp = (a.rows + 255) & ~(int64_t)255, mnp2 = (b.rows + 255) & ~(int64_t)255;
  const int64_t ntiles = ((mnp + mnp2) >> 4) * ((a.cols + 127) >> 7);
  const int64_t blocks = (ntiles + 3) / 4;                    // one tile per wave
  const Axis1Second sec{b.x, b.rows, b.ld, b.codes, b.scales, b.seed_lo, b.seed_hi};
  return launch(quant_axis1_kernel<ROT, RND, kFmtE2M1, true>, dim3((unsigned)blocks), dim3(256), 0,
                stream, a.x, a.rows, a.cols, a.ld, a.codes, a.scales, a.seed_lo, a.seed_hi, sec);
}

}  // namespace

hipError_t quantize_pair_launch(const QuantArgs &a, const QuantArgs &b, hipStream_t stream) {
  if (a.axis != 1 || b.axis != 1 || a.fmt != 0 || b.fmt != 0 || a.cols != b.cols ||
      a.rotate != b.rotate || a.round != b.round)
    return hipErrorInvalidValue;
  switch (a.rotate * 2 + a.round) {
    case 0: return launch_pair<0, 0>(a, b, stream);
    case 1: return launch_pair<0, 1>(a, b, stream);
    case 2: return launch_pair<1, 0>(a, b, stream);
    case 3: return launch_pair<1, 1>(a, b, stream);
    case 4: return launch_pair<2, 0>(a, b, stream);
    case 5: return launch_pair<2, 1>(a, b, stream);
    case 6: return launch_pair<3, 0>(a, b, stream);
    case 7: return launch_pair<3, 1>(a, b, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t quantize_dual_launch(const DualArgs &a, hipStream_t stream) {
  switch (a.rotate * 2 + a.round) {
    case 0: return launch_dual<0, 0>(a, stream);
    case 1: return launch_dual<0, 1>(a, stream);
    case 2: return launch_dual<1, 0>(a, stream);
    case 3: return launch_dual<1, 1>(a, stream);
    case 4: return launch_dual<2, 0>(a, stream);
    case 5: return launch_dual<2, 1>(a, stream);
    case 6: return launch_dual<3, 0>(a, stream);
    case 7: return launch_dual<3, 1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t quantize_launch(const QuantArgs &a, hipStream_t stream) {
  if (a.fmt == 1) {                       // E4M3 comparator: nearest rounding only
    if (a.round != MX_K_ROUND_RNE) return hipErrorInvalidValue;
    switch (a.rotate) {
      case 0: return launch_quant<0, 0, kFmtE4M3>(a, stream);
      case 1: return launch_quant<1, 0, kFmtE4M3>(a, stream);
      case 2: return launch_quant<2, 0, kFmtE4M3>(a, stream);
      case 3: return launch_quant<3, 0, kFmtE4M3>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.fmt != 0) return hipErrorInvalidValue;
  switch (a.rotate * 2 + a.round) {
    case 0: return launch_quant<0, 0, kFmtE2M1>(a, stream);
    case 1: return launch_quant<0, 1, kFmtE2M1>(a, stream);
    case 2: return launch_quant<1, 0, kFmtE2M1>(a, stream);
    case 3: return launch_quant<1, 1, kFmtE2M1>(a, stream);
    case 4: return launch_quant<2, 0, kFmtE2M1>(a, stream);
    case 5: return launch_quant<2, 1, kFmtE2M1>(a, stream);
    case 6: return launch_quant<3, 0, kFmtE2M1>(a, stream);
    case 7: return launch_quant<3, 1, kFmtE2M1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mx
