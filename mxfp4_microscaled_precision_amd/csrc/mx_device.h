// Device helpers shared by the gfx950 kernels: Philox4x32-10, bf16 widening,
// the E8M0 block exponent and the E2M1 element encoders.
//
// The MXFP4 format (36Kr article "Neue Studie von AMD durchbricht die
// bestehende Erkenntnis ...", section "Was ist MXFP4?"): 32-element blocks,
// one shared E8M0 exponent taken from the largest exponent in the block, and
// 4-bit elements rounded to the nearest representable value. The element bit
// split (1 sign, 2 exponent, 1 mantissa) is on the ShowAPI page
// "AMD颠覆认知：FP4不稳定性的真正原因", section 2.2; exponent bias 1 and the
// value set {0, 0.5, 1, 1.5, 2, 3, 4, 6} follow OCP MX, the standard the 36Kr
// page names in "Fazit".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

constexpr int kBlock = 32;

// fp32(1/sqrt(32)): the normalisation that makes the 32-point Sylvester
// Hadamard orthonormal.
constexpr uint32_t kInvSqrt32Bits = 0x3E3504F3u;

__device__ __forceinline__ float bits_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): 10 rounds of two 32x32->64 multiplies with the
// constants below, the key advanced by the two Weyl increments between rounds.
// ---------------------------------------------------------------------------
struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // full 64-bit products: one v_mad_u64_u32 each gives both halves
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    // the two three-way xors as one v_bitop3_b32 each (truth table 0x96:
    // odd parity of the three inputs)
    U4 n;
    n.x = __builtin_amdgcn_bitop3_b32(hi1, c.y, k0, 0x96);
    n.y = lo1;
    n.z = __builtin_amdgcn_bitop3_b32(hi0, c.w, k1, 0x96);
    n.w = lo0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

__device__ __forceinline__ uint32_t pick_word(const U4 &v, uint32_t j) {
  uint32_t r = v.x;
  r = (j == 1) ? v.y : r;
  r = (j == 2) ? v.z : r;
  r = (j == 3) ? v.w : r;
  return r;
}

// Random-sign words for reduction indices 4q .. 4q+3 (key (seed_lo, 0),
// counter (q, 0, 1, 0)); bit 31 of word j is the sign of index 4q + j.
__device__ __forceinline__ U4 sign_words(uint32_t q, uint32_t seed_lo) {
  return philox4x32_10(U4{q, 0u, 1u, 0u}, seed_lo, 0u);
}

// Stochastic-rounding words for source indices 4q .. 4q+3, q = L >> 2 (64-bit):
// key (seed_lo, seed_hi), counter (q mod 2^32, q >> 32, 0, 0).
__device__ __forceinline__ U4 sr_words(uint64_t q, uint32_t seed_lo, uint32_t seed_hi) {
  return philox4x32_10(U4{(uint32_t)q, (uint32_t)(q >> 32), 0u, 0u}, seed_lo, seed_hi);
}

// ---------------------------------------------------------------------------
// Block scale. amax_bits = max over the block of (fp32 bits & 0x7fffffff).
// Returns the unbiased exponent e = clamp(floor(log2 amax) - 2, -127, 127)
// (-127 for an all-zero block); the caller handles amax_bits >= 0x7f800000
// (a NaN or Inf in the block) separately.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_exponent(uint32_t amax_bits) {
  // floor(log2 amax) = (biased exponent) - 127 for a normal amax. A
  // subnormal or zero amax has biased exponent 0 and every such value has
  // floor(log2 amax) - 2 <= -129, so the lower clamp covers it; the largest
  // finite amax gives 125, inside the upper clamp.
  return max((int)(amax_bits >> 23) - 129, -127);
}

// 2^-e as fp32 for e in [-127, 125] (always a normal number there).
__device__ __forceinline__ float pow2_neg(int e) {
  return bits_f((uint32_t)(127 - e) << 23);
}

// ---------------------------------------------------------------------------
// E2M1 magnitude code of a = |t| (fp32 bits ab, sign cleared), nearest with
// ties to the even mantissa bit, saturating at 6. Decision thresholds:
// 0.25 (tie -> 0), 0.75 (tie -> 1.0), 1.25 (tie -> 1.0), 1.75 (tie -> 2),
// 2.5 (tie -> 2), 3.5 (tie -> 4), 5 (tie -> 4). Integer compares of the
// non-negative fp32 bit patterns are exact.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1_rne_mag(uint32_t ab) {
  uint32_t m = 0;
  m += ab > 0x3E800000u;   // > 0.25
  m += ab >= 0x3F400000u;  // >= 0.75
  m += ab > 0x3FA00000u;   // > 1.25
  m += ab >= 0x3FE00000u;  // >= 1.75
  m += ab > 0x40200000u;   // > 2.5
  m += ab >= 0x40600000u;  // >= 3.5
  m += ab > 0x40A00000u;   // > 5.0
  return m;
}

// Stochastic E2M1 magnitude code: lo <= a < hi neighbours, upper one taken
// when u24 < f * 2^24 with f = (a - lo) / (hi - lo); a >= 6 gives 6 (not
// randomised). With eb the biased fp32 exponent of a and ec = max(eb, 127),
// z = a * 2^(128 - ec) is an exact scaling that maps the gap to 1: z lies in
// [2, 4) for 1 <= a < 6 (gap 2^(eb - 128)), in [1, 2) for 0.5 <= a < 1 and in
// [0, 1) below (gap 0.5 for both). Then lo has code floor(z) + 2 (ec - 127)
// and f = z - floor(z), so f * 2^24 is exact, as is the comparison with the
// integer u24 < 2^24. It replaced a search over the seven neighbour
// boundaries (about forty-five VALU operations, partly as branches; the
// quantizers ran 22-37% faster with stochastic rounding); both forms agree
// on every fp32 magnitude at its threshold and either side of it.
__device__ __forceinline__ uint32_t e2m1_sr_mag(uint32_t ab, uint32_t u24) {
  const uint32_t ec = max(ab >> 23, 127u);
  const float z = __builtin_ldexpf(bits_f(ab), 128 - (int)ec);
  const uint32_t lo = (uint32_t)z;                           // floor(z), z >= 0
  const float thr = __fmul_rn(__builtin_amdgcn_fractf(z), 16777216.0f);
  const uint32_t code = lo + 2u * (ec - 127u) + ((float)u24 < thr ? 1u : 0u);
  return ab >= 0x40C00000u ? 7u : code;
}

}  // namespace mx
