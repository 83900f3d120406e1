// Dequantization of a packed operand back to fp32 in its source's shape:
//
//   value = (-1)^sign * E(magnitude) * 2^(s - 127)
//
// with E the E2M1 value of a 4-bit code, or the E4M3 value of an 8-bit code
// for the MXFP8 comparator, and s the block's E8M0 scale (36Kr article "Neue
// Studie von AMD durchbricht die bestehende Erkenntnis ...", section "Was ist
// MXFP4?": one shared exponent per 32-element block; the reconstruction
// formula, lost from the page, is taken as OCP MX's). Scale 0xFF marks a NaN
// block. Every such value is exact in fp32 while it is finite: the smallest
// magnitude is 2^-128 (E2M1) or 2^-136 (E4M3), above fp32's 2^-149, and
// values of 2^128 or more (only scales 126 and 127 reach them; the quantizer
// writes at most 125) become +-Inf.
//
// One thread per 16 code bytes: a 1 KB E2M1 tile holds, at byte 16 t, the 32
// codes of block c = t / 16 of row r = t % 16; a 2 KB E4M3 tile holds, at
// byte 16 t, the 16 codes of chunk j = t / 16 of row r = t % 16. Threads
// therefore read the code buffer front to back.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_kernels.h"

namespace mx {

namespace {

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  // magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 of the 3-bit magnitude code
  const uint32_t m = c & 7u;
  const float mag = m < 4 ? 0.5f * (float)m : (float)(2u << ((m - 4) >> 1)) * ((m & 1) ? 1.5f : 1.f);
  return (c & 8u) ? -mag : mag;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if ((c & 0x7Fu) == 0x7Fu) return __builtin_nanf("");
  // subnormal: m * 2^-9; normal: (8 + m) * 2^(e - 10)
  const float mag = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
  return (c & 0x80u) ? -mag : mag;
}

// Scale byte of operand row m (0-based, padded extent mnp) and 32-element
// block kb: tiled as [K slice q][256-row panel T][quarter h/4][block c][row
// r][row group h % 4].
__device__ __forceinline__ uint32_t scale_at(const uint8_t *scales, int64_t mnp, int64_t m,
                                             int64_t kb) {
  const int64_t q = kb >> 2, c = kb & 3;
  const int64_t T = m >> 8, h = (m >> 4) & 15, r = m & 15;
  return scales[(q * (mnp >> 8) + T) * 1024 + (h >> 2) * 256 + c * 64 + r * 4 + (h & 3)];
}

template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // per tile: 64 chunks of 32 E2M1 codes, or 128 chunks of 16 E4M3 codes
  constexpr int kChunks = FMT ? 128 : 64;
  constexpr int kElems = FMT ? 16 : 32;
  const int64_t tile = t / kChunks;
  const int within = (int)(t % kChunks);
  const int64_t kslices = a.kp >> 7;
  const int64_t g = tile / kslices, q = tile % kslices;
  const int r = within & 15, j = within >> 4;
  const int64_t m = g * 16 + r;
  const int64_t k0 = q * 128 + (int64_t)j * kElems;
  if (g * 16 >= a.mnp || m >= a.mn || k0 >= a.k) return;
  const uint4 v = *reinterpret_cast<const uint4 *>(a.codes + t * 16);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const int sexp = (int)scale_at(a.scales, a.mnp, m, k0 >> 5);
  float *out = a.out;
  // source element (row, col): axis 1 -> (m, k), axis 0 -> (k, m)
#pragma unroll
  for (int e = 0; e < kElems; ++e) {
    const uint32_t code = FMT ? (w[e >> 2] >> (8 * (e & 3))) & 0xFFu
                              : (w[e >> 3] >> (4 * (e & 7))) & 0xFu;
    const float val = sexp == 0xFF ? __builtin_nanf("")
                                   : ldexpf(FMT ? e4m3_value(code) : e2m1_value(code), sexp - 127);
    const int64_t k = k0 + e;
    if (a.axis == 1)
      out[m * a.ld + k] = val;
    else
      out[k * a.ld + m] = val;
  }
}

}  // namespace

hipError_t dequantize_launch(const DequantArgs &a, hipStream_t stream) {
  const int64_t chunks = a.mnp * a.kp / (a.fmt ? 16 : 32);
  const dim3 grid((unsigned)((chunks + 255) / 256));
  return a.fmt ? launch(dequant_kernel<1>, grid, dim3(256), 0, stream, a)
               : launch(dequant_kernel<0>, grid, dim3(256), 0, stream, a);
}

}  // namespace mx
