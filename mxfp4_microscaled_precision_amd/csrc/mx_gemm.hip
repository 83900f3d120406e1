// MXFP4 GEMM on gfx950's block-scaled FP4 matrix cores, fp32 accumulation.
//
//   C[m][n] = sum_k A(m, k) * B(n, k),   A(m, k) = E2M1(a) * 2^(sa - 127)
//
// (36Kr article "Neue Studie von AMD durchbricht die bestehende Erkenntnis
// ...", section "Fehlerdiagnoseexperiment": Fprop, Dgrad and Wgrad all reduce
// to this form once the operands are stored reduction-major; section "Was ist
// MXFP4?": one E8M0 scale per 32 elements.)
//
// Instruction: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in FP4
// (format code 4). For a 16x16 output tile and a 128-wide K slice, lane l
// supplies row (l % 16) of A and row (l % 16) of B, K elements
// [32 * (l / 16), 32 * (l / 16) + 32) as 16 packed bytes (element 2j in the
// low nibble of byte j), and the E8M0 scale of exactly that 32-element block
// in byte 0 of its scale operand. Lane l receives C rows 4 * (l / 16) + r,
// r = 0..3, of column l % 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_kernels.h"

namespace mx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kFmtFp4 = 4;

__device__ __forceinline__ v4f mfma_fp4(const uint4 &a, const uint4 &b, v4f c, uint32_t sa,
                                        uint32_t sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, kFmtFp4, kFmtFp4, 0,
                                                          (int)sa, 0, (int)sb);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// Reference-structure kernel: 128x128 block tile, four waves in a 2x2 grid,
// 64x64 per wave (4x4 MFMA tiles), operands loaded straight from global
// memory into the MFMA register layout. Rows past M / N are clamped to the
// last valid row for loading and masked on store; K slices past K load zero
// codes (which contribute exactly zero whatever the scale).
// ---------------------------------------------------------------------------
template <int OUT_BF16>
__global__ __launch_bounds__(256) void gemm_direct_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t m_base = (int64_t)blockIdx.y * 128 + (wave >> 1) * 64;
  const int64_t n_base = (int64_t)blockIdx.x * 128 + (wave & 1) * 64;
  const int64_t kbytes = g.K >> 1;
  const int64_t kblocks = g.K >> 5;
  const int row_in = lane & 15;
  const int kgrp = lane >> 4;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  int64_t arow[4], brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    arow[i] = min(m_base + 16 * i + row_in, g.M - 1);
    brow[i] = min(n_base + 16 * i + row_in, g.N - 1);
  }

  for (int64_t k0 = 0; k0 < g.K; k0 += 128) {
    const int64_t kb = (k0 >> 5) + kgrp;
    const bool kval = kb < kblocks;
    uint4 a[4], b[4];
    uint32_t sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kval) {
        a[i] = *reinterpret_cast<const uint4 *>(g.a_codes + arow[i] * kbytes + kb * 16);
        sa[i] = g.a_scales[arow[i] * kblocks + kb];
        b[i] = *reinterpret_cast<const uint4 *>(g.b_codes + brow[i] * kbytes + kb * 16);
        sb[i] = g.b_scales[brow[i] * kblocks + kb];
      } else {
        a[i] = make_uint4(0, 0, 0, 0);
        b[i] = make_uint4(0, 0, 0, 0);
        sa[i] = 127u;
        sb[i] = 127u;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_fp4(a[i], b[j], acc[i][j], sa[i], sb[j]);
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n_base + 16 * j + row_in;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m_base + 16 * i + 4 * kgrp + r;
        if (row < g.M && col < g.N) {
          if (OUT_BF16)
            reinterpret_cast<uint16_t *>(g.c)[row * g.ldc + col] = f32_to_bf16_rne(acc[i][j][r]);
          else
            reinterpret_cast<float *>(g.c)[row * g.ldc + col] = acc[i][j][r];
        }
      }
    }
  }
}

template <int OUT_BF16>
__global__ __launch_bounds__(256) void fill_zero_kernel(GemmArgs g) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = g.M * g.N;
  if (idx >= total) return;
  const int64_t row = idx / g.N;
  const int64_t col = idx - row * g.N;
  if (OUT_BF16)
    reinterpret_cast<uint16_t *>(g.c)[row * g.ldc + col] = 0;
  else
    reinterpret_cast<float *>(g.c)[row * g.ldc + col] = 0.f;
}

}  // namespace

hipError_t gemm_launch(const GemmArgs &g, hipStream_t stream) {
  if (g.K == 0) {
    const int64_t total = g.M * g.N;
    const dim3 grid((unsigned)((total + 255) / 256));
    return g.out_bf16 ? launch(fill_zero_kernel<1>, grid, dim3(256), 0, stream, g)
                      : launch(fill_zero_kernel<0>, grid, dim3(256), 0, stream, g);
  }
  const dim3 grid((unsigned)((g.N + 127) / 128), (unsigned)((g.M + 127) / 128));
  return g.out_bf16 ? launch(gemm_direct_kernel<1>, grid, dim3(256), 0, stream, g)
                    : launch(gemm_direct_kernel<0>, grid, dim3(256), 0, stream, g);
}

}  // namespace mx
