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
typedef int v4i __attribute__((ext_vector_type(4)));
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

template <int OUT_BF16>
__device__ __forceinline__ void store_tile(const GemmArgs &g, const v4f &acc, int64_t row0,
                                           int64_t col) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = row0 + r;
    if (row < g.M && col < g.N) {
      if (OUT_BF16)
        reinterpret_cast<uint16_t *>(g.c)[row * g.ldc + col] = f32_to_bf16_rne(acc[r]);
      else
        reinterpret_cast<float *>(g.c)[row * g.ldc + col] = acc[r];
    }
  }
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero.
__device__ __forceinline__ v4i make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32);   // stride 0
  r[2] = (int)bytes;                 // num_records in bytes
  r[3] = 0x00020000;                 // raw buffer, 32-bit data format
  return r;
}

// Direct-to-LDS loads: lane i's 16 (4) bytes from rsrc.base + voffset land at
// LDS byte address lds_base + 16 i (4 i). Written as inline asm so that the
// compiler neither serialises consecutive DMA loads nor waits for them before
// unrelated LDS reads (it cannot tell LDS destinations apart); the kernel
// waits for them explicitly (s_waitcnt vmcnt) before the barrier that
// publishes a stage.
__device__ __forceinline__ void dma_load16(v4i rsrc, int voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_load4(v4i rsrc, int voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

// ---------------------------------------------------------------------------
// Main kernel (K % 128 == 0): 256x256 block tile, K = 256 FP4 elements (128
// bytes) per stage, two LDS stages. Four waves in a 2x2 grid, 128x128 per
// wave = 8x8 MFMA tiles (256 fp32 accumulators per lane).
//
// Codes and scales move global -> LDS with direct-to-LDS buffer loads (no
// register staging); stage s + 1 is in flight while stage s is multiplied.
// Rows past M / N and K chunks past K read as zero through the buffer range
// check; zero codes contribute exactly zero whatever their scale.
//
// LDS codes layout: [row][8 chunks of 16 B]; logical chunk c of row r sits in
// slot c ^ g(r), g(r) = (r & 7) ^ ((r >> 3) & 1). The 16 rows one ds_read_b128
// touches (rows of one 16-row MFMA tile, same logical chunk) then fall in
// distinct bank groups for 32- and 64-bank LDS alike, and since g only
// depends on r & 15 every tile's fragment address is one base register plus
// an immediate. A DMA load writes lane i's 16 bytes to slot i of the wave's
// destination, so the swizzle is applied by choosing which global chunk each
// lane fetches. Scales layout: [row][8 bytes], byte q = K block q of the stage.
// ---------------------------------------------------------------------------
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBKBytes = 128;                      // 256 FP4 elements
constexpr int kStageA = kBM * kBKBytes;            // 32 KB
constexpr int kStageB = kBN * kBKBytes;            // 32 KB
constexpr int kStageSA = kBM * 8;                  // 2 KB
constexpr int kStageSB = kBN * 8;                  // 2 KB
constexpr int kStageBytes = kStageA + kStageB + kStageSA + kStageSB;
constexpr int kGroupM = 8;                         // tile rows per ordering group

__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

// Tile index -> (tile_m, tile_n): workgroups are dispatched round-robin over
// the 8 XCDs, so consecutive ids are first regrouped per XCD, then ordered in
// groups of kGroupM tile rows so that each XCD works on a compact 2-D region
// of C and shares its A and B panels through its own L2.
__device__ __forceinline__ void tile_coords(int64_t bid, int64_t tm, int64_t tn, int64_t *mi,
                                            int64_t *ni) {
  const int64_t T = tm * tn;
  int64_t id = bid;
  if ((T & 7) == 0) id = (bid & 7) * (T >> 3) + (bid >> 3);
  const int64_t per_group = kGroupM * tn;
  const int64_t grp = id / per_group;
  const int64_t first_m = grp * kGroupM;
  const int64_t gm = min((int64_t)kGroupM, tm - first_m);
  const int64_t r = id - grp * per_group;
  *mi = first_m + r % gm;
  *ni = r / gm;
}

template <int OUT_BF16>
__global__ __launch_bounds__(256, 1) void gemm_lds_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tm = (g.M + kBM - 1) / kBM, tn = (g.N + kBN - 1) / kBN;
  int64_t mi, ni;
  tile_coords(blockIdx.x, tm, tn, &mi, &ni);
  const int m0 = (int)(mi * kBM), n0 = (int)(ni * kBN);
  const int M = (int)g.M, N = (int)g.N;
  const int kbytes = (int)(g.K >> 1);
  const int kblocks = (int)(g.K >> 5);
  const int nstage = (kblocks + 7) >> 3;

  const int a_bytes = M * kbytes, b_bytes = N * kbytes;
  const int sa_bytes = M * kblocks, sb_bytes = N * kblocks;
  const v4i rsrc_a = make_rsrc(g.a_codes, (uint32_t)a_bytes);
  const v4i rsrc_b = make_rsrc(g.b_codes, (uint32_t)b_bytes);
  const v4i rsrc_sa = make_rsrc(g.a_scales, (uint32_t)sa_bytes);
  const v4i rsrc_sb = make_rsrc(g.b_scales, (uint32_t)sb_bytes);
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);

  // Codes DMA: wave w fills stage rows [64 w, 64 w + 64), eight rows per load
  // j; lane -> row 64 w + 8 j + (lane >> 3), slot lane & 7, whose logical
  // chunk is (lane & 7) ^ (lane >> 3) ^ (j & 1).
  const int lrow = lane >> 3;
  const int c0 = (lane & 7) ^ lrow;
  const int arow0 = m0 + wave * 64 + lrow;
  const int brow0 = n0 + wave * 64 + lrow;
  // Scales DMA: two 4-byte loads per operand per wave; lane -> row
  // 64 w + 32 q + (lane >> 1), half (lane & 1) of the stage's 8 scale bytes.
  const int srow0 = wave * 64 + (lane >> 1);
  const int shalf = lane & 1;

  auto issue = [&](int s, int buf) {
    const uint32_t stage = smem_base + (uint32_t)(buf * kStageBytes);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int chunk = c0 ^ (j & 1);
      const bool kval = s * 8 + chunk < kblocks;
      const int ra = arow0 + 8 * j, rb = brow0 + 8 * j;
      const int koff = s * kBKBytes + chunk * 16;
      const int ao = (kval && ra < M) ? ra * kbytes + koff : a_bytes;
      const int bo = (kval && rb < N) ? rb * kbytes + koff : b_bytes;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(stage + (wave * 64 + 8 * j) * kBKBytes);
      dma_load16(rsrc_a, ao, dst);
      dma_load16(rsrc_b, bo, dst + kStageA);
    }
    const bool sval = s * 8 + shalf * 4 < kblocks;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = srow0 + 32 * q;
      const int ra = m0 + r, rb = n0 + r;
      const int so = s * 8 + shalf * 4;
      const int sao = (sval && ra < M) ? ra * kblocks + so : sa_bytes;
      const int sbo = (sval && rb < N) ? rb * kblocks + so : sb_bytes;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          stage + kStageA + kStageB + (wave * 64 + 32 * q) * 8);
      dma_load4(rsrc_sa, sao, dst);
      dma_load4(rsrc_sb, sbo, dst + kStageSA);
    }
  };

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15;      // row within a 16-row MFMA tile
  const int lg = lane >> 4;      // 32-element K group within a 128-wide K slice

  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    if (s + 1 < nstage) issue(s + 1, (s + 1) & 1);
    const uint8_t *base = smem + (s & 1) * kStageBytes;
    const uint8_t *sA = base;
    const uint8_t *sB = base + kStageA;
    const uint8_t *sSA = base + kStageA + kStageB;
    const uint8_t *sSB = sSA + kStageSA;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // tile i's rows are base row + 16 i, and swz only depends on the row
      // within the tile, so one address per operand serves all eight tiles
      const uint8_t *pa = sA + (wm * 128 + lr) * kBKBytes + swz(lr, h * 4 + lg) * 16;
      const uint8_t *pb = sB + (wn * 128 + lr) * kBKBytes + swz(lr, h * 4 + lg) * 16;
      const uint8_t *psa = sSA + (wm * 128 + lr) * 8 + h * 4 + lg;
      const uint8_t *psb = sSB + (wn * 128 + lr) * 8 + h * 4 + lg;
      uint4 af[8], bf[8];
      uint32_t sa[8], sb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        af[i] = *reinterpret_cast<const uint4 *>(pa + i * 16 * kBKBytes);
        bf[i] = *reinterpret_cast<const uint4 *>(pb + i * 16 * kBKBytes);
        sa[i] = psa[i * 16 * 8];
        sb[i] = psb[i * 16 * 8];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma_fp4(af[i], bf[j], acc[i][j], sa[i], sb[j]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      store_tile<OUT_BF16>(g, acc[i][j], (int64_t)m0 + wm * 128 + i * 16 + 4 * lg,
                           (int64_t)n0 + wn * 128 + j * 16 + lr);
}

// ---------------------------------------------------------------------------
// General-K kernel (any K % 32 == 0): 128x128 block tile, four waves of 64x64,
// operands loaded from global memory straight into the MFMA register layout.
// Rows past M / N are clamped for loading and masked on store; K slices past
// K load zero codes.
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
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_tile<OUT_BF16>(g, acc[i][j], m_base + 16 * i + 4 * kgrp, n_base + 16 * j + row_in);
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
  // The LDS kernel addresses each operand through 32-bit buffer offsets.
  const bool fits32 = g.M * (g.K >> 1) < ((int64_t)1 << 31) &&
                      g.N * (g.K >> 1) < ((int64_t)1 << 31);
  if (g.K % 128 == 0 && fits32) {
    const int64_t tiles = ((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
    const dim3 grid((unsigned)tiles);
    return g.out_bf16 ? launch(gemm_lds_kernel<1>, grid, dim3(256), 0, stream, g)
                      : launch(gemm_lds_kernel<0>, grid, dim3(256), 0, stream, g);
  }
  const dim3 grid((unsigned)((g.N + 127) / 128), (unsigned)((g.M + 127) / 128));
  return g.out_bf16 ? launch(gemm_direct_kernel<1>, grid, dim3(256), 0, stream, g)
                    : launch(gemm_direct_kernel<0>, grid, dim3(256), 0, stream, g);
}

}  // namespace mx
