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
// in byte 0 of its scale operand; lane l receives rows 4 * (l / 16) + r,
// r = 0..3, of output column l % 16. The kernel passes B as the first
// operand, so lane l holds C[l % 16][4 * (l / 16) + r]: four consecutive
// columns of one row.
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

// Generic epilogue store of one quad: lane (lr, lg) of a 16x16 tile holds
// C[row][col .. col + 3] with row = tile row + lr, col = tile col + 4 lg.
// Element-wise and masked, for shapes the row-staged path does not take.
template <int OUT_BF16>
__device__ __forceinline__ void store_quad(const GemmArgs &g, const v4f &acc, int64_t row,
                                           int64_t col) {
  if (row >= g.M) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (col + r < g.N) {
      if (OUT_BF16)
        reinterpret_cast<uint16_t *>(g.c)[row * g.ldc + col + r] = f32_to_bf16_rne(acc[r]);
      else
        reinterpret_cast<float *>(g.c)[row * g.ldc + col + r] = acc[r];
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
// publishes a stage. The s_nop covers GFX9's one wait state between an M0
// write and an LDS DMA that reads it.
__device__ __forceinline__ void dma_load16(v4i rsrc, int voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_load4(v4i rsrc, int voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

// ---------------------------------------------------------------------------
// 256x256 block tile, eight waves (two per SIMD) in a 2x4 grid, 128x64 per
// wave = 8x4 MFMA tiles (128 fp32 accumulators per lane); two waves per SIMD
// let one wave's MFMAs cover the other's stalls.
//
// Operands are in the tiled layout the quantizer writes: a 1 KB tile holds 16
// rows x 128 K elements as [32-block c][row r][16 B], which is exactly the
// 16x16x128 MFMA fragment with lane l's 16 bytes at offset 16 l; scales of a
// 128-wide K slice are one contiguous run of 4 bytes per row. K advances one
// slice per stage through a ring of four LDS stage buffers with three stages
// in flight; each stage's copies are spread over its MFMA rows and the next
// stage's fragments are read while the current one's MFMAs run. Every copy is a direct-to-LDS load of one contiguous span (a
// 1 KB tile or 256 bytes of scales), and every LDS fragment read is one
// contiguous 1 KB span, the only pattern gfx950's LDS serves at its full 256
// bytes per clock (measured: a row-major layout takes 4x and an XOR-swizzled
// one 2x the cycles; gathering rows from a row-major operand made the copies
// 2.5x slower). Tiles past the operand's padded extent read as zero through
// the buffer range check; padded rows and K blocks hold encoded zeros.
// ---------------------------------------------------------------------------
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kThreads = 512;
constexpr int kStageA = kBM * 64;                  // 16 tiles of 1 KB
constexpr int kStageB = kBN * 64;
constexpr int kStageSA = kBM * 4;                  // 1 KB of scales
constexpr int kStageSB = kBN * 4;
constexpr int kStageBytes = kStageA + kStageB + kStageSA + kStageSB;
constexpr int kRing = 4;                           // stage buffers (136 KB)
constexpr int kAhead = kRing - 1;                  // stages in flight
constexpr int kGroupM = 8;                         // tile rows per ordering group

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
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRing * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0..7
  const int wm = wave >> 2, wn = wave & 3;                     // 2 x 4 wave grid
  const int64_t tm = (g.M + kBM - 1) / kBM, tn = (g.N + kBN - 1) / kBN;
  int64_t mi, ni;
  tile_coords(blockIdx.x, tm, tn, &mi, &ni);
  const int m0 = (int)(mi * kBM), n0 = (int)(ni * kBN);
  const int mp = (int)((g.M + 15) & ~15LL), np = (int)((g.N + 15) & ~15LL);   // padded rows
  const int nslices = (int)((g.K + 127) >> 7);
  const int a_bytes = mp * nslices * 64, b_bytes = np * nslices * 64;
  const int sa_bytes = nslices * mp * 4, sb_bytes = nslices * np * 4;
  const v4i rsrc_a = make_rsrc(g.a_codes, (uint32_t)a_bytes);
  const v4i rsrc_b = make_rsrc(g.b_codes, (uint32_t)b_bytes);
  const v4i rsrc_s = wave < 4 ? make_rsrc(g.a_scales, (uint32_t)sa_bytes)
                              : make_rsrc(g.b_scales, (uint32_t)sb_bytes);
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);

  // Codes: wave w copies row groups 2w, 2w + 1 of the block's A and B rows;
  // group G, slice s is the 1 KB at (G * nslices + s) * 1 KB. Groups past the
  // padded extent (wave-uniform test) load from the buffer end, i.e. zeros.
  const int ga = (m0 >> 4) + wave * 2, gb = (n0 >> 4) + wave * 2;
  const int a_lane = ga * nslices * 1024 + lane * 16;
  const int b_lane = gb * nslices * 1024 + lane * 16;
  // Scales: waves 0..3 copy A's rows 64 w .. 64 w + 63, waves 4..7 B's;
  // rows past the padded extent load zeros.
  const int s_rows = wave < 4 ? mp : np;
  const int s_row = (wave < 4 ? m0 : n0) + (wave & 3) * 64 + lane;
  const int s_bytes = wave < 4 ? sa_bytes : sb_bytes;
  const int s_lane = s_row * 4;
  const uint32_t s_lds = (uint32_t)(kStageA + kStageB + (wave < 4 ? 0 : kStageSA) + (wave & 3) * 256);

  // DMA instruction `part` (0, 1: A tiles; 2, 3: B tiles; 4: scales) of
  // stage s into ring buffer buf. Stages past the last slice read zeros, so
  // every stage issues the same five instructions and the vmcnt bookkeeping
  // stays uniform.
  auto issue_part = [&](int s, int buf, int part) {
    const uint32_t stage = smem_base + (uint32_t)(buf * kStageBytes);
    const bool live = s < nslices;
    if (part < 4) {
      const int j = part & 1;
      const bool is_b = part >= 2;
      int l = is_b ? b_lane : a_lane;
      asm volatile("" : "+v"(l));
      const int off = (j * nslices + s) * 1024;
      const bool ok = live && ((is_b ? gb : ga) + j) * 16 < (is_b ? np : mp);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          stage + (uint32_t)((wave * 2 + j) * 1024 + (is_b ? kStageA : 0)));
      dma_load16(is_b ? rsrc_b : rsrc_a, ok ? l + off : (is_b ? b_bytes : a_bytes), dst);
    } else {
      int l = s_lane;
      asm volatile("" : "+v"(l));
      dma_load4(rsrc_s, (live && s_row < s_rows) ? l + s * s_rows * 4 : s_bytes,
                __builtin_amdgcn_readfirstlane(stage + s_lds));
    }
  };

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15;      // row within a 16-row MFMA tile
  const int lg = lane >> 4;      // 32-element K block within the slice
  const uint32_t a_off = (uint32_t)((wm * 8) * 1024 + lane * 16);
  const uint32_t b_off = (uint32_t)(kStageA + (wn * 4) * 1024 + lane * 16);
  const uint32_t sa_off = (uint32_t)(kStageA + kStageB + (wm * 128 + lr) * 4);
  const uint32_t sb_off = (uint32_t)(kStageA + kStageB + kStageSA + (wn * 64 + lr) * 4);
  auto ld16 = [&](int buf, uint32_t off) {
    return *reinterpret_cast<const uint4 *>(smem + buf * kStageBytes + off);
  };
  // the MFMA reads byte 0 of its scale operand: shift K block lg's byte there
  auto ld_scale = [&](int buf, uint32_t off) {
    return *reinterpret_cast<const uint32_t *>(smem + buf * kStageBytes + off) >> (8 * lg);
  };

  for (int p = 0; p < kAhead; ++p)
#pragma unroll
    for (int part = 0; part < 5; ++part) issue_part(p, p, part);
  asm volatile("s_waitcnt vmcnt(10)" ::: "memory");   // this wave's part of stage 0
  __syncthreads();

  uint4 bf[4], bn[4], a0, a1;
  uint32_t sb[4], sbn[4], sa[8], san[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf[j] = ld16(0, b_off + j * 1024);
    sb[j] = ld_scale(0, sb_off + j * 64);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) sa[i] = ld_scale(0, sa_off + i * 64);
  a0 = ld16(0, a_off);
  a1 = ld16(0, a_off + 1024);

  // Stage s: 8 rows of 4 MFMAs. A fragments stream two rows ahead. After
  // row 3 the wave waits for its part of stage s + 1, and the barrier makes
  // every wave's part visible and frees the buffer of stage s - 1, which
  // rows 3..7 then refill with stage s + 3 (one DMA instruction per row).
  // Rows 4..7 also read stage s + 1's B fragments, scales and first two A
  // rows, so the next stage starts without an LDS round trip.
  for (int s = 0; s < nslices; ++s) {
    const int cur = s & 3, nxt = (s + 1) & 3, refill = (s + 3) & 3;
    uint4 af[8];
    af[0] = a0;
    af[1] = a1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i + 2 < 8) af[i + 2] = ld16(cur, a_off + (i + 2) * 1024);
      if (i == 4) {
        bn[0] = ld16(nxt, b_off);
        bn[1] = ld16(nxt, b_off + 1024);
        sbn[0] = ld_scale(nxt, sb_off);
        sbn[1] = ld_scale(nxt, sb_off + 64);
      } else if (i == 5) {
        bn[2] = ld16(nxt, b_off + 2048);
        bn[3] = ld16(nxt, b_off + 3072);
        sbn[2] = ld_scale(nxt, sb_off + 128);
        sbn[3] = ld_scale(nxt, sb_off + 192);
      } else if (i == 6) {
#pragma unroll
        for (int r = 0; r < 8; ++r) san[r] = ld_scale(nxt, sa_off + r * 64);
        a0 = ld16(nxt, a_off);
      } else if (i == 7) {
        a1 = ld16(nxt, a_off + 1024);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_fp4(bf[j], af[i], acc[i][j], sb[j], sa[i]);
      if (i == 3) {
        asm volatile("s_waitcnt vmcnt(5)" ::: "memory");   // own part of stage s + 1
        __syncthreads();
      }
      if (i >= 3) issue_part(s + kAhead, refill, i - 3);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf[j] = bn[j];
      sb[j] = sbn[j];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sa[i] = san[i];
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // zero-fill loads past the end

  // Epilogue. Fast path (N and ldc multiples of 8, C 16-byte aligned): the tile goes through the now idle LDS
  // ring in row-major order and leaves as whole 512-byte (bf16) or 1 KB
  // (fp32) rows, one 16-byte store per lane, so every store instruction
  // writes complete cache lines.
  const bool fast_epi = (g.N & 7) == 0 && (g.ldc & 7) == 0 &&
                        (reinterpret_cast<uintptr_t>(g.c) & 15) == 0;
  if (fast_epi) {
    constexpr int kEsz = OUT_BF16 ? 2 : 4;
    constexpr int kRowB = kBN * kEsz;                // bytes of one tile row
    constexpr int kPitch = kRowB + 16;               // padded LDS row
    constexpr int kRowsPerPass = OUT_BF16 ? 256 : 128;
    static_assert(kRowsPerPass * kPitch <= kRing * kStageBytes, "epilogue staging fits the ring");
    const int64_t rows_left = g.M - m0;
    const int cols_left = (int)min((int64_t)kBN, g.N - n0);
#pragma unroll
    for (int h = 0; h < 256 / kRowsPerPass; ++h) {
      __syncthreads();                               // ring (or previous pass) no longer read
      if (OUT_BF16 || wm == h) {
        const int rbase = OUT_BF16 ? wm * 128 : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint8_t *p = smem + (rbase + i * 16 + lr) * kPitch + (wn * 64 + j * 16 + 4 * lg) * kEsz;
            if (OUT_BF16) {
              uint2 v;
              v.x = (uint32_t)f32_to_bf16_rne(acc[i][j][0]) | ((uint32_t)f32_to_bf16_rne(acc[i][j][1]) << 16);
              v.y = (uint32_t)f32_to_bf16_rne(acc[i][j][2]) | ((uint32_t)f32_to_bf16_rne(acc[i][j][3]) << 16);
              *reinterpret_cast<uint2 *>(p) = v;
            } else {
              *reinterpret_cast<float4 *>(p) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
          }
      }
      __syncthreads();
      // 16 bytes per thread: kRowB / 16 threads per row
      constexpr int kThrPerRow = kRowB / 16;
      constexpr int kRowsPerIter = kThreads / kThrPerRow;
      const int r_in = tid / kThrPerRow, c16 = tid % kThrPerRow;
#pragma unroll 4
      for (int r = r_in; r < kRowsPerPass; r += kRowsPerIter) {
        const int trow = h * kRowsPerPass + r;
        const int col = c16 * (16 / kEsz);
        if (trow < rows_left && col < cols_left) {
          const uint4 v = *reinterpret_cast<const uint4 *>(smem + r * kPitch + c16 * 16);
          uint8_t *dst = reinterpret_cast<uint8_t *>(g.c) + ((m0 + trow) * g.ldc + n0 + col) * kEsz;
          *reinterpret_cast<uint4 *>(dst) = v;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_quad<OUT_BF16>(g, acc[i][j], (int64_t)m0 + wm * 128 + i * 16 + lr,
                             (int64_t)n0 + wn * 64 + j * 16 + 4 * lg);
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
  const int64_t tiles = ((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
  const dim3 grid((unsigned)tiles);
  return g.out_bf16 ? launch(gemm_tiled_kernel<1>, grid, dim3(kThreads), 0, stream, g)
                    : launch(gemm_tiled_kernel<0>, grid, dim3(kThreads), 0, stream, g);
}

}  // namespace mx
