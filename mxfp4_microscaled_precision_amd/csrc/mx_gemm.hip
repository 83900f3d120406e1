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
// in a byte of its scale operand chosen by the instruction's byte select;
// lane l receives rows 4 * (l / 16) + r,
// r = 0..3, of output column l % 16. The kernel passes B as the first
// operand, so lane l holds C[l % 16][4 * (l / 16) + r]: four consecutive
// columns of one row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <utility>

#include "mx_gemm_common.h"
#include "mx_kernels.h"

namespace mx {

namespace {

using namespace gemm;

typedef double d2 __attribute__((ext_vector_type(2)));

constexpr int kFmtFp4 = 4;

// One 16x16x128 FP4 MFMA. The E8M0 scale of each operand is byte SELA / SELB
// of the given register (the instruction's byte select).
template <int SELA, int SELB>
__device__ __forceinline__ v4f mfma_fp4(const uint4 &a, const uint4 &b, v4f c, uint32_t sa,
                                        uint32_t sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, kFmtFp4, kFmtFp4, SELA,
                                                          (int)sa, SELB, (int)sb);
}

// Entry e of a grouped launch, one field at a time (e is wave-uniform:
// scalar selects between fields at fixed offsets, so the kernel argument
// block is never indexed at run time, which would copy it to scratch).
static_assert(kMaxGemmBatch == 4, "entry selects");
#define MX_ENTRY_FIELD(g, e, f) \
  ((e) == 1 ? (g).more[0].f : (e) == 2 ? (g).more[1].f : (e) == 3 ? (g).more[2].f : (g).f)
__device__ __forceinline__ GemmEntry entry_of(const GemmArgs &g, int e) {
  return GemmEntry{MX_ENTRY_FIELD(g, e, a_codes), MX_ENTRY_FIELD(g, e, a_scales),
                   MX_ENTRY_FIELD(g, e, b_codes), MX_ENTRY_FIELD(g, e, b_scales),
                   MX_ENTRY_FIELD(g, e, c)};
}
#undef MX_ENTRY_FIELD

// A buffer resource the compiler can keep in scalar registers (the value is
// wave-uniform; the direct-to-LDS load takes it as an SGPR quad).
__device__ __forceinline__ v4i uniform(v4i r) {
  return v4i{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
             __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}

// Tile t of the launch's (tall, for a grouped launch) tile grid -> entry and
// the tile's coordinates within that entry's output. tm = tile rows per entry.
template <bool BATCHED>
__device__ __forceinline__ void tile_of(const GemmArgs &g, int t, int tm, int tn, int *e, int *mi,
                                        int *ni) {
  tile_coords(t, BATCHED ? tm * g.batch : tm, tn, mi, ni);
  *e = 0;
  if (BATCHED) {
    *e = *mi / tm;
    *mi -= *e * tm;
  }
}

// ---------------------------------------------------------------------------
// 256x256 block tile. Twelve waves, three per SIMD: eight consumer waves in
// a 2x4 grid, 128x64 each = 8x4 MFMA tiles (128 fp32 accumulators per lane),
// and four producer waves that only copy. A direct-to-LDS copy can hold its
// wave at issue for hundreds of cycles while the L1 waits on pending L2
// reads; on a wave that also issues MFMAs that stall idles the matrix core,
// on a producer it costs nothing.
//
// Operands are in the tiled layout the quantizer writes: a 1 KB tile holds 16
// rows x 128 K elements as [32-block c][row r][16 B], which is exactly the
// 16x16x128 MFMA fragment with lane l's 16 bytes at offset 16 l; the scales
// of a 128-wide K slice and a 256-row panel are one contiguous 1 KB block
// whose 256-byte quarter hq holds, at 4 l, the scales of row groups
// 4 hq .. 4 hq + 3 for lane l's (row l % 16, block l / 16). K
// advances one slice per stage through a ring of four LDS stage buffers with
// three stages in flight. Every copy is a direct-to-LDS load of one
// contiguous 1 KB span (a code tile or a scale block), and every LDS fragment
// read is one contiguous 1 KB span, the only pattern gfx950's LDS serves at
// its full 256 bytes per clock (measured: a row-major layout takes 4x and an
// XOR-swizzled one 2x the cycles; gathering rows from a row-major operand
// made the copies 2.5x slower). Tiles past the operand's padded extent read
// as zero through the buffer range check; padded rows and K blocks hold
// encoded zeros.
// ---------------------------------------------------------------------------
constexpr int kThreads = 768;                      // 8 consumer + 4 producer waves
constexpr int kConsumers = 8;
constexpr int kStageA = kBM * 64;                  // 16 tiles of 1 KB
constexpr int kStageB = kBN * 64;
constexpr int kStageSA = kBM * 4;                  // 1 KB of scales
constexpr int kStageSB = kBN * 4;
constexpr int kStageBytes = kStageA + kStageB + kStageSA + kStageSB;
constexpr int kRing = 4;                           // stage buffers (136 KB)
constexpr int kAhead = kRing - 1;                  // stages in flight
static_assert(kRing * kStageBytes + kConsumers * kSlab <= 160 * 1024, "LDS");

// Row I of a consumer's stage: read A fragment I + 2 (and, in row S - 1, every
// A fragment still unread), then the 4 MFMAs of row I. Rows from S on read
// nothing. Two rows ahead measured 1-3% faster than one on all three ops,
// with the clock settled; three would not fit the registers. B is the first
// MFMA operand (its scale byte j of sb), A the second (scale byte I % 4 of
// sa.x for rows 0..3, of sa.y for rows 4..7).
template <int I, int S, int ROWS>
__device__ __forceinline__ void consume_row(v4f (&acc)[ROWS][4], const uint4 (&bf)[4],
                                            uint4 (&af)[ROWS], const uint8_t *a_base, uint32_t sb,
                                            uint2 sa) {
  if (I < S) {
#pragma unroll
    for (int j = I + 2; j < (I == S - 1 ? ROWS : I + 3); ++j)
      if (j < ROWS) af[j < ROWS ? j : 0] = *reinterpret_cast<const uint4 *>(a_base + j * 1024);
  }
  const uint32_t sai = I < 4 ? sa.x : sa.y;
  acc[I][0] = mfma_fp4<0, I & 3>(bf[0], af[I], acc[I][0], sb, sai);
  acc[I][1] = mfma_fp4<1, I & 3>(bf[1], af[I], acc[I][1], sb, sai);
  acc[I][2] = mfma_fp4<2, I & 3>(bf[2], af[I], acc[I][2], sb, sai);
  acc[I][3] = mfma_fp4<3, I & 3>(bf[3], af[I], acc[I][3], sb, sai);
  __builtin_amdgcn_sched_barrier(0);
}

// Rows LO .. LO + sizeof...(I) - 1 of a stage whose A fragments are all read
// by the end of row S - 1.
template <int LO, int S, int ROWS, int... I>
__device__ __forceinline__ void consume_rows(std::integer_sequence<int, I...>,
                                             v4f (&acc)[ROWS][4], const uint4 (&bf)[4],
                                             uint4 (&af)[ROWS], const uint8_t *a_base, uint32_t sb,
                                             uint2 sa) {
  (consume_row<LO + I, S, ROWS>(acc, bf, af, a_base, sb, sa), ...);
}

// Whole 16-byte stores of output rows: C and its row pitch 16-byte aligned.
template <int OUT_BF16>
__device__ __forceinline__ bool c_line_ok(const void *c, int64_t ldc) {
  return ((reinterpret_cast<uintptr_t>(c) & 15) == 0) && ((ldc * (OUT_BF16 ? 2 : 4)) & 15) == 0;
}

// One 8-byte (bf16) or 16-byte (fp32) store per quad.
template <int OUT_BF16>
__device__ __forceinline__ bool c_vec_ok(const void *c, int64_t ldc) {
  return ((reinterpret_cast<uintptr_t>(c) & (OUT_BF16 ? 7 : 15)) == 0) && ((ldc & 3) == 0);
}

// The consumers' stage loop. The consumers of wave row 0 wait at the barrier
// that publishes stage G, then read its first fragments. Those of wave row 1
// (SHIFTED; waves 4..7, so each SIMD holds one of each kind) run most of a
// stage behind: they read stage G right after finishing stage G - 1, with no
// barrier in between (stage G was published one barrier earlier), issue its
// first kSplit = 6 rows, which read every A fragment of the stage, take the
// barrier that publishes stage G + 1, then issue the last 2 rows from
// registers. While one wave on a SIMD waits for its first fragments of a
// stage, the other's MFMAs keep the matrix core busy. Because a shifted wave
// has read all of stage G before that barrier, the producers may refill its
// buffer right after it, as with no shift. Every wave takes total + 1
// barriers. Measured against all consumers waiting at every barrier: 3-5%
// faster on Fprop, Dgrad and Wgrad; splitting after 5 or 4 rows (more
// fragments live across the barrier) was slower.
template <int OUT_BF16, bool SHIFTED, int ROWS, bool BATCHED>
__device__ __forceinline__ void consumer_loop(const GemmArgs &g, uint8_t *smem, int total,
                                              int nslices, int bid, int grid, int tm, int tn,
                                              bool vec_ok, bool line_ok, uint32_t a_off,
                                              uint32_t b_off, uint32_t sa_off, uint32_t sb_off,
                                              int lr, int lg, int wm, int wn) {
  uint8_t *slab = smem + kRing * kStageBytes + (wm * 4 + wn) * kSlab;
  constexpr int kSplit = ROWS == 8 ? 6 : 3;
  constexpr bool kHalf = ROWS == 4;
  v4f acc[ROWS][4];
#pragma unroll
  for (int i = 0; i < ROWS; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  if (SHIFTED) __syncthreads();                            // stage 0 landed
  int ck = 0, cs = 0;
  for (int G = 0; G < total; ++G) {
    if (!SHIFTED) __syncthreads();                         // stage G landed
    const uint8_t *base = smem + (G & 3) * kStageBytes;
    uint4 bf[4], af[ROWS];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const uint4 *>(base + b_off + j * 1024);
    const uint32_t sb = *reinterpret_cast<const uint32_t *>(base + sb_off);
    const uint2 sa = make_uint2(*reinterpret_cast<const uint32_t *>(base + sa_off),
                                ROWS == 8 ? *reinterpret_cast<const uint32_t *>(base + sa_off + 256)
                                          : 0u);
    af[0] = *reinterpret_cast<const uint4 *>(base + a_off);
    af[1] = *reinterpret_cast<const uint4 *>(base + a_off + 1024);
    // rows of 4 MFMAs, A fragments two rows ahead
    if (!SHIFTED) {
      consume_rows<0, ROWS, ROWS>(std::make_integer_sequence<int, ROWS>{}, acc, bf, af,
                                  base + a_off, sb, sa);
    } else {
      consume_rows<0, kSplit, ROWS>(std::make_integer_sequence<int, kSplit>{}, acc, bf, af,
                                    base + a_off, sb, sa);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // all of stage G read
      __syncthreads();                                     // stage G + 1 landed
      consume_rows<kSplit, kSplit, ROWS>(std::make_integer_sequence<int, ROWS - kSplit>{}, acc,
                                         bf, af, base + a_off, sb, sa);
    }
    if (++cs == nslices) {
      cs = 0;
      int e, mi, ni;
      tile_of<BATCHED>(g, g.tile_base + (kHalf ? (bid >> 1) : bid + ck * grid), tm, tn, &e, &mi,
                       &ni);
      ++ck;
      // a half tile is rows 128 (bid & 1) .. + 127 of the 256-row tile
      const int64_t rbase = (int64_t)mi * kBM + (kHalf ? (bid & 1) * 128 : 0) + wm * (ROWS * 16);
      const int64_t cbase = (int64_t)ni * kBN + wn * 64;
      void *c = g.c;
      bool lok = line_ok, vok = vec_ok;
      if (BATCHED) {
        c = entry_of(g, e).c;
        lok = c_line_ok<OUT_BF16>(c, g.ldc);
        vok = c_vec_ok<OUT_BF16>(c, g.ldc);
      }
      if (lok && rbase + ROWS * 16 <= g.M && cbase + 64 <= g.N) {
        store_tile_lds<OUT_BF16, ROWS>(g, c, acc, slab, rbase, cbase, lr, lg);
      } else {
        const int64_t row0 = rbase + lr, col0 = cbase + 4 * lg;
#pragma unroll
        for (int i = 0; i < ROWS; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            store_quad_vec<OUT_BF16>(g, c, acc[i][j], row0 + i * 16, col0 + j * 16, vok);
      }
#pragma unroll
      for (int i = 0; i < ROWS; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // two 64-bit moves per accumulator (the compiler otherwise copies a
          // zero register four times): 64 instead of 128 VALU instructions
          // per tile, about 1% on K = 4096 GEMMs (bitwise identical)
          double lo, hi;
          asm volatile("v_mov_b64 %0, 0" : "=v"(lo));
          asm volatile("v_mov_b64 %0, 0" : "=v"(hi));
          acc[i][j] = __builtin_bit_cast(v4f, d2{lo, hi});
        }
    }
  }
  if (!SHIFTED) __syncthreads();                           // the shifted consumers' last barrier
}

// Persistent: one workgroup per compute unit walks the tiles bid, bid + grid,
// ... of [tile_base, tile_base + tile_count) as one continuous sequence of
// stages; producers run three stages ahead across tile boundaries, and
// consumers store a finished tile while the next tile's first stages are
// already in flight.
//
// HALF = 1 is the tail launch: workgroup bid computes half bid & 1 (rows
// 128 (bid & 1) .. + 127) of tile tile_base + (bid >> 1), with the same
// twelve waves: consumers on 64x64 pieces (4 rows of 4 MFMAs), producers
// copying the half's 8 A row groups and all 16 of B. Each output element
// sees the same MFMAs in the same order as in a whole tile.
//
// BATCHED: a grouped launch (GemmArgs::batch entries of one shape, their tile
// rows stacked into one grid); each tile takes its entry's operands and
// output. Single GEMMs use the instances without it.
template <int OUT_BF16, int HALF, bool BATCHED>
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRing * kStageBytes + kConsumers * kSlab];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0..11
  const bool producer = wave >= kConsumers;
  const int wm = (wave >> 2) & 1, wn = wave & 3;               // consumers: 2 x 4 grid
  const int tm = (int)((g.M + kBM - 1) / kBM), tn = (int)((g.N + kBN - 1) / kBN);
  const int grid = (int)gridDim.x, bid = (int)blockIdx.x;
  const int ntl = HALF ? 1 : (g.tile_count - bid + grid - 1) / grid;   // tiles of this workgroup
  const int half = HALF ? (bid & 1) : 0;
  const int mp = (int)((g.M + 255) & ~255LL), np = (int)((g.N + 255) & ~255LL);   // padded rows
  const int nslices = (int)((g.K + 127) >> 7);
  const int total = ntl * nslices;                             // stages of this workgroup
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  const int lr = lane & 15;      // row within a 16-row MFMA tile
  const int lg = lane >> 4;      // 32-element K block within the slice

  if (producer) {
    // Producer p copies row groups 4p .. 4p + 3 of A (2p, 2p + 1 of the
    // half for HALF) and of B (1 KB tiles); producer 0 also copies the
    // stage's A scales and producer 1 its B scales: the 1 KB block of (K
    // slice, 256-row panel), copied whole. Stages past the last one read
    // zeros so the counts stay uniform.
    const int p = wave - kConsumers;
    const int a_bytes = mp * nslices * 64, b_bytes = np * nslices * 64;
    const int sa_bytes = nslices * mp * 4, sb_bytes = nslices * np * 4;
    const v4i rsrc_a0 = make_rsrc(g.a_codes, (uint32_t)a_bytes);
    const v4i rsrc_b0 = make_rsrc(g.b_codes, (uint32_t)b_bytes);
    const v4i rsrc_s0 = p == 0 ? make_rsrc(g.a_scales, (uint32_t)sa_bytes)
                               : make_rsrc(g.b_scales, (uint32_t)sb_bytes);
    // a grouped launch switches them to each tile's entry
    v4i rsrc_a = rsrc_a0, rsrc_b = rsrc_b0, rsrc_s = rsrc_s0;
    const int s_panels = (p == 0 ? mp : np) >> 8;              // 256-row panels
    const int s_bytes = p == 0 ? sa_bytes : sb_bytes;
    const int s_lane = lane * 16;
    int ga = 0, gb = 0, gs = 0;
    bool tile_live = false;
    auto set_tile = [&](int k) {
      tile_live = k < ntl;
      int e = 0, mi = 0, ni = 0;
      if (tile_live)
        tile_of<BATCHED>(g, g.tile_base + (HALF ? (bid >> 1) : bid + k * grid), tm, tn, &e, &mi,
                         &ni);
      if (BATCHED && tile_live) {                              // this tile's entry
        const GemmEntry en = entry_of(g, e);
        rsrc_a = uniform(make_rsrc(en.a_codes, (uint32_t)a_bytes));
        rsrc_b = uniform(make_rsrc(en.b_codes, (uint32_t)b_bytes));
        rsrc_s = uniform(p == 0 ? make_rsrc(en.a_scales, (uint32_t)sa_bytes)
                                : make_rsrc(en.b_scales, (uint32_t)sb_bytes));
      }
      ga = mi * (kBM / 16) + (HALF ? half * 8 + p * 2 : p * 4);
      gb = ni * (kBN / 16) + p * 4;
      gs = p == 0 ? mi : ni;                                   // the tile's panel
    };
    int ik = 0, is = 0;                                        // next stage to copy
    set_tile(0);
    auto issue = [&](int buf) {
      // the copies take their buffer resources in scalar registers
      const v4i ra = BATCHED ? uniform(rsrc_a) : rsrc_a0;
      const v4i rb = BATCHED ? uniform(rsrc_b) : rsrc_b0;
      const v4i rs = BATCHED ? uniform(rsrc_s) : rsrc_s0;
      const uint32_t stage = smem_base + (uint32_t)(buf * kStageBytes);
      int al = ga * nslices * 1024 + lane * 16, bl = gb * nslices * 1024 + lane * 16;
      int sl = s_lane + gs * 1024;
      asm volatile("" : "+v"(al), "+v"(bl), "+v"(sl));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int off = (j * nslices + is) * 1024;
        const uint32_t dst = __builtin_amdgcn_readfirstlane(stage + (uint32_t)((p * 4 + j) * 1024));
        if (!HALF || j < 2)
          dma_load16(ra, tile_live ? al + off : a_bytes,
                     HALF ? __builtin_amdgcn_readfirstlane(stage + (uint32_t)((p * 2 + j) * 1024))
                          : dst);
        dma_load16(rb, tile_live ? bl + off : b_bytes, dst + kStageA);
      }
      if (p < 2)
        dma_load16(rs, tile_live ? sl + is * s_panels * 1024 : s_bytes,
                   __builtin_amdgcn_readfirstlane(
                       stage + (uint32_t)(kStageA + kStageB + (p == 0 ? 0 : kStageSA))));
      if (++is == nslices) {
        is = 0;
        set_tile(++ik);
      }
    };
    for (int G = 0; G < kAhead; ++G) issue(G);
    for (int G = 0; G < total; ++G) {
      // own part of stage G landed: nine copies per stage on producers 0
      // and 1, eight on 2 and 3 (seven and six for HALF), two later stages
      // outstanding
      if (HALF) {
        if (p < 2)
          asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      } else {
        if (p < 2)
          asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      }
      __syncthreads();                                     // stage G visible; G - 1 free
      issue((G + kAhead) & 3);
    }
    __syncthreads();                                       // the shifted consumers' last barrier
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // zero-fill loads past the end
    return;
  }

  // consumers
  const bool line_ok = c_line_ok<OUT_BF16>(g.c, g.ldc);
  const bool vec_ok = c_vec_ok<OUT_BF16>(g.c, g.ldc);
  constexpr int kRows = HALF ? 4 : 8;                          // MFMA rows per consumer
  const uint32_t a_off = (uint32_t)((wm * kRows) * 1024 + lane * 16);
  const uint32_t b_off = (uint32_t)(kStageA + (wn * 4) * 1024 + lane * 16);
  // scales: the 256 B at quarter hq of a scale block hold byte hq * 4 + j
  // (row group) of every lane's (row lr, block lg) at lane * 4, so each read
  // is one linear 256-byte span; this wave's A rows are groups
  // 8 wm .. 8 wm + 7 (quarters 2 wm, 2 wm + 1; for HALF, groups
  // 8 half + 4 wm .. + 3, quarter 2 half + wm), its B rows groups
  // 4 wn .. 4 wn + 3 (quarter wn)
  const uint32_t sa_off = (uint32_t)(kStageA + kStageB) +
                          (HALF ? (2 * half + wm) * 256 : wm * 512) + lane * 4;
  const uint32_t sb_off = (uint32_t)(kStageA + kStageB + kStageSA) + wn * 256 + lane * 4;
  if (wm == 1)
    consumer_loop<OUT_BF16, true, kRows, BATCHED>(g, smem, total, nslices, bid, grid, tm, tn, vec_ok,
                                         line_ok, a_off, b_off, sa_off, sb_off, lr, lg, wm, wn);
  else
    consumer_loop<OUT_BF16, false, kRows, BATCHED>(g, smem, total, nslices, bid, grid, tm, tn, vec_ok,
                                          line_ok, a_off, b_off, sa_off, sb_off, lr, lg, wm, wn);
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

// Compute units of the current device (one persistent workgroup each).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t gemm_launch(const GemmArgs &g, hipStream_t stream) {
  if (g.batch < 1 || g.batch > kMaxGemmBatch) return hipErrorInvalidValue;
  if (g.K == 0) {
    const int64_t total = g.M * g.N;
    const dim3 grid((unsigned)((total + 255) / 256));
    hipError_t e = hipSuccess;
    for (int i = 0; i < g.batch && e == hipSuccess; ++i) {
      GemmArgs z = g;
      if (i > 0) z.c = g.more[i - 1].c;
      e = g.out_bf16 ? launch(fill_zero_kernel<1>, grid, dim3(256), 0, stream, z)
                     : launch(fill_zero_kernel<0>, grid, dim3(256), 0, stream, z);
    }
    return e;
  }
  // a grouped launch stacks the entries' tile rows into one tall grid
  const int64_t tiles = ((g.M + kBM - 1) / kBM) * g.batch * ((g.N + kBN - 1) / kBN);
  const int64_t cus = cu_count();
  // When the last round of whole tiles would fill at most half the compute
  // units (e.g. 896 tiles = 3.5 rounds on 256, or 64 tiles in all), the
  // whole rounds run first and the leftover tiles then run as twice as many
  // half tiles, one per workgroup.
  const int64_t rem = tiles % cus;
  const bool split = rem != 0 && 2 * rem <= cus;
  GemmArgs a = g;
  a.tile_base = 0;
  a.tile_count = (int)(split ? tiles - rem : tiles);
  hipError_t e = hipSuccess;
  // single GEMMs keep an instance without the grouped launch's per-tile
  // entry logic (measured 2-5% faster than sharing the grouped instance)
  const bool b = g.batch > 1;
  if (a.tile_count > 0) {
    const dim3 grid((unsigned)std::min<int64_t>(a.tile_count, cus));
    auto k = g.out_bf16 ? (b ? gemm_tiled_kernel<1, 0, true> : gemm_tiled_kernel<1, 0, false>)
                        : (b ? gemm_tiled_kernel<0, 0, true> : gemm_tiled_kernel<0, 0, false>);
    e = launch(k, grid, dim3(kThreads), 0, stream, a);
  }
  if (e != hipSuccess || !split) return e;
  GemmArgs h = g;
  h.tile_base = a.tile_count;
  h.tile_count = (int)rem;
  const dim3 hgrid((unsigned)(2 * rem));
  auto k = g.out_bf16 ? (b ? gemm_tiled_kernel<1, 1, true> : gemm_tiled_kernel<1, 1, false>)
                      : (b ? gemm_tiled_kernel<0, 1, true> : gemm_tiled_kernel<0, 1, false>);
  return launch(k, hgrid, dim3(kThreads), 0, stream, h);
}

}  // namespace mx
