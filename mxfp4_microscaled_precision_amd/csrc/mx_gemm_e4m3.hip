// MXFP8 (E4M3) comparator GEMM on gfx950's block-scaled matrix cores, fp32
// accumulation, on the same tiled, reduction-major operands as the MXFP4
// GEMM:
//
//   C[m][n] = sum_k A(m, k) * B(n, k),   A(m, k) = E4M3(a) * 2^(sa - 127)
//
// The pages measure MXFP4 training against an FP8 baseline (36Kr article
// "Neue Studie von AMD durchbricht die bestehende Erkenntnis ...", opening
// section: FP4 has in theory twice FP8's compute; section
// "Ende-zu-Ende-Effizienz": the step-throughput gain over FP8); the ShowAPI
// page "AMD颠覆认知：FP4不稳定性的真正原因", section 2.2, names E4M3 as an FP8
// format. This kernel is that comparator: same 32-element blocks and E8M0
// scales, E4M3 elements, so the two kernels' speeds can be set side by side.
//
// Instruction: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in FP8
// E4M3 (format code 0). Lane l = 16 g + r supplies row r of A and of B as 32
// bytes: bytes 0..15 are K elements [16 g, 16 g + 16) of the 128-wide slice
// and bytes 16..31 are [64 + 16 g, 64 + 16 g + 16); the E8M0 scale of
// 32-element block b (K [32 b, 32 b + 32)) is the one lane group b supplies
// through the byte select (measured on gfx950 with one-hot operands and
// distinct per-group scales). As in the MXFP4 kernel B is the first operand,
// so lane l receives C[r][4 g + i], i = 0..3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <utility>

#include "mx_gemm_common.h"
#include "mx_kernels.h"

namespace mx {

namespace {

using namespace gemm;

constexpr int kFmtE4M3 = 0;

template <int SELA, int SELB>
__device__ __forceinline__ v4f mfma_e4m3(const v8i &a, const v8i &b, v4f c, uint32_t sa,
                                         uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtE4M3, kFmtE4M3, SELA,
                                                          (int)sa, SELB, (int)sb);
}

// ---------------------------------------------------------------------------
// 256x256 block tile, eight waves (two per SIMD) in a 2x4 grid of 128x64
// each, 8x4 MFMA tiles per wave. An E4M3 code tile (16 rows x 128 K) is
// 2 KB stored as [16-element chunk j][row r][16 B], so lane l's MFMA
// fragment (chunks g and g + 4 of row r) is the 16 bytes at 16 l and at
// 1024 + 16 l: two contiguous 1 KB LDS reads per fragment. A stage (one
// 128-wide K slice) is 32 KB of A codes, 32 KB of B codes and the two 1 KB
// scale blocks; two stage buffers (132 KB of LDS) alternate, so one stage is
// in flight while the other is consumed. Every
// wave copies its share of the next stage (four 1 KB A pieces, four B
// pieces, waves 0 and 1 also a scale block) with direct-to-LDS loads, one
// per MFMA row so that the copies interleave with the matrix work. With the
// larger fragments a wave needs about 200 registers, which leaves no room for
// separate copy waves next to eight consumers.
// ---------------------------------------------------------------------------
constexpr int kThreads = 512;
constexpr int kStageA = kBM * 128;                 // 16 tiles of 2 KB
constexpr int kStageB = kBN * 128;
constexpr int kStageS = 2048;                      // A scale block, then B's
constexpr int kStageBytes = kStageA + kStageB + kStageS;
constexpr int kRing = 2;                           // 132 KB

__device__ __forceinline__ v8i load_frag(const uint8_t *p) {
  const uint4 lo = *reinterpret_cast<const uint4 *>(p);
  const uint4 hi = *reinterpret_cast<const uint4 *>(p + 1024);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Row I of a wave's stage: issue copy I of the next stage (if any), read A
// fragment I + 1, then the 4 MFMAs of row I. B is the first MFMA operand
// (scale byte j of sb), A the second (byte I % 4 of sa.x for rows 0..3, of
// sa.y for rows 4..7).
template <int I, typename Copy>
__device__ __forceinline__ void consume_row(v4f (&acc)[8][4], const v8i (&bf)[4], v8i (&af)[8],
                                            const uint8_t *a_base, uint32_t sb, uint2 sa,
                                            const Copy &copy) {
  copy(I);
  if (I + 1 < 8) af[I + 1 < 8 ? I + 1 : 0] = load_frag(a_base + (I + 1) * 2048);
  const uint32_t sai = I < 4 ? sa.x : sa.y;
  acc[I][0] = mfma_e4m3<0, I & 3>(bf[0], af[I], acc[I][0], sb, sai);
  acc[I][1] = mfma_e4m3<1, I & 3>(bf[1], af[I], acc[I][1], sb, sai);
  acc[I][2] = mfma_e4m3<2, I & 3>(bf[2], af[I], acc[I][2], sb, sai);
  acc[I][3] = mfma_e4m3<3, I & 3>(bf[3], af[I], acc[I][3], sb, sai);
  __builtin_amdgcn_sched_barrier(0);
}

template <typename Copy, int... I>
__device__ __forceinline__ void consume_rows(std::integer_sequence<int, I...>, v4f (&acc)[8][4],
                                             const v8i (&bf)[4], v8i (&af)[8],
                                             const uint8_t *a_base, uint32_t sb, uint2 sa,
                                             const Copy &copy) {
  (consume_row<I>(acc, bf, af, a_base, sb, sa, copy), ...);
}

// Persistent: one workgroup per compute unit walks the tiles bid, bid + grid,
// ... as one continuous sequence of stages; the copy of a tile's first stage
// overlaps the previous tile's last stage.
template <int OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void gemm_e4m3_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRing * kStageBytes + 8 * kSlab];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0..7
  const int wm = wave >> 2, wn = wave & 3;                     // 2 x 4 grid
  const int tm = (int)((g.M + kBM - 1) / kBM), tn = (int)((g.N + kBN - 1) / kBN);
  const int tiles = tm * tn;
  const int grid = (int)gridDim.x, bid = (int)blockIdx.x;
  const int ntl = (tiles - bid + grid - 1) / grid;             // tiles of this workgroup
  const int mp = (int)((g.M + 255) & ~255LL), np = (int)((g.N + 255) & ~255LL);
  const int nslices = (int)((g.K + 127) >> 7);
  const int total = ntl * nslices;                             // stages of this workgroup
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  const int lr = lane & 15;
  const int lg = lane >> 4;

  // ---- copies: wave w moves 1 KB pieces 4w .. 4w + 3 of the stage's A
  // codes and of its B codes (piece p = half p % 2, i.e. chunks 4 (p % 2) ..
  // 4 (p % 2) + 3, of row group p / 2), wave 0 the A scale block and wave 1
  // the B scale block of (slice, panel).
  const int a_bytes = mp * nslices * 128, b_bytes = np * nslices * 128;
  const v4i rsrc_a = make_rsrc(g.a_codes, (uint32_t)a_bytes);
  const v4i rsrc_b = make_rsrc(g.b_codes, (uint32_t)b_bytes);
  const v4i rsrc_s = wave == 0 ? make_rsrc(g.a_scales, (uint32_t)(nslices * mp * 4))
                               : make_rsrc(g.b_scales, (uint32_t)(nslices * np * 4));
  const int s_panels = (wave == 0 ? mp : np) >> 8;
  int ik = 0, is = 0;                                          // next stage to copy
  int ga = 0, gb = 0, gs = 0;
  auto set_tile = [&](int k) {
    int mi = 0, ni = 0;
    if (k < ntl) tile_coords(bid + k * grid, tm, tn, &mi, &ni);
    ga = mi * (kBM / 16);
    gb = ni * (kBN / 16);
    gs = wave == 0 ? mi : ni;
  };
  set_tile(0);
  // copy j of the stage at LDS address `stage`: j = 0..3 A pieces, 4..7 B pieces;
  // the scale block goes with j = 0
  auto copy_one = [&](int j, uint32_t stage) {
    const int piece = wave * 4 + (j & 3);
    const int grp = piece >> 1, half = piece & 1;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        stage + (uint32_t)((j < 4 ? 0 : kStageA) + piece * 1024));
    const int off = (((j < 4 ? ga : gb) + grp) * nslices + is) * 2048 + half * 1024 + lane * 16;
    dma_load16(j < 4 ? rsrc_a : rsrc_b, off, dst);
    if (j == 0 && wave < 2)
      dma_load16(rsrc_s, lane * 16 + (is * s_panels + gs) * 1024,
                 __builtin_amdgcn_readfirstlane(stage + (uint32_t)(kStageA + kStageB + wave * 1024)));
  };
  auto advance = [&]() {
    if (++is == nslices) {
      is = 0;
      set_tile(++ik);
    }
  };
#pragma unroll
  for (int j = 0; j < 8; ++j) copy_one(j, smem_base);
  advance();

  // ---- consumers
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(g.c) & (OUT_BF16 ? 7 : 15)) == 0) &&
                      ((g.ldc & 3) == 0);
  // whole 16-byte stores through the wave's LDS slab: C and its row pitch
  // 16-byte aligned
  const bool line_ok = ((reinterpret_cast<uintptr_t>(g.c) & 15) == 0) &&
                       ((g.ldc * (OUT_BF16 ? 2 : 4)) & 15) == 0;
  uint8_t *slab = smem + kRing * kStageBytes + wave * kSlab;
  const uint32_t a_off = (uint32_t)((wm * 8) * 2048 + lane * 16);
  const uint32_t b_off = (uint32_t)(kStageA + (wn * 4) * 2048 + lane * 16);
  // scales: the 256 B at quarter hq of a scale block hold byte hq * 4 + j
  // (row group) of every lane's (row lr, block lg) at lane * 4, so each read
  // is one linear 256-byte span; this wave's A rows are groups
  // 8 wm .. 8 wm + 7 (quarters 2 wm, 2 wm + 1), its B rows groups
  // 4 wn .. 4 wn + 3 (quarter wn)
  const uint32_t sa_off = (uint32_t)(kStageA + kStageB) + wm * 512 + lane * 4;
  const uint32_t sb_off = (uint32_t)(kStageA + kStageB + 1024) + wn * 256 + lane * 4;
  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  int ck = 0, cs = 0;
  for (int G = 0; G < total; ++G) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // own copies of stage G landed
    __syncthreads();                                       // all of stage G; G - 1 consumed
    const uint8_t *base = smem + (G & 1) * kStageBytes;
    const bool more = G + 1 < total;
    const uint32_t next = smem_base + (uint32_t)(((G + 1) & 1) * kStageBytes);
    auto copy = [&](int j) {
      if (more) copy_one(j, next);
    };
    v8i bf[4], af[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = load_frag(base + b_off + j * 2048);
    const uint32_t sb = *reinterpret_cast<const uint32_t *>(base + sb_off);
    const uint2 sa = make_uint2(*reinterpret_cast<const uint32_t *>(base + sa_off),
                                *reinterpret_cast<const uint32_t *>(base + sa_off + 256));
    af[0] = load_frag(base + a_off);
    consume_rows(std::make_integer_sequence<int, 8>{}, acc, bf, af, base + a_off, sb, sa, copy);
    if (more) advance();
    if (++cs == nslices) {
      cs = 0;
      int mi, ni;
      tile_coords(bid + ck * grid, tm, tn, &mi, &ni);
      ++ck;
      const int64_t rbase = (int64_t)mi * kBM + wm * 128, cbase = (int64_t)ni * kBN + wn * 64;
      if (line_ok && rbase + 128 <= g.M && cbase + 64 <= g.N) {
        store_tile_lds<OUT_BF16, 8>(g, g.c, acc, slab, rbase, cbase, lr, lg);
      } else {
        const int64_t row0 = rbase + lr, col0 = cbase + 4 * lg;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            store_quad_vec<OUT_BF16>(g, g.c, acc[i][j], row0 + i * 16, col0 + j * 16, vec_ok);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

hipError_t gemm_e4m3_launch(const GemmArgs &g, hipStream_t stream) {
  if (g.K == 0) return gemm_launch(g, stream);             // C = 0, codes never read
  const int64_t tiles = ((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
  const dim3 grid((unsigned)std::min<int64_t>(tiles, cu_count()));
  return g.out_bf16 ? launch(gemm_e4m3_kernel<1>, grid, dim3(kThreads), 0, stream, g)
                    : launch(gemm_e4m3_kernel<0>, grid, dim3(kThreads), 0, stream, g);
}

}  // namespace mx
