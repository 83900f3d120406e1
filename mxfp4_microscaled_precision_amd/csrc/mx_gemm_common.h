// Pieces shared by the gfx950 GEMM kernels (MXFP4 and the MXFP8 comparator):
// vector types, the bf16 epilogue conversion and stores, raw buffer
// resources with direct-to-LDS loads, and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_kernels.h"

namespace mx {
namespace gemm {

constexpr int kBM = 256;                           // block tile rows (A)
constexpr int kBN = 256;                           // block tile columns (B)
constexpr int kGroupM = 4;                         // tile rows per ordering group (measured best of 2, 4, 8, 16)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));


// Two fp32 values as packed bf16, the first in the low half: gfx950's
// v_cvt_pk_bf16_f32, round to nearest even. Measured on every one of the
// 2^32 fp32 patterns: identical to the integer rule (u + 0x7FFF + bit 16)
// >> 16 for non-NaN u, and to (u >> 16) | 0x40 (sign and payload kept,
// quieted) for NaN. One instruction per two elements instead of about six
// per element, which kept the epilogue's VALU work off the matrix core's
// critical path.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return (uint16_t)pack_bf16x2_rne(f, 0.f);
}

// Generic epilogue store of one quad: lane (lr, lg) of a 16x16 tile holds
// C[row][col .. col + 3] with row = tile row + lr, col = tile col + 4 lg.
// Element-wise and masked, for shapes the row-staged path does not take.
// c is the output (g.c, or a grouped launch's entry's); g gives its extents
// and row pitch.
template <int OUT_BF16>
__device__ __forceinline__ void store_quad(const GemmArgs &g, void *c, const v4f &acc, int64_t row,
                                           int64_t col) {
  if (row >= g.M) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (col + r < g.N) {
      if (OUT_BF16)
        reinterpret_cast<uint16_t *>(c)[row * g.ldc + col + r] = f32_to_bf16_rne(acc[r]);
      else
        reinterpret_cast<float *>(c)[row * g.ldc + col + r] = acc[r];
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

// Direct-to-LDS load: lane i's 16 bytes from rsrc.base + voffset land at LDS
// byte address lds_base + 16 i. Written as inline asm so that the
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


// Tile index -> (tile_m, tile_n): workgroups are dispatched round-robin over
// the 8 XCDs, so consecutive ids are first regrouped per XCD, then ordered in
// groups of kGroupM tile rows so that each XCD works on a compact 2-D region
// of C and shares its A and B panels through its own L2.
__device__ __forceinline__ void tile_coords(int bid, int tm, int tn, int *mi, int *ni) {
  const int T = tm * tn;
  int id = bid;
  if ((T & 7) == 0) id = (bid & 7) * (T >> 3) + (bid >> 3);
  const int per_group = kGroupM * tn;
  const int grp = id / per_group;
  const int first_m = grp * kGroupM;
  const int gm = min(kGroupM, tm - first_m);
  const int r = id - grp * per_group;
  *mi = first_m + r % gm;
  *ni = r / gm;
}

// One finished quad: lane (lr, lg) of a 16x16 tile holds C[row][col .. col + 3]
// (B is the MFMA's first operand). One 8-byte (bf16) or 16-byte (fp32)
// store when the address allows it, else element-wise.
template <int OUT_BF16>
__device__ __forceinline__ void store_quad_vec(const GemmArgs &g, void *c, const v4f &acc,
                                               int64_t row, int64_t col, bool vec_ok) {
  if (row >= g.M) return;
  if (vec_ok && col + 3 < g.N) {
    if (OUT_BF16) {
      uint2 v;
      v.x = pack_bf16x2_rne(acc[0], acc[1]);
      v.y = pack_bf16x2_rne(acc[2], acc[3]);
      *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(c) + row * g.ldc + col) = v;
    } else {
      *reinterpret_cast<float4 *>(reinterpret_cast<float *>(c) + row * g.ldc + col) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  } else {
    store_quad<OUT_BF16>(g, c, acc, row, col);
  }
}

constexpr int kSlab = 2048;                        // epilogue staging per 128x64 wave tile

// Stores a finished (16 ROWS)x64 wave tile (rows row0.., columns col0..) through
// the wave's private 2 KB LDS slab, 16 rows at a time: lane (lr, lg) writes
// its quads of row lr, then lane l reads back 16 contiguous bytes of row
// l / 8 (chunk l % 8) and stores them, so that each store instruction
// writes eight whole 128-byte row segments instead of sixteen 32-byte
// pieces. Chunk c of slab row r sits at chunk c ^ (r & 7) (fewer bank
// conflicts for the column-strided writes). A wave's LDS operations run in
// order, so a slab row group is read back before the next overwrites it.
// Measured on the MXFP4 kernel against the direct quad stores (bitwise
// identical output): Fprop 70.7 -> 61.0 us, Dgrad 236 -> 204 us, Wgrad (fp32
// out) 228 -> 222 us. Wave tiles that cross the edge of C, or a C that is not
// 16-byte aligned, keep the quad stores.
template <int OUT_BF16, int ROWS>
__device__ __forceinline__ void store_tile_lds(const GemmArgs &g, void *c,
                                               const v4f (&acc)[ROWS][4], uint8_t *slab,
                                               int64_t row0, int64_t col0, int lr, int lg) {
  // Opaque copies: keeps the compiler from hoisting these lane addresses
  // out of the stage loop, where they would hold registers the MFMA loop
  // needs.
  asm volatile("" : "+v"(lr), "+v"(lg));
  const int lane = lg * 16 + lr;
  const int rr = lane >> 3, ch = lane & 7;                 // read-back row (of 8), chunk
  // byte address of this lane's first 16 bytes (row row0 + rr); each further
  // 8 rows add `step`, the fp32 halves add 128 bytes (an immediate offset)
  constexpr int kEsize = OUT_BF16 ? 2 : 4;
  const int64_t step = 8 * g.ldc * kEsize;
  uint8_t *pi = reinterpret_cast<uint8_t *>(c) + ((row0 + rr) * g.ldc + col0) * kEsize + ch * 16;
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
#pragma unroll
    for (int h = 0; h < (OUT_BF16 ? 1 : 2); ++h) {
      if (OUT_BF16) {
        // row of 64 bf16 = 128 B: quad j of lane lg is bytes 32 j + 8 lg
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 2 * j + (lg >> 1);
          uint2 v;
          v.x = pack_bf16x2_rne(acc[i][j][0], acc[i][j][1]);
          v.y = pack_bf16x2_rne(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<uint2 *>(slab + lr * 128 + ((c ^ (lr & 7)) << 4) + ((lg & 1) << 3)) = v;
        }
      } else {
        // columns 32 h .. 32 h + 31 as fp32 = 128 B: quad 2 h + jj of lane
        // lg is bytes 64 jj + 16 lg
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int c = jj * 4 + lg;
          *reinterpret_cast<v4f *>(slab + lr * 128 + ((c ^ (lr & 7)) << 4)) = acc[i][2 * h + jj];
        }
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int r = k * 8 + rr;
        const v4i d = *reinterpret_cast<const v4i *>(slab + r * 128 + ((ch ^ (r & 7)) << 4));
        // fp32 tiles (Wgrad) store non-temporally: measured 2-3% faster
        // there; the bf16 ops measured slower with it and keep plain stores
        if (OUT_BF16)
          *reinterpret_cast<v4i *>(pi + k * step + h * 128) = d;
        else
          __builtin_nontemporal_store(d, reinterpret_cast<v4i *>(pi + k * step + h * 128));
      }
    }
    pi += 2 * step;
  }
}

}  // namespace gemm
}  // namespace mx
