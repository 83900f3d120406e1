// Internal launch interface between the C ABI (mx_api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace mx {

// Launch `kernel` and return that launch's own status (never a sticky error
// left behind by an unrelated earlier HIP call). Arguments are converted to
// the kernel's exact parameter types before their addresses are taken.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> params{static_cast<KArgs>(args)...};
  void *ptrs[sizeof...(KArgs)];
  std::apply([&](auto &...p) {
    int i = 0;
    ((ptrs[i++] = static_cast<void *>(&p)), ...);
  }, params);
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, shmem, stream);
}

enum { MX_K_ROT_NONE = 0, MX_K_ROT_HADAMARD = 1, MX_K_ROT_RAND_SIGN = 2, MX_K_ROT_HADAMARD16 = 3 };
enum { MX_K_ROUND_RNE = 0, MX_K_ROUND_SR = 1 };

struct QuantArgs {
  const uint16_t *x;   // bf16 [rows, cols], leading dimension ld
  int64_t rows, cols, ld;
  int axis;            // 0 or 1
  int rotate, round;
  uint32_t seed_lo, seed_hi;
  uint8_t *codes;      // tiled codes
  uint8_t *scales;     // tiled scales
  int rb;              // axis-0 row blocks per lane (0 = default)
  int fmt;             // 0: E2M1 (MXFP4), 1: E4M3 (MXFP8 comparator, RNE only)
};

hipError_t quantize_launch(const QuantArgs &a, hipStream_t stream);

// Two axis-1 MXFP4 quantizations of sources with the same column count (and
// the same rotation and rounding) in one launch.
hipError_t quantize_pair_launch(const QuantArgs &a, const QuantArgs &b, hipStream_t stream);

// Both orientations of one source (rows % 32 == 0, cols % 32 == 0).
struct DualArgs {
  const uint16_t *x;   // bf16 [rows, cols], leading dimension ld
  int64_t rows, cols, ld;
  int rotate, round;
  uint32_t seed1_lo, seed1_hi;   // axis-1 operand
  uint32_t seed0_lo, seed0_hi;   // axis-0 operand
  uint8_t *codes1, *scales1;
  uint8_t *codes0, *scales0;
};

hipError_t quantize_dual_launch(const DualArgs &a, hipStream_t stream);

// Operands and output of one GEMM of a grouped launch.
struct GemmEntry {
  const uint8_t *a_codes, *a_scales;
  const uint8_t *b_codes, *b_scales;
  void *c;
};

constexpr int kMaxGemmBatch = 4;

struct GemmArgs {
  const uint8_t *a_codes, *a_scales;  // [M][K/2], [M][K/32]
  const uint8_t *b_codes, *b_scales;  // [N][K/2], [N][K/32]
  void *c;                            // [M][N], leading dimension ldc
  int64_t M, N, K, ldc;
  int out_bf16;
  // Set by the launcher: the output tiles (in its ordering) one launch of
  // the MXFP4 GEMM covers, [tile_base, tile_base + tile_count).
  int tile_base, tile_count;
  // Grouped launch (MXFP4 only): `batch` GEMMs of this one shape, entry 0 in
  // the fields above and entry e > 0 in more[e - 1]. Their tile rows are
  // stacked into one tall grid: tile row i of entry e is row e * tiles_m + i.
  int batch = 1;
  GemmEntry more[kMaxGemmBatch - 1] = {};
};

hipError_t gemm_launch(const GemmArgs &g, hipStream_t stream);

// The MXFP8 (E4M3) comparator GEMM on the same tiled operands (2 KB code
// tiles); same arguments.
hipError_t gemm_e4m3_launch(const GemmArgs &g, hipStream_t stream);

// Compute units of the current device (one persistent GEMM workgroup each).
int cu_count();

// fp32 values of a packed operand in its source's shape.
struct DequantArgs {
  const uint8_t *codes, *scales;   // tiled (E2M1 or E4M3 codes)
  int64_t mn, k, mnp, kp;          // operand extents and their padded ones
  int axis;                        // source orientation: 1 -> [mn][k], 0 -> [k][mn]
  int fmt;                         // 0: E2M1, 1: E4M3
  float *out;                      // leading dimension ld
  int64_t ld;
};

hipError_t dequantize_launch(const DequantArgs &a, hipStream_t stream);

}  // namespace mx
