"""Plain, slow CPU oracle of the MXFP4 linear-layer triple (NumPy, fp64 GEMM).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg; never by the product path.

Sources (the three web pages on AMD's MXFP4 pretraining study):
  [36Kr]  "Neue Studie von AMD durchbricht die bestehende Erkenntnis: Die
          Instabilitaet von FP4-Training liegt nicht an unzureichender
          Zufaelligkeit" (eu.36kr.com, German).
  [HTX]   "New AMD paper overturns conventional wisdom: FP4 training ..."
          (htx.com news, Indonesian translation of the same article).
  [ShowAPI] "AMD颠覆认知：FP4不稳定性的真正原因" (showapi.com).

What the pages fix, and the readings taken where they are silent:
  * [36Kr] "Was ist MXFP4?" / [HTX] "Apa itu MXFP4": a tensor is cut into
    blocks of 32 elements; each block shares one exponent stored as E8M0;
    each element is a 4-bit float rounded to the nearest representable
    value; the shared exponent is "the largest exponent in the block".
    The reconstruction formula itself is missing from both pages. Reading
    (OCP MX, the standard the pages name in "Fazit"): value = 2^(s-127) *
    E2M1(code), and the block exponent is floor(log2(amax)) - 2, the "-2"
    being E2M1's largest exponent so that the block maximum lands in [4, 8).
  * [ShowAPI] section 2.2: FP4 is 1 sign, 2 exponent, 1 mantissa bit.
    Reading (OCP E2M1): exponent bias 1, subnormal step 0.5, no Inf/NaN, so
    the magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
  * Ties go to the even mantissa bit; magnitudes beyond 6 saturate to 6.
  * [36Kr] "Fehlerdiagnoseexperiment": stochastic rounding makes the expected
    rounding error zero; the randomized Hadamard flips signs at random before
    the transform; the deterministic Hadamard applies the same orthogonal
    transform every step, before quantization. [36Kr] "Ende-zu-Ende-Effizienz"
    labels the stabilised run "H16": the variant rotate="hadamard16" applies
    block-diag(H16, H16) / 4 inside each 32-element block (4 butterfly stages,
    an exact normalisation). Readings: the default rotation is the
    32-point Sylvester Hadamard H (H_ij = (-1)^popcount(i&j)) scaled by
    c = fp32(1/sqrt(32)), block-diagonal along the GEMM reduction axis and
    aligned with the MX blocks; evaluated in fp32 as a radix-2 butterfly with
    strides 1, 2, 4, 8, 16 (lower index gets a+b, upper gets a-b), then one
    fp32 multiply by c. Random signs: one per reduction index, shared by both
    GEMM operands, from Philox4x32-10. Stochastic rounding picks the upper
    neighbour with probability (a - lo) / (hi - lo) using a 24-bit uniform
    from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
    as easy as 1, 2, 3", SC'11).
  * [36Kr] "Fehlerdiagnoseexperiment": Fprop Y = X W^T, Dgrad dX = dY W,
    Wgrad dW = dY^T X. The GEMM is the exact sum over dequantized values,
    evaluated here in fp64.
  * Comparator: [36Kr] intro and "Ende-zu-Ende-Effizienz" measure MXFP4
    against FP8; [ShowAPI] section 2.2 names E4M3 and E5M2 as the FP8
    formats. Reading: the FP8 comparator is MXFP8 with E4M3 elements (OCP:
    bias 7, subnormals, 448 largest, NaN at S.1111.111, no Inf), the same
    32-element blocks and E8M0 scale, block exponent floor(log2 amax) - 8,
    elements rounded to nearest even and saturated at 448. Only RNE: the
    pages compare stochastic rounding within MXFP4, not within FP8.

What pins each function (tests/test_oracle_*.py, all "not gpu"):
  e2m1_value            OCP E2M1 table (tests/golden/e2m1_table.txt) and the
                        1-2-1 bit split; fixed-point re-quantization.
  sylvester_hadamard    scipy.linalg.hadamard(32); H H^T = 32 I.
  fwht32_f32            exact integer H x for dyadic inputs (explicit matrix
                        product); Parseval; one-hot and constant blocks.
  fwht16x2_f32          scipy.linalg.hadamard(16); exact integer
                        block-diag(H16, H16) x / 4 on dyadic inputs; R R x = x;
                        Parseval; the exact one-hot block.
  philox4x32_10         published Random123 known answers
                        (tests/golden/philox4x32_10_kat.txt) and rocRAND's
                        host engine compiled at test time.
  e8m0_exponent         brute force over all 256 scale codes.
  round_e2m1_rne        brute force argmin over all 16 codes, ties to even,
                        on every bf16 value and all threshold neighbours.
  round_e2m1_sr         unbiasedness over 10^4 seeds; limits f -> 0 and 1.
  quantize_ref          worked one-hot / constant / zero / NaN blocks;
                        re-quantizing a representable block is a fixed point.
  tile_codes/scales     element-by-element address formula written out in a
                        test loop; round trip through untile_*.
  operand_mse           exhaustive search for the nearest E2M1 value of every
                        element under its block scale (the error RNE must
                        reach); zero on representable blocks; the one-hot
                        block's exact error (0.1875 - c)^2.
  dequantize_ref,
  mx_gemm_ref           explicit triple loop and exact fractions.Fraction sums;
                        the rotation cancels in the product.
  e4m3_value            torch.float8_e4m3fn decode of all 256 codes.
  round_e4m3_rne        torch's fp32 -> float8_e4m3fn conversion on every
                        midpoint and its neighbours; brute-force nearest
                        search; saturation at 448.
  quantize_ref (fp8)    worked one-hot (H32) / constant / zero / NaN blocks;
                        fixed-point re-quantization; exact-fraction GEMM;
                        tile_codes_fp8 address loop and round trip.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "MX_BLOCK",
    "E2M1_EMAX",
    "HADAMARD_C_F32",
    "e2m1_value",
    "e2m1_magnitudes",
    "sylvester_hadamard",
    "fwht32_f32",
    "philox4x32_10",
    "rand_sign_bits",
    "sr_uniform24",
    "e8m0_exponent",
    "round_e2m1_rne",
    "round_e2m1_sr",
    "QuantRef",
    "quantize_ref",
    "dequantize_ref",
    "pack_codes",
    "unpack_codes",
    "TILE_ROWS",
    "TILE_K",
    "PANEL_ROWS",
    "padded_extents",
    "tile_codes",
    "tile_scales",
    "untile_codes",
    "untile_scales",
    "mx_gemm_ref",
    "operand_mse",
    "linear_ref",
    "bf16_round_ref",
    "fwht16x2_f32",
    "ROT_HADAMARD16",
    "FMT_FP4",
    "FMT_FP8",
    "e4m3_value",
    "e4m3_magnitudes",
    "round_e4m3_rne",
    "tile_codes_fp8",
    "untile_codes_fp8",
]

MX_BLOCK = 32          # elements per shared exponent ([36Kr] "Was ist MXFP4?")
E2M1_EMAX = 2          # largest unbiased exponent of E2M1 (OCP reading)
HADAMARD_C_F32 = np.float32(1.0 / np.sqrt(np.float64(32)))  # fp32(1/sqrt 32)

ROT_NONE, ROT_HADAMARD, ROT_RAND_SIGN = "none", "hadamard", "rand_sign_hadamard"
ROT_HADAMARD16 = "hadamard16"
H16_HALF = 16                 # points per transform of the 16-point variant
H16_C_F32 = np.float32(0.25)  # 1/sqrt(16), exact in fp32
ROUND_RNE, ROUND_SR = "rne", "sr"
FMT_FP4, FMT_FP8 = "fp4_e2m1", "fp8_e4m3"   # element formats (MXFP4; MXFP8 comparator)
E4M3_EMAX = 8          # largest unbiased exponent of E4M3 (OCP reading)
E4M3_MAX_CODE = 0x7E   # 448 = 1.75 * 2^8; 0x7F is NaN

_M32 = np.uint64(0xFFFFFFFF)


# ---------------------------------------------------------------------------
# Element format: E2M1 ([ShowAPI] section 2.2 bit split; OCP bias 1)
# ---------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: sign | 2-bit exponent | 1-bit mantissa."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:                       # subnormal: 0.m * 2^(1 - bias), bias 1
        mag = man * 0.5
    else:                              # normal: 1.m * 2^(exp - bias)
        mag = (1.0 + 0.5 * man) * 2.0 ** (exp - 1)
    return sign * mag


def e2m1_magnitudes() -> np.ndarray:
    """The 8 non-negative E2M1 values, indexed by the 3-bit magnitude code."""
    return np.array([e2m1_value(c) for c in range(8)], dtype=np.float64)


# ---------------------------------------------------------------------------
# Comparator element format: E4M3 (OCP MXFP8). The pages compare FP4 with
# FP8 training ([36Kr] intro: FP4 theoretically twice the compute of FP8;
# "Ende-zu-Ende-Effizienz": the step-throughput gain over FP8).
# ---------------------------------------------------------------------------
def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 code: sign | 4-bit exponent (bias 7) | 3-bit
    mantissa; exponent 0 is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN."""
    if (code & 0x7F) == 0x7F:
        return float("nan")
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 15
    man = code & 7
    if exp == 0:
        mag = man / 8.0 * 2.0 ** -6
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return sign * mag


def e4m3_magnitudes() -> np.ndarray:
    """The 127 finite non-negative E4M3 values, indexed by the 7-bit code."""
    return np.array([e4m3_value(c) for c in range(E4M3_MAX_CODE + 1)], dtype=np.float64)


def round_e4m3_rne(a: np.ndarray) -> np.ndarray:
    """Magnitude code (0..126) of the E4M3 value nearest to a >= 0, ties to
    the even code (even mantissa bit). Values above 448 go to 448 (the
    saturating conversion of OCP MX)."""
    g = e4m3_magnitudes()
    a64 = np.minimum(np.asarray(a, dtype=np.float32).astype(np.float64), 512.0)
    flat = a64.reshape(-1)
    idx = np.clip(np.searchsorted(g, flat, side="right") - 1, 0, E4M3_MAX_CODE)
    hi = np.minimum(idx + 1, E4M3_MAX_CODE)
    d_lo = np.abs(flat - g[idx])
    d_hi = np.abs(g[hi] - flat)
    code = np.where(d_hi < d_lo, hi, idx)
    tie = (d_hi == d_lo) & (hi != idx)
    code = np.where(tie, np.where(idx % 2 == 0, idx, hi), code)
    return code.reshape(a64.shape).astype(np.uint8)


# ---------------------------------------------------------------------------
# Rotation ([36Kr] "Fehlerdiagnoseexperiment": Hadamard before quantization)
# ---------------------------------------------------------------------------
def sylvester_hadamard(n: int = MX_BLOCK) -> np.ndarray:
    """Integer Sylvester Hadamard matrix, H_ij = (-1)^popcount(i & j)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def fwht32_f32(x: np.ndarray) -> np.ndarray:
    """y = fp32(fp32 butterfly(x) * c) along the last axis (length 32 blocks).

    Butterfly stages with stride h = 1, 2, 4, 8, 16; for every pair (i, i+h)
    with (i & h) == 0 the lower index gets fl32(a + b), the upper fl32(a - b).
    Then one fp32 multiply by c = fp32(1/sqrt(32)). No fused multiply-add.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    lead = y.shape[:-1]
    assert y.shape[-1] == MX_BLOCK
    h = 1
    while h < MX_BLOCK:
        y = y.reshape(lead + (MX_BLOCK // (2 * h), 2, h))
        a = y[..., 0, :]
        b = y[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2)   # float32 + float32 -> float32
        h *= 2
    y = y.reshape(lead + (MX_BLOCK,))
    return (y * HADAMARD_C_F32).astype(np.float32)


def fwht16x2_f32(x: np.ndarray) -> np.ndarray:
    """The 16-point variant: block-diag(H16, H16) / 4 inside each 32-block.

    [36Kr] "Ende-zu-Ende-Effizienz" labels the stabilised run "H16". Each half
    of a 32-element MX block (elements 0..15 and 16..31) is transformed on its
    own: butterfly stages with stride h = 1, 2, 4, 8 (lower index fl32(a + b),
    upper fl32(a - b)), then one multiply by 1/sqrt(16) = 0.25, which is exact.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    lead = y.shape[:-1]
    assert y.shape[-1] == MX_BLOCK
    h = 1
    while h < H16_HALF:
        y = y.reshape(lead + (MX_BLOCK // (2 * h), 2, h))
        a = y[..., 0, :]
        b = y[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2)   # float32 + float32 -> float32
        h *= 2
    y = y.reshape(lead + (MX_BLOCK,))
    return (y * H16_C_F32).astype(np.float32)


# ---------------------------------------------------------------------------
# Counter-based RNG: Philox4x32-10 (Salmon et al., SC'11)
# ---------------------------------------------------------------------------
_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = np.uint64(0x9E3779B9)
_PHILOX_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(ctr: Sequence, key: Sequence) -> Tuple[np.ndarray, ...]:
    """Philox4x32 with 10 rounds. ctr: 4 arrays/ints, key: 2 arrays/ints (32-bit).

    Round: (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2 (64-bit products);
    c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0). Between rounds the key is
    bumped by the Weyl constants (W0, W1) modulo 2^32.
    """
    c0, c1, c2, c3 = (np.asarray(v, dtype=np.uint64) & _M32 for v in ctr)
    k0, k1 = (np.asarray(v, dtype=np.uint64) & _M32 for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _PHILOX_W0) & _M32
            k1 = (k1 + _PHILOX_W1) & _M32
        p0 = _PHILOX_M0 * c0
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _M32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _M32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(v.astype(np.uint32) for v in (c0, c1, c2, c3))


def _philox_word(ctr, key, word):
    out = philox4x32_10(ctr, key)
    word = np.asarray(word)
    res = np.zeros(np.broadcast(*out, word).shape, dtype=np.uint32)
    for w in range(4):
        res = np.where(word == w, out[w], res)
    return res


def rand_sign_bits(k: np.ndarray, seed: int) -> np.ndarray:
    """Sign bit (0/1) of the random +-1 for reduction index k.

    key = (seed_lo, 0), counter = (k >> 2, 0, 1, 0), word k & 3, bit 31.
    Only the low 32 bits of the seed enter, so both GEMM operands (which pass
    the same user seed) draw the same signs and the rotation cancels in A B^T.
    """
    k = np.asarray(k, dtype=np.uint64)
    seed_lo = np.uint64(seed & 0xFFFFFFFF)
    w = _philox_word((k >> np.uint64(2), 0, 1, 0), (seed_lo, 0), k & np.uint64(3))
    return (w >> np.uint32(31)).astype(np.uint8)


def sr_uniform24(L: np.ndarray, seed: int) -> np.ndarray:
    """24-bit uniform for the element with row-major source index L.

    key = (seed_lo, seed_hi), counter = (low 32 bits of L >> 2, L >> 34, 0, 0),
    word L & 3, top 24 bits.
    """
    L = np.asarray(L, dtype=np.uint64)
    key = (np.uint64(seed & 0xFFFFFFFF), np.uint64((seed >> 32) & 0xFFFFFFFF))
    ctr = ((L >> np.uint64(2)) & _M32, L >> np.uint64(34), 0, 0)
    w = _philox_word(ctr, key, L & np.uint64(3))
    return (w >> np.uint32(8)).astype(np.uint32)


# ---------------------------------------------------------------------------
# Shared scale: E8M0 from the block maximum ([36Kr] "Was ist MXFP4?")
# ---------------------------------------------------------------------------
def e8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """Unbiased block exponent e = clamp(floor(log2 amax) - 2, -127, 127).

    amax == 0 gives e = -127. floor(log2) is read exactly from frexp of the
    fp64 value (every fp32, subnormals included, is a normal fp64).
    """
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(a)                  # a = m * 2^ex, m in [0.5, 1)
    e = (ex.astype(np.int64) - 1) - E2M1_EMAX
    e = np.clip(e, -127, 127)
    e = np.where(a == 0.0, -127, e)
    return e.astype(np.int64)


# ---------------------------------------------------------------------------
# Element rounding
# ---------------------------------------------------------------------------
def round_e2m1_rne(a: np.ndarray) -> np.ndarray:
    """Magnitude code (0..7) of the E2M1 value nearest to a >= 0, ties to even.

    Values above 6 go to 6 (the nearest representable magnitude).
    """
    g = e2m1_magnitudes()
    # Clamping at 8 keeps the distances below exact in fp64; every a >= 6
    # (8 included) is nearest to 6.
    a64 = np.minimum(np.asarray(a, dtype=np.float32).astype(np.float64), 8.0)
    dist = np.abs(a64[..., None] - g)                     # exact in fp64
    lo = np.argmin(dist, axis=-1)                         # first (lower) minimum
    lo_c = np.minimum(lo + 1, 7)
    d_lo = np.take_along_axis(dist, lo[..., None], -1)[..., 0]
    d_hi = np.take_along_axis(dist, lo_c[..., None], -1)[..., 0]
    tie = (lo < 7) & (d_hi == d_lo)
    code = np.where(tie & (lo % 2 == 1), lo + 1, lo)      # even code wins a tie
    return code.astype(np.uint8)


def round_e2m1_sr(a: np.ndarray, u24: np.ndarray) -> np.ndarray:
    """Stochastic magnitude code for a >= 0 with a 24-bit uniform u24.

    With lo <= a < hi the neighbouring magnitudes, the upper one is taken when
    u24 < f * 2^24, f = (a - lo) / (hi - lo). a >= 6 gives 6 (not randomised).
    """
    g = e2m1_magnitudes()
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    idx = np.searchsorted(g, a64, side="right") - 1       # lo = g[idx] <= a
    idx = np.clip(idx, 0, 7)
    sat = idx >= 7
    idx_c = np.minimum(idx, 6)
    lo = g[idx_c]
    hi = g[idx_c + 1]
    f = (a64 - lo) / (hi - lo)                            # exact (gap is 2^k)
    up = np.asarray(u24, dtype=np.float64) < f * float(1 << 24)
    code = np.where(sat, 7, idx_c + up.astype(np.int64))
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# The quantizer
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class QuantRef:
    """A quantized operand in reduction-major orientation.

    codes  uint8 [MN, K]: one 4-bit code per element (sign << 3 | magnitude).
    scales uint8 [MN, K/32]: E8M0 codes (0xFF = NaN block).
    rotated float32 [MN, K]: the values that were quantized (after rotation).
    For axis = 1 the source [R, C] maps to MN = R, K = C; for axis = 0 the
    source is read transposed: MN = C, K = R.
    """
    codes: np.ndarray
    scales: np.ndarray
    rotated: np.ndarray
    axis: int
    fmt: str = FMT_FP4


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_ref(x_bits: np.ndarray, axis: int, block: int = MX_BLOCK,
                 rotate: str = ROT_HADAMARD, rounding: str = ROUND_RNE,
                 seed: int = 0, *, row_index: Optional[np.ndarray] = None,
                 col_index: Optional[np.ndarray] = None,
                 total_cols: Optional[int] = None, fmt: str = FMT_FP4) -> QuantRef:
    """Rotate, scale and round a bfloat16 tensor [R, C] in blocks along `axis`.

    row_index / col_index give the global row / column of each supplied row /
    column when x_bits is a slice of a larger tensor with total_cols columns
    (they set the random-sign index k and the stochastic-rounding index L).
    Along `axis` the slice must start at a multiple of 32 and be contiguous.
    """
    if block != MX_BLOCK:
        raise ValueError("only 32-element blocks are defined")
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    rows = np.arange(R, dtype=np.int64) if row_index is None else np.asarray(row_index, np.int64)
    cols = np.arange(C, dtype=np.int64) if col_index is None else np.asarray(col_index, np.int64)
    ncols = C if total_cols is None else int(total_cols)

    # 1. widen bf16 -> fp32 (exact) and orient reduction-major: [MN, K]
    x = _bf16_to_f32(x_bits)
    if axis == 1:
        xk = x
        k_index = cols
        L = rows[:, None] * ncols + cols[None, :]
    elif axis == 0:
        xk = x.T
        k_index = rows
        L = rows[None, :] * ncols + cols[:, None]
    else:
        raise ValueError("axis must be 0 or 1")
    MN, K = xk.shape
    if K % block:
        raise ValueError("reduction extent must be a multiple of 32")
    xk = np.array(xk, dtype=np.float32, copy=True)

    # 2. random signs (before the transform), shared by both operands
    if rotate == ROT_RAND_SIGN:
        s = rand_sign_bits(k_index, seed).astype(np.uint32) << np.uint32(31)
        xk = (xk.view(np.uint32) ^ s[None, :]).view(np.float32)
    elif rotate not in (ROT_NONE, ROT_HADAMARD, ROT_HADAMARD16):
        raise ValueError(rotate)

    # 3. 32-point Hadamard (or the 16-point variant) on every block of the
    #    reduction axis
    blocks = xk.reshape(MN, K // block, block)
    if rotate == ROT_HADAMARD16:
        blocks = fwht16x2_f32(blocks)
    elif rotate != ROT_NONE:
        blocks = fwht32_f32(blocks)
    y = blocks

    # 4. block amax -> 5. E8M0 scale (the element format's largest exponent
    #    is taken off: 2 for E2M1, 8 for the E4M3 comparator)
    absy = np.abs(y.astype(np.float64))
    bad = ~np.isfinite(absy).all(axis=-1)
    amax = np.where(bad, 0.0, np.max(np.where(np.isfinite(absy), absy, 0.0), axis=-1))
    e = e8m0_exponent(amax)
    if fmt == FMT_FP8:
        e = np.clip(e + E2M1_EMAX - E4M3_EMAX, -127, 127)
        e = np.where(amax == 0.0, -127, e)
    elif fmt != FMT_FP4:
        raise ValueError(fmt)
    scales = (e + 127).astype(np.uint8)
    scales = np.where(bad, np.uint8(0xFF), scales)

    # 6. scale each element: t = fl32(y * 2^-e)
    pow2 = np.ldexp(np.float32(1.0), (-e).astype(np.int32)).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        t = (y * pow2[..., None]).astype(np.float32)
    a = np.abs(t)

    # 7./8. magnitude code
    if fmt == FMT_FP8:
        if rounding != ROUND_RNE:
            raise ValueError("the E4M3 comparator rounds to nearest even only")
        mag = round_e4m3_rne(np.where(np.isfinite(a), a, 0.0))
        sign = np.signbit(y).astype(np.uint8)
        codes = (sign << 7) | mag
        codes = np.where(bad[..., None], np.uint8(0), codes).astype(np.uint8)
        return QuantRef(codes.reshape(MN, K), scales.astype(np.uint8),
                        y.reshape(MN, K).astype(np.float32), axis, FMT_FP8)
    if rounding == ROUND_RNE:
        mag = round_e2m1_rne(np.where(np.isfinite(a), a, 0.0))
    elif rounding == ROUND_SR:
        u = sr_uniform24(L, seed).reshape(MN, K // block, block)
        mag = round_e2m1_sr(np.where(np.isfinite(a), a, 0.0), u)
    else:
        raise ValueError(rounding)

    # 9. sign bit of y
    sign = np.signbit(y).astype(np.uint8)
    codes = (sign << 3) | mag
    codes = np.where(bad[..., None], np.uint8(0), codes).astype(np.uint8)
    return QuantRef(codes.reshape(MN, K), scales.astype(np.uint8),
                    y.reshape(MN, K).astype(np.float32), axis)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along K: even index in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


TILE_ROWS = 16      # reduction-major rows per tile
TILE_K = 128        # reduction elements per tile (four 32-element blocks)
PANEL_ROWS = 256    # MN is padded to whole panels of 256 rows


def padded_extents(mn: int, k: int) -> Tuple[int, int]:
    """Extents of the tiled layout: MN up to a multiple of 256, K of 128."""
    return -(-mn // PANEL_ROWS) * PANEL_ROWS, -(-k // TILE_K) * TILE_K


def tile_codes(codes: np.ndarray) -> np.ndarray:
    """Packed codes [MN, K] (one 4-bit code per element) -> tiled byte buffer.

    The operand is zero-padded to [MNp, Kp] (padded_extents; the codes of a
    zero element are 0) and stored tile by tile: tile (g, q) holds rows
    16g..16g+15 and K elements 128q..128q+127 at byte offset
    (g * Kp/128 + q) * 1024; inside a tile, 32-element block c of row r is the
    16 bytes at c * 256 + r * 16 (two codes per byte, even K index low).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    mn, k = codes.shape
    mnp, kp = padded_extents(mn, k)
    full = np.zeros((mnp, kp), np.uint8)
    full[:mn, :k] = codes
    packed = pack_codes(full)                                   # [MNp, Kp/2]
    t = packed.reshape(mnp // TILE_ROWS, TILE_ROWS, kp // TILE_K, 4, 16)   # g r q c byte
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1, 4)).reshape(-1)    # g q c r byte


def tile_scales(scales: np.ndarray, k: int) -> np.ndarray:
    """Scales [MN, K/32] -> tiled buffer [Kp/128][MNp/256][4][4][16][4]
    (padding scale code 0, the code of an all-zero block).

    The scale of row m = 256 T + 16 h + r (panel T, row group h inside it, row
    r) and block kb = 4 q + c is the byte at
    (q * MNp/256 + T) * 1024 + (h // 4) * 256 + c * 64 + r * 4 + h % 4: one
    1 KB block per K slice and 256-row panel; its 256-byte quarter h // 4
    holds, for every (r, c), the scales of four consecutive row groups as 4
    consecutive bytes at (16 c + r) * 4.
    """
    scales = np.asarray(scales, dtype=np.uint8)
    mn = scales.shape[0]
    mnp, kp = padded_extents(mn, k)
    full = np.zeros((mnp, kp // 32), np.uint8)
    full[:mn, :scales.shape[1]] = scales
    t = full.reshape(mnp // PANEL_ROWS, 4, 4, TILE_ROWS, kp // TILE_K, 4)  # T hq hl r q c
    return np.ascontiguousarray(t.transpose(4, 0, 1, 5, 3, 2)).reshape(-1)  # q T hq c r hl


def tile_codes_fp8(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes [MN, K] (one byte per element) -> tiled byte buffer.

    Zero-padded to [MNp, Kp] like the FP4 layout; tile (g, q) -- rows
    16g..16g+15, K elements 128q..128q+127 -- is the 2 KB at byte
    (g * Kp/128 + q) * 2048. Inside it, the 16-element chunk j (K elements
    16j..16j+15 of the slice) of row r is the 16 bytes at j * 256 + r * 16,
    element k of the slice at (k // 16) * 256 + r * 16 + k % 16.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    mn, k = codes.shape
    mnp, kp = padded_extents(mn, k)
    full = np.zeros((mnp, kp), np.uint8)
    full[:mn, :k] = codes
    t = full.reshape(mnp // TILE_ROWS, TILE_ROWS, kp // TILE_K, 8, 16)     # g r q j byte
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1, 4)).reshape(-1)   # g q j r byte


def untile_codes_fp8(buf: np.ndarray, mn: int, k: int) -> np.ndarray:
    """Inverse of tile_codes_fp8."""
    mnp, kp = padded_extents(mn, k)
    t = np.asarray(buf, np.uint8)[: mnp * kp].reshape(mnp // TILE_ROWS, kp // TILE_K, 8,
                                                      TILE_ROWS, 16)
    return t.transpose(0, 3, 1, 2, 4).reshape(mnp, kp)[:mn, :k]


def untile_codes(buf: np.ndarray, mn: int, k: int) -> np.ndarray:
    """Inverse of tile_codes: tiled bytes -> codes [MN, K]."""
    mnp, kp = padded_extents(mn, k)
    t = np.asarray(buf, np.uint8)[: mnp * kp // 2].reshape(mnp // TILE_ROWS, kp // TILE_K, 4,
                                                           TILE_ROWS, 16)
    packed = t.transpose(0, 3, 1, 2, 4).reshape(mnp, kp // 2)
    return unpack_codes(packed)[:mn, :k]


def untile_scales(buf: np.ndarray, mn: int, k: int) -> np.ndarray:
    """Inverse of tile_scales: tiled bytes -> scales [MN, K/32]."""
    mnp, kp = padded_extents(mn, k)
    t = np.asarray(buf, np.uint8)[: mnp * kp // 32].reshape(
        kp // TILE_K, mnp // PANEL_ROWS, 4, 4, TILE_ROWS, 4)                   # q T hq c r hl
    return t.transpose(1, 2, 5, 4, 0, 3).reshape(mnp, kp // 32)[:mn, : k // 32]


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def dequantize_ref(codes: np.ndarray, scales: np.ndarray, fmt: str = FMT_FP4) -> np.ndarray:
    """fp64 values (-1)^s * E2M1(mag) * 2^(scale - 127) (E4M3 for fmt =
    fp8_e4m3); scale 0xFF is NaN."""
    codes = np.asarray(codes, dtype=np.uint8)
    MN, K = codes.shape
    if fmt == FMT_FP8:
        table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    else:
        table = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
    vals = table[codes].reshape(MN, K // MX_BLOCK, MX_BLOCK)
    s = np.asarray(scales, dtype=np.int64)
    factor = np.where(s == 0xFF, np.nan, np.ldexp(1.0, s - 127))
    return (vals * factor[..., None]).reshape(MN, K)


def mx_gemm_ref(qa: QuantRef, qb: QuantRef) -> np.ndarray:
    """C[m, n] = sum_k deqA[m, k] * deqB[n, k], fp64."""
    da = dequantize_ref(qa.codes, qa.scales, qa.fmt)
    db = dequantize_ref(qb.codes, qb.scales, qb.fmt)
    return da @ db.T


def operand_mse(q: QuantRef) -> float:
    """Operand-level quantization error: mean over the operand of
    (deq - y)^2 in fp64, y the rotated values that were quantized and deq
    their dequantized codes ([36Kr] "Fehlerdiagnoseexperiment": the
    quantization error of the Wgrad operands with and without the rotation).
    R is orthonormal, so this is also the error in the source's own domain,
    up to the fp32 rounding of y."""
    d = dequantize_ref(q.codes, q.scales, q.fmt) - np.asarray(q.rotated, np.float64)
    return float(np.mean(d * d))


def linear_ref(op: str, a_src: np.ndarray, b_src: np.ndarray, rotate: str = ROT_HADAMARD,
               rounding: str = ROUND_RNE, seed: int = 0, fmt: str = FMT_FP4):
    """One GEMM of the triple ([36Kr] "Fehlerdiagnoseexperiment").

    fprop: a_src = X [T, in], b_src = W [out, in] -> Y [T, out] = X W^T
    dgrad: a_src = dY [T, out], b_src = W [out, in] -> dX [T, in] = dY W
    wgrad: a_src = dY [T, out], b_src = X [T, in] -> dW [out, in] = dY^T X
    The A operand uses stochastic-rounding role 0 (seed), B role 1
    (seed | 1 << 32); random signs depend only on the low 32 bits.
    Returns (C fp64, QuantRef A, QuantRef B).
    """
    axes = {"fprop": (1, 1), "dgrad": (1, 0), "wgrad": (0, 0)}[op]
    seed_a = seed & 0xFFFFFFFF
    seed_b = seed_a | (1 << 32)
    qa = quantize_ref(a_src, axes[0], rotate=rotate, rounding=rounding, seed=seed_a, fmt=fmt)
    qb = quantize_ref(b_src, axes[1], rotate=rotate, rounding=rounding, seed=seed_b, fmt=fmt)
    return mx_gemm_ref(qa, qb), qa, qb


def bf16_round_ref(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of fp32 values, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    out = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    out = out.astype(np.uint16)
    nan = np.isnan(x)
    out[nan] = np.uint16(0x7FC0)
    return out
