"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Every check here compares the oracle with something it does not compute the
same way: a published table or known-answer vector, a library routine
(scipy, torch, rocRAND), a closed form, a brute-force search or an invariant.
All tests run on the CPU.
"""
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
from datagen import f32_to_bf16_bits, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------- E2M1 table
def test_e2m1_table_matches_ocp():
    rows = _golden_rows("e2m1_table.txt")
    assert len(rows) == 16
    for code_s, sign, expf, man, val in rows:
        code = int(code_s, 16)
        v = oracle.e2m1_value(code)
        assert v == float(val), (code, v, val)
        assert np.signbit(v) == bool(int(sign))
        assert (code >> 1) & 3 == int(expf) and code & 1 == int(man)


# ------------------------------------------------------------ Hadamard matrix
def test_sylvester_matches_scipy_and_is_orthogonal():
    scipy_linalg = pytest.importorskip("scipy.linalg")
    H = oracle.sylvester_hadamard(32)
    assert np.array_equal(H, scipy_linalg.hadamard(32).astype(np.int64))
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=np.int64))


def test_hadamard_constant_is_correctly_rounded():
    c = oracle.HADAMARD_C_F32
    assert int(np.float32(c).view(np.uint32)) == 0x3E3504F3
    # c is the fp32 nearest to 1/sqrt(32): compare squared distances exactly.
    target_sq = Fraction(1, 32)
    bits = int(np.float32(c).view(np.uint32))
    cand = [Fraction(float(np.uint32(b).view(np.float32))) for b in (bits - 1, bits, bits + 1)]
    # |x - 1/sqrt32| ordering equals |x^2 - 1/32| ordering near the root only
    # up to a factor; check the exact root lies between the midpoints.
    lo_mid = (cand[0] + cand[1]) / 2
    hi_mid = (cand[1] + cand[2]) / 2
    assert lo_mid * lo_mid < target_sq < hi_mid * hi_mid


def test_fwht_exact_on_dyadic_inputs():
    """Small-integer blocks: every butterfly add is exact, so the fp32
    transform must equal fl32(fl32(H x) * c) with H x an exact integer product."""
    rng = np.random.default_rng(1)
    H = oracle.sylvester_hadamard(32)
    x = rng.integers(-1000, 1000, size=(500, 32)).astype(np.int64)
    x[0] = 0
    x[1] = 0
    x[1, 5] = 1
    exact = (x @ H.T)  # y_i = sum_j H_ij x_j (H symmetric)
    want = (exact.astype(np.float32) * oracle.HADAMARD_C_F32).astype(np.float32)
    got = oracle.fwht32_f32(x.astype(np.float32))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # power-of-two scaled dyadic inputs stay exact too
    sc = np.float32(2.0 ** -20)
    got2 = oracle.fwht32_f32(x.astype(np.float32) * sc)
    want2 = ((exact.astype(np.float32) * sc) * oracle.HADAMARD_C_F32).astype(np.float32)
    assert np.array_equal(got2.view(np.uint32), want2.view(np.uint32))


def test_fwht_parseval_and_involution():
    rng = np.random.default_rng(2)
    x = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((4000, 32)).astype(np.float32)))
    y = oracle.fwht32_f32(x)
    nx = np.sum(x.astype(np.float64) ** 2, axis=1)
    ny = np.sum(y.astype(np.float64) ** 2, axis=1)
    assert np.max(np.abs(ny - nx) / nx) < 2e-6
    # applying the orthonormal transform twice gives the input back (H^2 = 32 I)
    z = oracle.fwht32_f32(y)
    assert np.max(np.abs(z - x)) < 1e-5 * np.max(np.abs(x))


# --------------------------------------------------------------------- Philox
# ---------------------------------------------------- 16-point variant (H16)
def test_h16_matches_scipy():
    scipy_linalg = pytest.importorskip("scipy.linalg")
    H = oracle.sylvester_hadamard(16)
    assert np.array_equal(H, scipy_linalg.hadamard(16).astype(np.int64))
    assert np.array_equal(H @ H.T, 16 * np.eye(16, dtype=np.int64))


def test_fwht16x2_exact_on_dyadic_inputs():
    """Small-integer blocks: each half must equal (H16 x_half) / 4 exactly,
    the two halves independent (block-diag(H16, H16))."""
    rng = np.random.default_rng(21)
    H = oracle.sylvester_hadamard(16)
    x = rng.integers(-1000, 1000, size=(500, 32)).astype(np.int64)
    exact = np.concatenate([x[:, :16] @ H.T, x[:, 16:] @ H.T], axis=1)
    want = (exact.astype(np.float32) * np.float32(0.25)).astype(np.float32)
    got = oracle.fwht16x2_f32(x.astype(np.float32))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # block-diagonal: a one-hot in the first half leaves the second at zero
    e = np.zeros((1, 32), np.float32)
    e[0, 3] = 1.0
    y = oracle.fwht16x2_f32(e)[0]
    assert np.array_equal(y[:16], 0.25 * H[:, 3].astype(np.float32)) and not y[16:].any()


def test_fwht16x2_involution_and_parseval():
    """R = block-diag(H16, H16) / 4 is orthonormal and its own inverse: on
    dyadic inputs R R x = x exactly."""
    rng = np.random.default_rng(22)
    x = (rng.integers(-500, 500, size=(300, 32)) * 4).astype(np.float32)
    assert np.array_equal(oracle.fwht16x2_f32(oracle.fwht16x2_f32(x)), x)
    xb = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((2000, 32)).astype(np.float32)))
    y = oracle.fwht16x2_f32(xb)
    nx = np.sum(xb.astype(np.float64) ** 2, axis=1)
    ny = np.sum(y.astype(np.float64) ** 2, axis=1)
    assert np.max(np.abs(ny - nx) / nx) < 1e-6


def test_h16_one_hot_block_is_exact():
    """x = e_j: its half becomes +-0.25, the other half 0; amax 0.25 gives
    e = -4 (scale code 123), t = 0.25 * 16 = 4 -> magnitude code 6 on the 16
    entries of j's half, 0 elsewhere; the dequantized block equals y exactly."""
    H = oracle.sylvester_hadamard(16)
    for j in (0, 7, 16, 31):
        x = np.zeros((1, 32), np.float32)
        x[0, j] = 1.0
        q = oracle.quantize_ref(_bf16(x), axis=1, rotate="hadamard16")
        assert q.scales[0, 0] == 123
        half = slice(0, 16) if j < 16 else slice(16, 32)
        other = slice(16, 32) if j < 16 else slice(0, 16)
        want = np.where(H[:, j % 16] > 0, 6, 14)
        assert np.array_equal(q.codes[0, half], want)
        assert not q.codes[0, other].any()
        d = oracle.dequantize_ref(q.codes, q.scales)[0]
        assert np.array_equal(d, q.rotated[0].astype(np.float64))


def test_philox_published_known_answers():
    for row in _golden_rows("philox4x32_10_kat.txt"):
        v = [int(t, 16) for t in row]
        out = oracle.philox4x32_10(v[0:4], v[4:6])
        assert [int(o) for o in out] == v[6:10]


_ROCRAND_PROBE = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
int main() {
  const unsigned long long seeds[4] = {0ull, 7ull, 0x100000007ull, 0xfedcba9876543210ull};
  for (int s = 0; s < 4; ++s) {
    rocrand_device::philox4x32_10_engine e(seeds[s], 0, 0);
    for (int i = 0; i < 5; ++i) {
      uint4 v = e.next4();
      std::printf("%llu %d %u %u %u %u\n", seeds[s], i, v.x, v.y, v.z, v.w);
    }
  }
  return 0;
}
"""


def test_philox_matches_rocrand_host_engine():
    """rocRAND's philox4x32_10 engine seeded with s at subsequence 0 returns
    Philox(ctr = (i, 0, 0, 0), key = (s_lo, s_hi)) as its i-th 4-word block."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("hipcc / rocRAND headers not available")
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "p.hip")
        exe = os.path.join(td, "p")
        with open(src, "w") as fh:
            fh.write(_ROCRAND_PROBE)
        r = subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-I/opt/rocm/include",
                            src, "-o", exe], capture_output=True, text=True)
        if r.returncode != 0:
            pytest.skip("could not build the rocRAND host probe: " + r.stderr[-400:])
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    lines = out.strip().splitlines()
    assert len(lines) == 20
    for line in lines:
        s, i, *w = (int(t) for t in line.split())
        got = oracle.philox4x32_10((i, 0, 0, 0), (s & 0xFFFFFFFF, s >> 32))
        assert [int(g) for g in got] == w


def test_sr_uniform_is_uniform():
    u = oracle.sr_uniform24(np.arange(1 << 18, dtype=np.uint64), 12345)
    assert u.max() < (1 << 24)
    hist = np.bincount((u >> 16).astype(np.int64), minlength=256)
    exp = (1 << 18) / 256
    chi2 = float(np.sum((hist - exp) ** 2 / exp))
    assert chi2 < 330.0   # 255 dof; p ~ 1e-3 tail
    # role (seed_hi) changes the stream; the same seed reproduces it
    u2 = oracle.sr_uniform24(np.arange(1024, dtype=np.uint64), 12345 | (1 << 32))
    assert not np.array_equal(u[:1024], u2)
    assert np.array_equal(u[:1024], oracle.sr_uniform24(np.arange(1024, dtype=np.uint64), 12345))


def test_rand_signs_balanced_and_role_free():
    k = np.arange(1 << 16, dtype=np.uint64)
    s = oracle.rand_sign_bits(k, 11)
    assert abs(int(s.sum()) - (1 << 15)) < 5 * np.sqrt(1 << 14)
    assert np.array_equal(s, oracle.rand_sign_bits(k, 11 | (5 << 32)))
    assert not np.array_equal(s, oracle.rand_sign_bits(k, 12))


# ---------------------------------------------------------------- E8M0 scales
def test_e8m0_brute_force_over_all_scale_codes():
    rng = np.random.default_rng(3)
    bits = rng.integers(1, 0x7F800000, size=20000, dtype=np.uint32)
    specials = []
    for e in range(-149, 128):
        for m in (1.0, 1.5, 1.999999):
            v = np.float32(np.ldexp(m, e)) if e >= -126 else np.float32(np.ldexp(1.0, e))
            if np.isfinite(v) and v > 0:
                specials.append(v)
    amax = np.concatenate([bits.view(np.float32), np.array(specials, np.float32)])
    e = oracle.e8m0_exponent(amax)
    for a, ee in zip(amax.astype(np.float64), e):
        fr_a = Fraction(float(a))
        ok = [s for s in range(255)
              if Fraction(4) <= fr_a / (Fraction(2) ** (s - 127)) < Fraction(8)]
        if ok:
            assert len(ok) == 1 and ok[0] - 127 == ee, (a, ok, ee)
        else:   # below the E8M0 range: clamped to the smallest scale
            assert fr_a / (Fraction(2) ** -127) < 4 and ee == -127, (a, ee)
    assert oracle.e8m0_exponent(np.float32(0.0)) == -127


def test_e8m0_decode_matches_torch():
    torch = pytest.importorskip("torch")
    s = np.arange(256, dtype=np.uint8)
    codes = np.zeros((256, 32), np.uint8)
    codes[:, 0] = 2   # E2M1 1.0
    d = oracle.dequantize_ref(codes, s[:, None])[:, 0]
    t = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)
    assert np.array_equal(d[:255], t[:255])
    assert np.isnan(d[255]) and np.isnan(t[255])


# ------------------------------------------------------------ E2M1 rounding
def _brute_rne(a):
    """Nearest of all 16 codes' values by exact distance; ties to the even
    mantissa bit (code & 1 == 0); only non-negative codes can win for a >= 0."""
    vals = np.array([oracle.e2m1_value(c) for c in range(16)])
    out = []
    for x in a:
        d = [abs(Fraction(float(x)) - Fraction(v)) for v in vals]
        best = min(d)
        cands = [c for c in range(16) if d[c] == best and not (c & 8)]
        even = [c for c in cands if c & 1 == 0]
        out.append((even or cands)[0])
    return np.array(out, dtype=np.uint8)


def _threshold_rne(a):
    a = np.asarray(a, np.float64)
    return ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0)).astype(np.uint8)


def test_rne_against_brute_force():
    pts = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0, 8.0]
    a = []
    for p in pts:
        b = int(np.float32(p).view(np.uint32))
        for d in range(-3, 4):
            if b + d >= 0:
                a.append(np.uint32(b + d).view(np.float32))
    rng = np.random.default_rng(4)
    a += list(rng.uniform(0, 9, 3000).astype(np.float32))
    a += list(np.float32(np.ldexp(1.0, -140)) * np.arange(1, 5, dtype=np.float32))
    a = np.array(a, np.float32)
    got = oracle.round_e2m1_rne(a)
    assert np.array_equal(got, _brute_rne(a))
    assert np.array_equal(got, _threshold_rne(a))


def test_rne_exhaustive_bf16_and_threshold_table():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)   # every non-negative finite bf16
    a = bf16_bits_to_f32(bits)
    assert np.array_equal(oracle.round_e2m1_rne(a), _threshold_rne(a))
    # every fp32 pattern within +-2048 ulps of each rounding threshold
    for th in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0):
        b = int(np.float32(th).view(np.uint32))
        near = np.arange(b - 2048, b + 2049, dtype=np.uint32).view(np.float32)
        assert np.array_equal(oracle.round_e2m1_rne(near), _threshold_rne(near))


def test_sr_limits():
    a = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 7.5], np.float32)
    g = [0, 1, 2, 3, 4, 5, 6, 7, 7]
    for u in (0, 1, (1 << 24) - 1):
        assert list(oracle.round_e2m1_sr(a, np.full(a.shape, u))) == g
    # a = 1 - 2^-24: lo = 0.5, gap 0.5, f = 1 - 2^-23, so f * 2^24 = 2^24 - 2
    just_below = np.nextafter(np.float32(1.0), np.float32(0.0))
    assert oracle.round_e2m1_sr(np.array([just_below]), np.array([(1 << 24) - 3]))[0] == 2
    assert oracle.round_e2m1_sr(np.array([just_below]), np.array([(1 << 24) - 2]))[0] == 1


def test_sr_unbiased_over_1e4_seeds():
    """Expected dequantized value over seeds equals the input: for each of 32
    non-saturated values, the mean over seeds 0..9999 lies within 3 sigma of
    it, sigma = gap * sqrt(f (1 - f) / 10^4) the standard error of the mean
    of a two-point draw; and the mean z-score over the 32 values lies within
    3 / sqrt(32) (the pooled test, 3 sigma for the mean of 32 unit-variance
    z-scores). The seed list is fixed, so the test is deterministic; for an
    unbiased rounder with a fresh seed list each per-value bound would fail
    with probability 0.27%, the 32 together with about 8% (measured here:
    largest |z| 2.25, pooled 0.93 sigma)."""
    rng = np.random.default_rng(5)
    n = 32
    vals = rng.uniform(0.0, 5.9, n).astype(np.float32)
    seeds = np.arange(10000, dtype=np.uint64)
    L = np.arange(n, dtype=np.uint64)
    codes = np.empty((seeds.size, n), np.uint8)
    for i, s in enumerate(seeds):
        codes[i] = oracle.round_e2m1_sr(vals, oracle.sr_uniform24(L, int(s)))
    g = oracle.e2m1_magnitudes()
    deq = g[codes]
    mean = deq.mean(axis=0)
    idx = np.searchsorted(g, vals.astype(np.float64), side="right") - 1
    gap = g[idx + 1] - g[idx]
    f = (vals - g[idx]) / gap
    sigma = gap * np.sqrt(f * (1 - f) / seeds.size)
    z = (mean - vals) / np.where(sigma > 0, sigma, 1)
    assert np.all(np.abs(z) < 3.0)
    assert abs(z.mean()) < 3 / np.sqrt(n)


def test_operand_mse_is_the_nearest_value_error():
    """operand_mse against an exhaustive search: under each block's scale 2^e,
    the squared distance from y to the nearest of the 16 values
    E2M1(code) * 2^e (which round-to-nearest must reach, ties included),
    summed with exact fractions; on blocks of N(0,1), of 1e-4 t_3 and with a
    large outlier, with and without the rotation."""
    from fractions import Fraction
    rng = np.random.default_rng(12)
    g = [Fraction(oracle.e2m1_value(c)) for c in range(16)]
    srcs = [rng.standard_normal((3, 64)), 1e-4 * rng.standard_t(3, (3, 64)),
            np.r_[rng.standard_normal(63), 300.0].reshape(1, 64)]
    for x in srcs:
        bits = f32_to_bf16_bits(x.astype(np.float32))
        for rot in ("none", "hadamard"):
            q = oracle.quantize_ref(bits, 1, rotate=rot)
            tot = Fraction(0)
            for m in range(q.rotated.shape[0]):
                for k in range(q.rotated.shape[1]):
                    sc = Fraction(2) ** (int(q.scales[m, k // 32]) - 127)
                    y = Fraction(float(q.rotated[m, k]))
                    tot += min((v * sc - y) ** 2 for v in g)
            want = tot / q.rotated.size
            got = oracle.operand_mse(q)
            assert abs(Fraction(got) - want) <= want * Fraction(1, 10 ** 12), rot


def test_operand_mse_zero_and_one_hot():
    """A block of representable values (no rotation) has zero error; the
    one-hot block under H32 has y = +-c everywhere and dequantizes to
    +-0.1875, so its error is exactly (0.1875 - c)^2 per element."""
    from fractions import Fraction
    x = f32_to_bf16_bits(np.array([[0.5, -1.5, 6.0, 0.0, 3.0, -4.0, 2.0, 1.0] * 4], np.float32))
    assert oracle.operand_mse(oracle.quantize_ref(x, 1, rotate="none")) == 0.0
    one = np.zeros((1, 32), np.float32)
    one[0, 9] = 1.0
    q = oracle.quantize_ref(f32_to_bf16_bits(one), 1, rotate="hadamard")
    c = Fraction(float(oracle.HADAMARD_C_F32))
    assert Fraction(oracle.operand_mse(q)) == (Fraction(3, 16) - c) ** 2


# ------------------------------------------------------ quantizer worked cases
def _bf16(vals):
    return f32_to_bf16_bits(np.asarray(vals, np.float32))


def test_one_hot_block():
    """x = e_j: y = c * H[:, j] = +-0.1767767; floor(log2 c) = -3 -> e = -5
    (scale code 122); t = c * 32 = 5.656854 -> magnitude 6 (code 7) everywhere."""
    H = oracle.sylvester_hadamard(32)
    for j in (0, 5, 31):
        x = np.zeros((1, 32), np.float32)
        x[0, j] = 1.0
        q = oracle.quantize_ref(_bf16(x), axis=1, rotate="hadamard")
        assert q.scales[0, 0] == 122
        want = np.where(H[:, j] > 0, 7, 15)
        assert np.array_equal(q.codes[0], want)
        d = oracle.dequantize_ref(q.codes, q.scales)[0]
        assert np.allclose(np.abs(d), 0.1875)
    # under SR the upper neighbour 6 is taken with probability (5.656854-4)/2
    x = np.zeros((4096, 32), np.float32)
    x[:, 0] = 1.0
    q = oracle.quantize_ref(_bf16(x), axis=1, rotate="hadamard", rounding="sr", seed=9)
    p6 = np.mean((q.codes & 7) == 7)
    t = float(np.float32(oracle.HADAMARD_C_F32) * np.float32(32.0))
    assert abs(p6 - (t - 4) / 2) < 4 * np.sqrt(0.83 * 0.17 / q.codes.size)


def test_constant_block():
    """x = 1 (32 times): y_0 = fl32(32 c) = 5.656854, the rest are +0;
    e = 0 (scale 127); code 7 at index 0 and 0 elsewhere."""
    q = oracle.quantize_ref(_bf16(np.ones((1, 32))), axis=1, rotate="hadamard")
    assert q.scales[0, 0] == 127
    assert q.codes[0, 0] == 7 and np.all(q.codes[0, 1:] == 0)


def test_zero_nan_and_signed_zero_blocks():
    x = np.zeros((3, 64), np.float32)
    x[1, :32] = -0.0
    x[2, 40] = np.nan
    q = oracle.quantize_ref(_bf16(x), axis=1, rotate="none")
    assert np.all(q.scales[0] == 0) and np.all(q.codes[0] == 0)
    assert np.all(q.codes[1, :32] == 8) and q.scales[1, 0] == 0
    assert q.scales[2, 1] == 0xFF and np.all(q.codes[2, 32:] == 0)
    assert q.scales[2, 0] == 0


def test_requantizing_representable_block_is_fixed_point():
    rng = np.random.default_rng(6)
    for trial in range(400):
        s = int(rng.integers(1, 250))           # keep 6 * 2^(s-127) inside bf16
        codes = rng.integers(0, 16, 32).astype(np.uint8)
        codes[rng.integers(0, 32)] = rng.choice([6, 7, 14, 15])   # block max 4 or 6
        d = oracle.dequantize_ref(codes[None], np.array([[s]], np.uint8))
        x = _bf16(d.astype(np.float32))
        assert np.array_equal(bf16_bits_to_f32(x).astype(np.float64), d)
        q = oracle.quantize_ref(x, axis=1, rotate="none")
        assert q.scales[0, 0] == s
        assert np.array_equal(q.codes[0], codes)


def test_axis0_is_transpose_of_axis1():
    rng = np.random.default_rng(7)
    x = f32_to_bf16_bits(rng.standard_normal((96, 64)).astype(np.float32))
    q0 = oracle.quantize_ref(x, axis=0, rotate="hadamard")
    q1 = oracle.quantize_ref(np.ascontiguousarray(x.T), axis=1, rotate="hadamard")
    assert np.array_equal(q0.codes, q1.codes) and np.array_equal(q0.scales, q1.scales)


def test_sliced_quantization_uses_global_indices():
    rng = np.random.default_rng(8)
    x = f32_to_bf16_bits(rng.standard_normal((64, 96)).astype(np.float32))
    full = oracle.quantize_ref(x, axis=1, rotate="rand_sign_hadamard", rounding="sr", seed=5)
    rows = np.array([3, 17, 60])
    part = oracle.quantize_ref(x[rows], axis=1, rotate="rand_sign_hadamard", rounding="sr",
                               seed=5, row_index=rows, total_cols=96)
    assert np.array_equal(part.codes, full.codes[rows])
    full0 = oracle.quantize_ref(x, axis=0, rotate="rand_sign_hadamard", rounding="sr", seed=5)
    cols = np.array([0, 1, 50, 95])
    part0 = oracle.quantize_ref(x[:, cols], axis=0, rotate="rand_sign_hadamard", rounding="sr",
                                seed=5, col_index=cols, total_cols=96)
    assert np.array_equal(part0.codes, full0.codes[cols])


def test_pack_roundtrip_and_nibble_order():
    c = np.array([[1, 2, 3, 4]], np.uint8)
    p = oracle.pack_codes(c)
    assert list(p[0]) == [0x21, 0x43]
    assert np.array_equal(oracle.unpack_codes(p), c)


# ----------------------------------------------------------------------- GEMM
def test_gemm_matches_triple_loop_and_exact_fractions():
    rng = np.random.default_rng(9)
    a = f32_to_bf16_bits(rng.standard_normal((12, 64)).astype(np.float32))
    b = f32_to_bf16_bits(rng.standard_normal((10, 64)).astype(np.float32))
    qa = oracle.quantize_ref(a, 1)
    qb = oracle.quantize_ref(b, 1)
    C = oracle.mx_gemm_ref(qa, qb)
    vals = [oracle.e2m1_value(c) for c in range(16)]
    for m in range(12):
        for n in range(10):
            acc = Fraction(0)
            for k in range(64):
                va = Fraction(vals[qa.codes[m, k]]) * Fraction(2) ** (int(qa.scales[m, k // 32]) - 127)
                vb = Fraction(vals[qb.codes[n, k]]) * Fraction(2) ** (int(qb.scales[n, k // 32]) - 127)
                acc += va * vb
            assert C[m, n] == float(acc)


def test_rotation_cancels_in_product():
    rng = np.random.default_rng(10)
    a = f32_to_bf16_bits(rng.standard_normal((40, 128)).astype(np.float32))
    b = f32_to_bf16_bits(rng.standard_normal((24, 128)).astype(np.float32))
    exact = bf16_bits_to_f32(a).astype(np.float64) @ bf16_bits_to_f32(b).astype(np.float64).T
    for rot, seed in (("hadamard", 0), ("rand_sign_hadamard", 11), ("hadamard16", 0)):
        qa = oracle.quantize_ref(a, 1, rotate=rot, seed=seed)
        qb = oracle.quantize_ref(b, 1, rotate=rot, seed=seed | (1 << 32))
        rot_prod = qa.rotated.astype(np.float64) @ qb.rotated.astype(np.float64).T
        assert np.max(np.abs(rot_prod - exact)) < 1e-5 * np.max(np.abs(exact))


def test_linear_ops_follow_their_definitions():
    """Fprop Y = X W^T, Dgrad dX = dY W, Wgrad dW = dY^T X: the MX result sits
    within MXFP4 quantization error of the exact product of the bf16 inputs."""
    rng = np.random.default_rng(11)
    T, o, i = 96, 64, 128
    X = f32_to_bf16_bits(rng.standard_normal((T, i)).astype(np.float32))
    W = f32_to_bf16_bits(rng.standard_normal((o, i)).astype(np.float32))
    dY = f32_to_bf16_bits(rng.standard_normal((T, o)).astype(np.float32))
    Xf, Wf, dYf = (bf16_bits_to_f32(t).astype(np.float64) for t in (X, W, dY))
    cases = {"fprop": (X, W, Xf @ Wf.T), "dgrad": (dY, W, dYf @ Wf), "wgrad": (dY, X, dYf.T @ Xf)}
    for op, (a, b, exact) in cases.items():
        for rot, rnd in (("hadamard", "rne"), ("none", "rne"), ("rand_sign_hadamard", "sr"),
                         ("hadamard16", "rne")):
            C, _, _ = oracle.linear_ref(op, a, b, rotate=rot, rounding=rnd, seed=3)
            assert C.shape == exact.shape
            rel = np.linalg.norm(C - exact) / np.linalg.norm(exact)
            assert rel < 0.25, (op, rot, rnd, rel)


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round_ref(x), want)


def test_tiled_layout_addresses_and_roundtrip():
    """Every element's byte address in the tiled buffer follows the layout
    formula (written here as an explicit loop), and untile inverts tile."""
    rng = np.random.default_rng(13)
    for mn, k in ((37, 160), (16, 128), (5, 32), (33, 256), (300, 128)):
        codes = rng.integers(0, 16, (mn, k)).astype(np.uint8)
        scales = rng.integers(0, 255, (mn, k // 32)).astype(np.uint8)
        tb = oracle.tile_codes(codes)
        sb = oracle.tile_scales(scales, k)
        mnp, kp = oracle.padded_extents(mn, k)
        assert tb.size == mnp * kp // 2 and sb.size == mnp * kp // 32
        assert mnp % 256 == 0 and mnp >= mn and mnp - mn < 256
        NT = mnp // 256
        for m in range(mn):
            for kk in range(0, k, 7):
                g, r, q, c = m // 16, m % 16, kk // 128, (kk % 128) // 32
                byte = (g * (kp // 128) + q) * 1024 + c * 256 + r * 16 + (kk % 32) // 2
                nib = (tb[byte] >> 4) if kk % 2 else (tb[byte] & 15)
                assert nib == codes[m, kk]
            for kb in range(k // 32):
                T, h, r, q, c = m // 256, (m // 16) % 16, m % 16, kb // 4, kb % 4
                assert sb[(q * NT + T) * 1024 + (h // 4) * 256 + c * 64 + r * 4 + h % 4] == \
                    scales[m, kb]
        # padding: zero codes, scale code 0
        full = oracle.untile_codes(tb, mnp, kp)
        assert np.all(full[mn:] == 0) and np.all(full[:, k:] == 0)
        assert np.array_equal(oracle.untile_codes(tb, mn, k), codes)
        assert np.array_equal(oracle.untile_scales(sb, mn, k), scales)


# ------------------------------------------------- E4M3 comparator (MXFP8)
def _e4m3_torch_decode():
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_table_matches_torch():
    """All 256 E4M3 codes decode as torch's float8_e4m3fn does (bias 7,
    subnormals at exponent 0, NaN only at S.1111.111, largest finite 448)."""
    want = _e4m3_torch_decode()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9
    assert np.all(np.diff(oracle.e4m3_magnitudes()) > 0)


def test_e4m3_rne_matches_torch_and_brute_force():
    """Round to nearest even: torch's fp32 -> float8_e4m3fn conversion on
    every midpoint, its fp32 neighbours and random values below 464 (torch
    rounds 448..464 down to 448 like the saturating rule); a brute-force
    nearest search decides the non-ties."""
    torch = pytest.importorskip("torch")
    g = oracle.e4m3_magnitudes()
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    rng = np.random.default_rng(21)
    vals = np.concatenate([
        g.astype(np.float32), mids, np.nextafter(mids, np.float32(0)),
        np.nextafter(mids, np.float32(1e9)),
        (rng.random(200000) * 463.9).astype(np.float32),
        (2.0 ** rng.uniform(-14, 8.8, 200000)).astype(np.float32)])
    vals = vals[vals < 464]
    got = oracle.round_e4m3_rne(vals)
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    # brute force: a non-tie goes to the strictly nearest magnitude
    v64 = vals.astype(np.float64)[:5000]
    d = np.abs(v64[:, None] - g[None, :])
    best = np.argmin(d, axis=1)
    srt = np.sort(d, axis=1)
    clear = srt[:, 0] < srt[:, 1]
    assert np.array_equal(got[:5000][clear], best[clear])


def test_e4m3_saturates_at_448():
    """Scaled values t in [448, 512) (possible since 2^-e * amax < 2^9) take
    the largest finite code 0x7E, never the NaN code."""
    for v in (448.0, 448.5, 463.9, 464.0, 480.0, 511.99):
        assert oracle.round_e4m3_rne(np.array([v], np.float32))[0] == 0x7E


def test_e4m3_one_hot_block():
    """H32 of a one-hot block: every y = +-c, c = 0.17677669; floor(log2 c) =
    -3 -> e = -3 - 8 = -11 (scale code 116); t = c * 2^11 = 362.04, between
    352 and 384 -> 352 = 1.375 * 2^8 (code 0x7B); dequantized 0.171875."""
    H = oracle.sylvester_hadamard(32)
    for j in (0, 9, 31):
        x = np.zeros((1, 32), np.float32)
        x[0, j] = 1.0
        q = oracle.quantize_ref(_bf16(x), axis=1, rotate="hadamard", fmt="fp8_e4m3")
        assert q.scales[0, 0] == 116
        assert np.array_equal(q.codes[0], np.where(H[:, j] > 0, 0x7B, 0xFB))
        d = oracle.dequantize_ref(q.codes, q.scales, "fp8_e4m3")[0]
        assert np.allclose(np.abs(d), 0.171875)


def test_e4m3_constant_zero_and_nan_blocks():
    """x = 1 without rotation: e = 0 - 8 (scale 119), t = 256 -> code 0x78.
    A zero block takes scale code 0 and zero codes; a NaN block scale 0xFF."""
    x = np.zeros((3, 64), np.float32)
    x[0, :32] = 1.0
    x[2, 33] = np.nan
    q = oracle.quantize_ref(_bf16(x), axis=1, rotate="none", fmt="fp8_e4m3")
    assert q.scales[0, 0] == 119 and np.all(q.codes[0, :32] == 0x78)
    assert q.scales[1, 0] == 0 and np.all(q.codes[1] == 0)
    assert q.scales[2, 1] == 0xFF and np.all(q.codes[2, 32:] == 0)
    with pytest.raises(ValueError):
        oracle.quantize_ref(_bf16(x), axis=1, rounding="sr", fmt="fp8_e4m3")


def test_e4m3_requantizing_representable_block_is_fixed_point():
    rng = np.random.default_rng(22)
    for trial in range(400):
        s = int(rng.integers(10, 240))
        codes = rng.integers(0, 256, 32).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0
        codes[rng.integers(0, 32)] = rng.integers(0x78, 0x7F) | (rng.integers(0, 2) << 7)
        d = oracle.dequantize_ref(codes[None], np.array([[s]], np.uint8), "fp8_e4m3")
        x = _bf16(d.astype(np.float32))
        assert np.array_equal(bf16_bits_to_f32(x).astype(np.float64), d)
        q = oracle.quantize_ref(x, axis=1, rotate="none", fmt="fp8_e4m3")
        assert q.scales[0, 0] == s
        # -0 codes come back as +0 only where the input bf16 was +0
        assert np.array_equal(q.codes[0] & 0x7F, codes & 0x7F)
        nz = (codes & 0x7F) != 0
        assert np.array_equal(q.codes[0][nz], codes[nz])


def test_e4m3_gemm_matches_exact_fractions():
    rng = np.random.default_rng(23)
    a = f32_to_bf16_bits(rng.standard_normal((9, 64)).astype(np.float32))
    b = f32_to_bf16_bits(rng.standard_normal((7, 64)).astype(np.float32))
    qa = oracle.quantize_ref(a, 1, fmt="fp8_e4m3")
    qb = oracle.quantize_ref(b, 1, fmt="fp8_e4m3")
    C = oracle.mx_gemm_ref(qa, qb)
    for m in range(9):
        for n in range(7):
            acc = Fraction(0)
            for k in range(64):
                va = Fraction(oracle.e4m3_value(int(qa.codes[m, k]))) * \
                    Fraction(2) ** (int(qa.scales[m, k // 32]) - 127)
                vb = Fraction(oracle.e4m3_value(int(qb.codes[n, k]))) * \
                    Fraction(2) ** (int(qb.scales[n, k // 32]) - 127)
                acc += va * vb
            assert C[m, n] == float(acc)


def test_e4m3_linear_error_is_below_e2m1():
    """With three mantissa bits instead of one the MXFP8 product of the same
    operands sits far closer to the exact product than the MXFP4 one."""
    rng = np.random.default_rng(24)
    X = f32_to_bf16_bits(rng.standard_normal((64, 128)).astype(np.float32))
    W = f32_to_bf16_bits(rng.standard_normal((48, 128)).astype(np.float32))
    exact = bf16_bits_to_f32(X).astype(np.float64) @ bf16_bits_to_f32(W).astype(np.float64).T
    for rot in ("hadamard", "none"):
        c8, _, _ = oracle.linear_ref("fprop", X, W, rotate=rot, fmt="fp8_e4m3")
        c4, _, _ = oracle.linear_ref("fprop", X, W, rotate=rot)
        e8 = np.linalg.norm(c8 - exact) / np.linalg.norm(exact)
        e4 = np.linalg.norm(c4 - exact) / np.linalg.norm(exact)
        assert e8 < 0.05 and e8 < e4 / 3, (rot, e8, e4)


def test_e4m3_tiled_layout_addresses_and_roundtrip():
    rng = np.random.default_rng(25)
    for mn, k in ((37, 160), (16, 128), (300, 64)):
        codes = rng.integers(0, 256, (mn, k)).astype(np.uint8)
        tb = oracle.tile_codes_fp8(codes)
        mnp, kp = oracle.padded_extents(mn, k)
        assert tb.size == mnp * kp
        for m in range(mn):
            for kk in range(0, k, 5):
                g, r, q = m // 16, m % 16, kk // 128
                j, i = (kk % 128) // 16, kk % 16
                assert tb[(g * (kp // 128) + q) * 2048 + j * 256 + r * 16 + i] == codes[m, kk]
        full = oracle.untile_codes_fp8(tb, mnp, kp)
        assert np.all(full[mn:] == 0) and np.all(full[:, k:] == 0)
        assert np.array_equal(oracle.untile_codes_fp8(tb, mn, k), codes)
