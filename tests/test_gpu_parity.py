"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bar: E2M1 codes and E8M0 scales bit-exact (stochastic rounding included, for
a given seed); GEMM outputs within 1e-5 relative Frobenius error of the fp64
oracle GEMM over the dequantized operands, and every element within
(K/32 + 4) 2^-23 sum_k |a b| of it (fp32 accumulation of exact block sums);
bf16 outputs equal to the round-to-nearest-even of the same GEMM's fp32
output.
"""
import numpy as np
import pytest

import oracle
from datagen import (WORKLOADS, f32_to_bf16_bits, operands_for, workload_tensors)
from gpu_util import host_u8, rel_fro, to_dev, to_dev_strided
from oracle_util import oracle_operand

pytestmark = pytest.mark.gpu

ROTS = ("none", "hadamard", "rand_sign_hadamard", "hadamard16")
RNDS = ("rne", "sr")
GEMM_TOL = 1e-5


def _sync():
    import torch
    torch.cuda.synchronize()


def _check_q(q_gpu, ref, what=""):
    """Byte-exact comparison of the GPU's tiled buffers with the oracle's
    codes and scales packed into the same tiled layout (padding included)."""
    codes = host_u8(q_gpu.codes)
    scales = host_u8(q_gpu.scales)
    k = ref.codes.shape[1]
    want_codes = oracle.tile_codes(ref.codes)
    want_scales = oracle.tile_scales(ref.scales, k)
    assert codes.shape == want_codes.shape and scales.shape == want_scales.shape, what
    bad = np.count_nonzero(codes != want_codes)
    bad_s = np.count_nonzero(scales != want_scales)
    assert bad == 0 and bad_s == 0, f"{what}: {bad} code bytes, {bad_s} scales differ"


def _check_elementwise(got, C_ref, ra, rb, what=""):
    """Every element within (K/32 + 4) 2^-23 sum_k |a b| of the fp64 product:
    fp32 accumulation of K/128 exactly summed MFMA blocks, with a wide
    margin."""
    da = np.abs(oracle.dequantize_ref(ra.codes, ra.scales, ra.fmt))
    db = np.abs(oracle.dequantize_ref(rb.codes, rb.scales, rb.fmt))
    k = ra.codes.shape[1]
    bound = (k / 32 + 4) * 2.0 ** -23 * (da @ db.T)
    over = np.count_nonzero(np.abs(np.asarray(got, np.float64) - C_ref) > bound)
    assert over == 0, f"{what}: {over} elements beyond the per-element bound"


def _rand_bits(rng, shape, scale=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


# ------------------------------------------------------------------ quantizer
@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("rot", ROTS)
@pytest.mark.parametrize("rnd", RNDS)
def test_quantize_small_ragged(mx, axis, rot, rnd):
    rng = np.random.default_rng(100 + axis)
    shape = (37, 160) if axis == 1 else (160, 37)      # ragged non-axis extent
    x = _rand_bits(rng, shape)
    seed = 0x1234 | (1 << 32)
    q = mx.quantize(to_dev(x), axis=axis, rotate=rot, round=rnd, seed=seed)
    _sync()
    ref = oracle.quantize_ref(x, axis, rotate=rot, rounding=rnd, seed=seed)
    _check_q(q, ref, f"axis={axis} rot={rot} rnd={rnd}")


@pytest.mark.parametrize("axis", [1, 0])
def test_quantize_strided_input(mx, axis):
    rng = np.random.default_rng(7)
    shape = (64, 96) if axis == 1 else (96, 66)
    x = _rand_bits(rng, shape, 3.0)
    t = to_dev_strided(x, ld=shape[1] + 30 + (8 - (shape[1] + 30) % 8) % 8)
    q = mx.quantize(t, axis=axis, rotate="rand_sign_hadamard", round="sr", seed=99)
    _sync()
    _check_q(q, oracle.quantize_ref(x, axis, rotate="rand_sign_hadamard", rounding="sr", seed=99))


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("rot", ("none", "hadamard", "hadamard16"))
@pytest.mark.parametrize("rnd", RNDS)
def test_quantize_every_bf16_pattern(mx, axis, rot, rnd):
    """All 65536 bf16 bit patterns (NaN/Inf/subnormal included), plus every
    pattern again with a 7.97 anchor leading each block; both roundings (the
    stochastic one puts every E2M1 interval and its subnormal range under
    the Philox draws)."""
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    blocks = allv.reshape(2048, 32)
    n_anch = -(-65536 // 31)
    pad = np.zeros(n_anch * 31, np.uint16)
    pad[:65536] = allv
    anch = np.concatenate([np.full((n_anch, 1), 0x40FF, np.uint16), pad.reshape(n_anch, 31)], 1)
    x = np.concatenate([blocks, anch], 0)
    if axis == 0:
        x = np.ascontiguousarray(x.T)
    q = mx.quantize(to_dev(x), axis=axis, rotate=rot, round=rnd, seed=0x5EED)
    _sync()
    _check_q(q, oracle.quantize_ref(x, axis, rotate=rot, rounding=rnd, seed=0x5EED),
             f"axis={axis} rot={rot} rnd={rnd}")


@pytest.mark.parametrize("rot", ROTS)
def test_quantize_every_bf16_pattern_axis0_quad_sr(mx, rot):
    """Every bf16 pattern down the columns of an axis-0 operand whose column
    count is a multiple of four, the case where stochastic rounding takes the
    quad-shared Philox kernel (one zero column pads 4163 columns to 4164)."""
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    n_anch = -(-65536 // 31)
    pad = np.zeros(n_anch * 31, np.uint16)
    pad[:65536] = allv
    anch = np.concatenate([np.full((n_anch, 1), 0x40FF, np.uint16), pad.reshape(n_anch, 31)], 1)
    x = np.concatenate([allv.reshape(2048, 32), anch, np.zeros((1, 32), np.uint16)], 0)
    x = np.ascontiguousarray(x.T)
    assert x.shape[1] % 4 == 0
    q = mx.quantize(to_dev(x), axis=0, rotate=rot, round="sr", seed=0x5EED | (1 << 32))
    _sync()
    _check_q(q, oracle.quantize_ref(x, 0, rotate=rot, rounding="sr", seed=0x5EED | (1 << 32)),
             f"quad sr rot={rot}")


@pytest.mark.parametrize("rot", ROTS)
@pytest.mark.parametrize("rnd", RNDS)
def test_quantize_special_blocks(mx, rot, rnd):
    f = np.float32
    rows = [
        np.zeros(32, f), np.full(32, -0.0, f), np.ones(32, f),
        np.eye(32, dtype=f)[3], np.full(32, 3.0e38, f),            # overflow inside the butterfly
        np.where(np.arange(32) % 2 == 0, 3.0e38, -3.0e38).astype(f),
        np.full(32, 1e-40, f), np.linspace(-1e-39, 1e-39, 32).astype(f),
        np.r_[np.full(31, 1.0, f), f(np.inf)], np.r_[np.full(31, 1.0, f), f(-np.inf)],
        np.r_[np.full(31, 1.0, f), f(np.nan)], np.r_[np.full(16, f(np.inf)), np.full(16, -np.inf)].astype(f),
        np.full(32, 5.0, f), np.full(32, 2.5, f), np.full(32, 0.75, f),
        np.linspace(-6, 6, 32).astype(f), np.ldexp(np.ones(32, f), np.arange(-16, 16)).astype(f),
    ]
    x = f32_to_bf16_bits(np.stack(rows))
    x = np.concatenate([x, x[::-1]], 1)                    # 64 columns
    for axis in (1, 0):
        xa = x if axis == 1 else np.ascontiguousarray(x.T)
        q = mx.quantize(to_dev(xa), axis=axis, rotate=rot, round=rnd, seed=3)
        _sync()
        _check_q(q, oracle.quantize_ref(xa, axis, rotate=rot, rounding=rnd, seed=3),
                 f"axis={axis} rot={rot} rnd={rnd}")


def test_quantize_determinism_and_seed_use(mx):
    rng = np.random.default_rng(11)
    x = to_dev(_rand_bits(rng, (128, 256)))
    a = mx.quantize(x, 1, "hadamard", "rne", seed=1)
    b = mx.quantize(x, 1, "hadamard", "rne", seed=2)            # seed unused
    c = mx.quantize(x, 1, "none", "sr", seed=5)
    d = mx.quantize(x, 1, "none", "sr", seed=5)
    e = mx.quantize(x, 1, "none", "sr", seed=6)
    _sync()
    assert np.array_equal(host_u8(a.codes), host_u8(b.codes))
    assert np.array_equal(host_u8(c.codes), host_u8(d.codes))
    assert not np.array_equal(host_u8(c.codes), host_u8(e.codes))


def test_quantize_empty(mx):
    import torch
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q = mx.quantize(x, 1)
    assert q.codes.numel() == 0 and q.scales.numel() == 0


# ------------------------------------------------------------ dual output
@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (96, 160), (320, 384), (160, 256)])
@pytest.mark.parametrize("rot", ROTS)
@pytest.mark.parametrize("rnd", RNDS)
def test_quantize_dual_matches_oracle_and_single(mx, shape, rot, rnd):
    """Both outputs equal the oracle's axis-1 and axis-0 quantizations (tiled,
    padding included) and the two single-axis launches, byte for byte."""
    rng = np.random.default_rng(shape[0] * 13 + shape[1])
    x = _rand_bits(rng, shape)
    xd = to_dev(x)
    q1, q0 = mx.quantize_dual(xd, rot, rnd, seed1=21, seed0=22 | (1 << 32))
    s1 = mx.quantize(xd, 1, rot, rnd, seed=21)
    s0 = mx.quantize(xd, 0, rot, rnd, seed=22 | (1 << 32))
    _sync()
    _check_q(q1, oracle.quantize_ref(x, 1, rotate=rot, rounding=rnd, seed=21), f"dual axis 1 {shape}")
    _check_q(q0, oracle.quantize_ref(x, 0, rotate=rot, rounding=rnd, seed=22 | (1 << 32)),
             f"dual axis 0 {shape}")
    for a, b in ((q1, s1), (q0, s0)):
        assert np.array_equal(host_u8(a.codes), host_u8(b.codes))
        assert np.array_equal(host_u8(a.scales), host_u8(b.scales))


@pytest.mark.parametrize("rot", ROTS)
@pytest.mark.parametrize("rnd", RNDS)
def test_quantize_dual_every_bf16_pattern(mx, rot, rnd):
    """Every bf16 bit pattern (NaN/Inf/subnormal included) through the dual
    quantizer's fp32 staging, in row blocks (axis 1) and column blocks
    (axis 0): the 65536 patterns, every pattern again behind a 7.97 anchor,
    and the special blocks (zeros, overflow inside the butterfly, lone
    NaN/Inf, subnormal ramps); both outputs against the oracle."""
    f = np.float32
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    n_anch = -(-65536 // 31)
    pad = np.zeros(n_anch * 31, np.uint16)
    pad[:65536] = allv
    anch = np.concatenate([np.full((n_anch, 1), 0x40FF, np.uint16), pad.reshape(n_anch, 31)], 1)
    special = f32_to_bf16_bits(np.stack([
        np.zeros(32, f), np.full(32, -0.0, f), np.full(32, 3.0e38, f),
        np.where(np.arange(32) % 2 == 0, 3.0e38, -3.0e38).astype(f),
        np.full(32, 1e-40, f), np.linspace(-1e-39, 1e-39, 32).astype(f),
        np.r_[np.full(31, 1.0, f), f(np.inf)], np.r_[np.full(31, 1.0, f), f(np.nan)],
        np.r_[np.full(16, f(np.inf)), np.full(16, -np.inf)].astype(f),
        np.linspace(-6, 6, 32).astype(f), np.ldexp(np.ones(32, f), np.arange(-16, 16)).astype(f)]))
    x = np.concatenate([allv.reshape(2048, 32), anch, special], 0)
    x = np.concatenate([x, np.zeros((-x.shape[0] % 32, 32), np.uint16)], 0)   # rows % 32 == 0
    x = np.concatenate([x, x[::-1]], 1)      # 64 columns; column blocks mix other patterns
    s1, s0 = 0x5EED, 0x5EED | (1 << 32)
    q1, q0 = mx.quantize_dual(to_dev(x), rot, rnd, seed1=s1, seed0=s0)
    _sync()
    _check_q(q1, oracle.quantize_ref(x, 1, rotate=rot, rounding=rnd, seed=s1), f"dual axis 1 {rot} {rnd}")
    _check_q(q0, oracle.quantize_ref(x, 0, rotate=rot, rounding=rnd, seed=s0), f"dual axis 0 {rot} {rnd}")


def test_quantize_dual_strided_and_full_size(mx):
    """A row-strided source, and the full-size Fprop activation (8192 x 4096)
    against the single-axis launches."""
    import torch
    rng = np.random.default_rng(77)
    x = _rand_bits(rng, (128, 192))
    q1, q0 = mx.quantize_dual(to_dev_strided(x, ld=200), "hadamard", "rne")   # NaN in the gap
    _sync()
    _check_q(q1, oracle.quantize_ref(x, 1), "strided dual axis 1")
    _check_q(q0, oracle.quantize_ref(x, 0), "strided dual axis 0")
    w = WORKLOADS["fprop_q_proj"]
    X = to_dev(workload_tensors(w)["X"])
    q1, q0 = mx.quantize_dual(X, "hadamard", "rne", seed1=0, seed0=0)
    s1 = mx.quantize(X, 1)
    s0 = mx.quantize(X, 0)
    _sync()
    for a, b in ((q1, s1), (q0, s0)):
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


# ----------------------------------------------------------------------- GEMM
def _gemm_case(mx, op, a_src, b_src, rot, rnd, seed, check_bf16=True):
    ax_a, ax_b = mx.OP_AXES[op]
    qa = mx.quantize(to_dev(a_src), ax_a, rot, rnd, seed=seed & 0xFFFFFFFF)
    qb = mx.quantize(to_dev(b_src), ax_b, rot, rnd, seed=(seed & 0xFFFFFFFF) | (1 << 32))
    c32 = mx.linear(op, qa, qb, "f32")
    c16 = mx.linear(op, qa, qb, "bf16") if check_bf16 else None
    _sync()
    C_ref, ra, rb = oracle.linear_ref(op, a_src, b_src, rotate=rot, rounding=rnd, seed=seed)
    _check_q(qa, ra, f"{op} A")
    _check_q(qb, rb, f"{op} B")
    got = c32.cpu().numpy()
    err = rel_fro(got, C_ref)
    assert err <= GEMM_TOL, f"{op} {rot} {rnd}: rel Frobenius {err:.3e}"
    _check_elementwise(got, C_ref, ra, rb, f"{op} {rot} {rnd}")
    if check_bf16:
        import torch
        b16 = c16.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(b16, oracle.bf16_round_ref(got)), "bf16 epilogue != RNE(fp32)"
    return err


def _designed_operand(mx, codes, scales):
    """A quantized operand built directly from codes [MN, K] and E8M0 scales
    [MN, K/32] (reduction-major, no rotation), tiled by the oracle's layout
    functions, as an axis-1 descriptor of a [MN, K] source."""
    import torch
    mn, k = codes.shape
    c = torch.from_numpy(oracle.tile_codes(codes)).cuda()
    s = torch.from_numpy(oracle.tile_scales(scales, k)).cuda()
    d = mx.QTensorDesc(c.data_ptr(), s.data_ptr(), mn, k, 1, 32, mx.ROTATE["none"],
                       mx.ROUND["rne"], 0, mx.FORMATS["fp4_e2m1"])
    return mx.QTensor(c, s, d)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_exact_on_designed_operands(mx, out_dtype):
    """Every pair of E2M1 codes (both signs, both zeros) meets in the
    products, under per-block scales 2^-2 .. 2^2 (A) and 2^-1 .. 2^1 (B)
    that change from block to block. Every product is a multiple of 2^-5
    and every partial sum stays below 2^17, so fp32 accumulation in any
    order is exact: the output must equal the fp64 product exactly (bf16:
    its nearest-even rounding). Four output tiles, three K slices."""
    M, N, K = 512, 512, 384
    m, n, k = np.arange(M)[:, None], np.arange(N)[:, None], np.arange(K)[None, :]
    kb = np.arange(K // 32)[None, :]
    ca = ((m * 7 + k) % 16).astype(np.uint8)
    cb = ((n * 5 + 3 * k) % 16).astype(np.uint8)
    sa = (125 + (m + kb) % 5).astype(np.uint8)
    sb = (126 + (3 * n + kb) % 3).astype(np.uint8)
    qa, qb = _designed_operand(mx, ca, sa), _designed_operand(mx, cb, sb)
    got = mx.linear("fprop", qa, qb, out_dtype)
    _sync()
    ref = oracle.dequantize_ref(ca, sa) @ oracle.dequantize_ref(cb, sb).T
    assert np.all(np.abs(ref) < 2.0 ** 17)
    want = ref.astype(np.float32)
    assert np.array_equal(want.astype(np.float64), ref)              # exact in fp32
    if out_dtype == "bf16":
        import torch
        g = got.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(g, oracle.bf16_round_ref(want))
    else:
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_gemm_nan_scale_block(mx):
    """A block whose scale is the NaN code 0xFF (what the quantizers write,
    with zero codes, for a block holding a NaN or Inf) makes every output
    that reduces over it NaN, as in the oracle's fp64 product; the rest of
    C is unaffected."""
    M, N, K = 256, 256, 256
    rng = np.random.default_rng(5)
    ca = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, (N, K)).astype(np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    ca[37, 64:96] = 0
    sa[37, 2] = 0xFF                      # row 37 of A, block 2
    cb[200, 224:256] = 0
    sb[200, 7] = 0xFF                     # row 200 of B (column 200 of C), block 7
    qa, qb = _designed_operand(mx, ca, sa), _designed_operand(mx, cb, sb)
    got = mx.linear("fprop", qa, qb, "f32")
    _sync()
    ref = oracle.dequantize_ref(ca, sa) @ oracle.dequantize_ref(cb, sb).T
    g = got.cpu().numpy()
    assert np.array_equal(np.isnan(g), np.isnan(ref))
    assert np.isnan(ref[37]).all() and np.isnan(ref[:, 200]).all()
    fin = ~np.isnan(ref)
    assert np.array_equal(g[fin], ref[fin].astype(np.float32))       # small exact sums


def test_gemm_tiny_wgrad_workload(mx):
    """dY 256x128 and X 256x96, N(0,1), seed 0; H32 + RNE along the 256 tokens;
    dW = dY^T X, 128x96 fp32."""
    w = WORKLOADS["tiny_wgrad"]
    t = workload_tensors(w)
    a, _, b, _ = operands_for(w, t)
    _gemm_case(mx, "wgrad", a, b, "hadamard", "rne", 0)


@pytest.mark.parametrize("op", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("rot,rnd", [("hadamard", "rne"), ("rand_sign_hadamard", "rne"),
                                     ("none", "sr"), ("none", "rne"), ("hadamard16", "rne"),
                                     ("hadamard16", "sr")])
def test_gemm_ops_ragged(mx, op, rot, rnd):
    """T=224, out=96, in=160: every op has M, N off the 128 tile and a K tail."""
    rng = np.random.default_rng(21)
    T, o, i = 224, 96, 160
    X = _rand_bits(rng, (T, i))
    W = _rand_bits(rng, (o, i), 0.02)
    dY = f32_to_bf16_bits((rng.standard_t(3, (T, o)) * 1e-4).astype(np.float32))
    a, b = {"fprop": (X, W), "dgrad": (dY, W), "wgrad": (dY, X)}[op]
    _gemm_case(mx, op, a, b, rot, rnd, 11)


@pytest.mark.parametrize("M,N,K", [(300, 200, 384), (520, 260, 640), (256, 256, 128),
                                   (1, 1, 128), (257, 513, 1152)])
def test_gemm_lds_path_tails(mx, M, N, K):
    """K % 128 == 0 (the LDS-staged kernel) with ragged M / N and a half-stage
    K tail (K % 256 == 128)."""
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A = _rand_bits(rng, (M, K))
    B = _rand_bits(rng, (N, K), 0.5)
    _gemm_case(mx, "fprop", A, B, "hadamard", "rne", 0)


@pytest.mark.parametrize("op", ["fprop", "wgrad"])
@pytest.mark.parametrize("M,N", [(1243, 15355), (2148, 4133), (1000, 900)])
def test_gemm_launch_paths(mx, op, M, N):
    """The launcher's three paths on a 256-compute-unit MI355X (tiles of
    256 x 256): 1243 x 15355 is 300 tiles, 256 whole ones then the other 44 as
    88 half tiles (rows 128 h .. 128 h + 127 of a tile); 2148 x 4133 is 153
    whole tiles; 1000 x 900 is 16 tiles, all run as 32 half tiles. Ragged in
    M, N and K (224); both output dtypes against the oracle, and a misaligned
    output pitch (the per-quad stores) equal bit for bit to the contiguous
    result."""
    import torch
    rng = np.random.default_rng(404 + M)
    K = 224
    if op == "fprop":                                  # X [T=M, in=K], W [out=N, in=K]
        a, b = _rand_bits(rng, (M, K)), _rand_bits(rng, (N, K), 0.02)
    else:                                              # dY [T=K, out=M], X [T=K, in=N]
        a, b = _rand_bits(rng, (K, M), 1e-2), _rand_bits(rng, (K, N))
    _gemm_case(mx, op, a, b, "hadamard", "rne", 0)
    ax_a, ax_b = mx.OP_AXES[op]
    qa = mx.quantize(to_dev(a), ax_a, "hadamard", "rne", seed=0)
    qb = mx.quantize(to_dev(b), ax_b, "hadamard", "rne", seed=1 << 32)
    for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        ref = mx.linear(op, qa, qb, dt)
        big = torch.full((M, N + 3), 7.0, dtype=tdt, device="cuda")
        mx.linear(op, qa, qb, dt, out=big[:, :N])
        _sync()
        assert torch.equal(big[:, :N], ref), f"{op} {dt}: strided output differs"
        assert torch.all(big[:, N:] == 7.0), f"{op} {dt}: pad columns written"


def test_gemm_several_tiles(mx):
    rng = np.random.default_rng(22)
    A = _rand_bits(rng, (640, 1024))
    B = _rand_bits(rng, (392, 1024))
    _gemm_case(mx, "fprop", A, B, "hadamard", "rne", 0)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("pad", [8, 4, 0, 1])
def test_gemm_strided_out(mx, out_dtype, pad):
    """Row-strided output: ldc = N + pad (the vector quad stores need ldc a
    multiple of 4; odd N and ldc take the element-wise stores in
    test_gemm_lds_path_tails). The result must equal the contiguous one bit
    for bit and the pad columns stay untouched."""
    import torch
    rng = np.random.default_rng(31 + pad)
    M, N, K = 300, 264, 384
    qa = mx.quantize(to_dev(_rand_bits(rng, (M, K))), 1)
    qb = mx.quantize(to_dev(_rand_bits(rng, (N, K))), 1)
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    ref = mx.linear("fprop", qa, qb, out_dtype)
    big = torch.full((M, N + pad), -7.0, dtype=dt, device="cuda")
    got = mx.linear("fprop", qa, qb, out_dtype, out=big[:, :N])
    _sync()
    iv = torch.int32 if out_dtype == "f32" else torch.int16
    assert torch.equal(got.contiguous().view(iv), ref.view(iv))
    if pad:
        assert torch.all(big[:, N:] == -7.0).item()


def test_gemm_k_zero_writes_zeros(mx):
    import torch
    A = mx.quantize(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), 0)
    B = mx.quantize(torch.empty((0, 48), dtype=torch.bfloat16, device="cuda"), 0)
    out = torch.full((64, 48), float("nan"), device="cuda")
    mx.linear("wgrad", A, B, "f32", out=out)
    _sync()
    assert torch.count_nonzero(out).item() == 0


def test_gemm_deterministic(mx):
    rng = np.random.default_rng(23)
    qa = mx.quantize(to_dev(_rand_bits(rng, (512, 2048))), 1)
    qb = mx.quantize(to_dev(_rand_bits(rng, (384, 2048))), 1)
    c1 = mx.linear("fprop", qa, qb)
    c2 = mx.linear("fprop", qa, qb)
    _sync()
    assert np.array_equal(c1.cpu().numpy().view(np.uint32), c2.cpu().numpy().view(np.uint32))


# --------------------------------------------- full-size workloads, sampled
FULL = [("fprop_q_proj", "det_hadamard"), ("fprop_q_proj", "det_hadamard16"),
        ("wgrad_gate_proj", "no_rotation"),
        ("wgrad_gate_proj", "det_hadamard"), ("dgrad_down_proj", "det_hadamard"),
        ("dgrad_down_proj", "det_hadamard_sr7")]


def _tile_cover(M, N):
    """256 x 256 output tiles such that every tile row and every tile column
    holds at least one whole tile: (i, i mod tn) and (j mod tm, j)."""
    tm, tn = -(-M // 256), -(-N // 256)
    return sorted({(i, i % tn) for i in range(tm)} | {(j % tm, j) for j in range(tn)})


@pytest.mark.parametrize("name,variant", FULL)
def test_full_size_sampled(mx, name, variant):
    """Full workload sizes in the launch configuration the bench times: both
    whole operands bit-exact against the oracle (codes and scales, padding
    excluded); the output on a set of whole 256 x 256 tiles covering every
    tile row and tile column within the per-element bound and 1e-5 relative
    Frobenius error; the bf16 epilogue over the whole output."""
    import torch
    w = WORKLOADS[name]
    print(f"[full] {name} {variant}", flush=True)
    _, rot, rnd, seed = [v for v in w.variants if v[0] == variant][0]
    t = workload_tensors(w)
    a_src, ax_a, b_src, ax_b = operands_for(w, t)
    seed_a, seed_b = seed & 0xFFFFFFFF, (seed & 0xFFFFFFFF) | (1 << 32)
    qa = mx.quantize(to_dev(a_src), ax_a, rot, rnd, seed=seed_a)
    qb = mx.quantize(to_dev(b_src), ax_b, rot, rnd, seed=seed_b)
    c = mx.linear(w.op, qa, qb, "f32")
    _sync()
    M, N = qa.mn, qb.mn
    ra = oracle_operand(a_src, ax_a, rot, rnd, seed_a)
    rb = oracle_operand(b_src, ax_b, rot, rnd, seed_b)
    for q, r, nm in ((qa, ra, "A"), (qb, rb, "B")):
        codes = oracle.untile_codes(host_u8(q.codes), q.mn, q.k)
        scales = oracle.untile_scales(host_u8(q.scales), q.mn, q.k)
        nb, ns = np.count_nonzero(codes != r.codes), np.count_nonzero(scales != r.scales)
        assert nb == 0 and ns == 0, f"{name}/{variant} {nm}: {nb} codes, {ns} scales differ"
        del codes, scales
    c_host = c.cpu().numpy()
    got_all, ref_all = [], []
    for ti, tj in _tile_cover(M, N):
        rs, cs = slice(256 * ti, min(M, 256 * ti + 256)), slice(256 * tj, min(N, 256 * tj + 256))
        sa_ = oracle.QuantRef(ra.codes[rs], ra.scales[rs], np.empty((0, 0), np.float32), ax_a)
        sb_ = oracle.QuantRef(rb.codes[cs], rb.scales[cs], np.empty((0, 0), np.float32), ax_b)
        C_ref = oracle.mx_gemm_ref(sa_, sb_)
        got = c_host[rs, cs]
        _check_elementwise(got, C_ref, sa_, sb_, f"{name}/{variant} tile ({ti}, {tj})")
        got_all.append(got.astype(np.float64).ravel())
        ref_all.append(C_ref.ravel())
    err = rel_fro(np.concatenate(got_all), np.concatenate(ref_all))
    assert err <= GEMM_TOL, f"{name}/{variant}: rel Frobenius {err:.3e}"
    if w.out_dtype == "bf16":
        # the bf16 epilogue over the whole output: RNE of the fp32 result
        cb = mx.linear(w.op, qa, qb, "bf16")
        _sync()
        got_b = cb.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got_b, oracle.bf16_round_ref(c_host))


# ------------------------------------------------- structural-error harness
def test_structural_error_harness_against_the_oracle(mx):
    """The repeated-Wgrad harness on a small problem, anchored on the oracle:
    for every variant and its first three steps, the quantized operands the
    harness used are bit-exact against oracle.linear_ref with the step's seed
    (seed k for the randomized variants, 0 otherwise; B takes k | 1 << 32)
    and each dW_k lies within 1e-5 of the oracle's product; the harness's
    reported errors (single-step and the 2-step mean, against the exact
    product of the bf16 operands) equal those recomputed from the oracle's
    dW_k within 1e-4 relative. Then the property the harness measures: a
    deterministic rotation reproduces dW bit for bit every step, so the
    K-step mean keeps the single-step error; a new seed per step (random
    signs, stochastic rounding) lets the mean's error fall."""
    import bench
    T, n_out, n_in = 512, 160, 96
    res = bench.structural_error(mx, T=T, n_out=n_out, n_in=n_in, steps=16, keep_steps=3)
    dY, X = bench.structural_inputs(T, n_out, n_in)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    exact = f(dY).T @ f(X)
    ex_norm = np.linalg.norm(exact)
    for label, rot, rnd, reseed in bench.STRUCTURAL_VARIANTS:
        steps = res["_steps"][label]
        refs = []
        for k, st in enumerate(steps, start=1):
            seed = bench.structural_step_seed(k, reseed)
            assert st["seed"] == seed
            C_ref, ra, rb = oracle.linear_ref("wgrad", dY, X, rotate=rot, rounding=rnd, seed=seed)
            want_a = (oracle.tile_codes(ra.codes), oracle.tile_scales(ra.scales, T))
            want_b = (oracle.tile_codes(rb.codes), oracle.tile_scales(rb.scales, T))
            assert np.array_equal(st["a_codes"], want_a[0]) and np.array_equal(st["a_scales"], want_a[1]), (label, k)
            assert np.array_equal(st["b_codes"], want_b[0]) and np.array_equal(st["b_scales"], want_b[1]), (label, k)
            err = rel_fro(st["dW"], C_ref)
            assert err <= GEMM_TOL, f"{label} step {k}: rel Frobenius {err:.3e}"
            refs.append(C_ref)
        v = res["variants"][label]
        want_single = [np.linalg.norm(r - exact) / ex_norm for r in refs]
        want_mean2 = np.linalg.norm((refs[0] + refs[1]) / 2 - exact) / ex_norm
        assert np.allclose(v["single_step_rel_err"][:3], want_single, rtol=1e-4), label
        assert abs(v["mean_rel_err"]["2"] - want_mean2) <= 1e-4 * want_mean2, label
    v = res["variants"]
    for det in ("det_hadamard", "det_hadamard16"):
        s_ = v[det]["single_step_rel_err"]
        assert len(set(s_)) == 1, det
        assert abs(v[det]["mean_rel_err"]["16"] - s_[0]) <= 1e-6 * s_[0], det
        dws = [st["dW"] for st in res["_steps"][det]]
        assert all(np.array_equal(dws[0], d) for d in dws[1:]), det
    for rnd in ("rand_sign_hadamard", "no_rotation_sr", "hadamard_sr"):
        assert v[rnd]["mean_rel_err"]["16"] < 0.7 * v[rnd]["single_step_rel_err"][0], rnd


# ----------------------------------------------------------- dequantization
@pytest.mark.parametrize("fmt", ["fp4_e2m1", "fp8_e4m3"])
@pytest.mark.parametrize("axis", [1, 0])
def test_dequantize_matches_oracle(mx, fmt, axis):
    """mx_dequantize against the oracle's dequantization of the oracle's
    codes, bit for bit (every value is exact in fp32): a ragged operand in
    its source orientation, a row-strided output whose pad columns stay
    untouched, and NaN / zero / denormal blocks."""
    import torch
    rng = np.random.default_rng(88 + axis)
    shape = (300, 224) if axis == 1 else (224, 300)
    x = _rand_bits(rng, shape, 2.0)
    f = np.float32
    specials = f32_to_bf16_bits(np.stack([np.zeros(32, f), np.r_[np.ones(31, f), f(np.nan)],
                                          np.full(32, 1e-39, f)]))
    if axis == 1:
        x[:3, :32] = specials
    else:
        x[:32, :3] = specials.T
    xd = to_dev(x)
    if fmt == "fp4_e2m1":
        q = mx.quantize(xd, axis, "hadamard", "sr", seed=5)
        ref = oracle.quantize_ref(x, axis, rotate="hadamard", rounding="sr", seed=5)
    else:
        q = mx.quantize_fp8(xd, axis, "hadamard", seed=5)
        ref = oracle.quantize_ref(x, axis, rotate="hadamard", fmt="fp8_e4m3", seed=5)
    want = oracle.dequantize_ref(ref.codes, ref.scales, ref.fmt).astype(np.float32)   # [MN, K]
    if axis == 0:
        want = np.ascontiguousarray(want.T)
    got = mx.dequantize(q)
    big = torch.full((shape[0], shape[1] + 5), 7.0, dtype=torch.float32, device="cuda")
    mx.dequantize(q, out=big[:, :shape[1]])
    _sync()
    g = got.cpu().numpy()
    assert np.array_equal(np.isnan(g), np.isnan(want)) and np.isnan(want).any()
    assert np.array_equal(np.nan_to_num(g).view(np.uint32), np.nan_to_num(want).view(np.uint32))
    assert torch.equal(big[:, :shape[1]].nan_to_num(), got.nan_to_num())
    assert torch.all(big[:, shape[1]:] == 7.0)


def test_quantize_axis1_many_tiles_ragged(mx):
    """More tiles than resident waves (8200 x 2048: 8448 tiles of 16 x 128, the
    last 256-row panel ragged), so waves walk several tiles; every byte is
    checked, padding included, in both element formats."""
    rng = np.random.default_rng(61)
    x = _rand_bits(rng, (8200, 2048), 2.0)
    q = mx.quantize(to_dev(x), axis=1, rotate="hadamard", round="rne")
    q8 = mx.quantize_fp8(to_dev(x), axis=1, rotate="hadamard")
    _sync()
    _check_q(q, oracle.quantize_ref(x, 1, rotate="hadamard"), "fp4")
    ref8 = oracle.quantize_ref(x, 1, rotate="hadamard", fmt="fp8_e4m3")
    assert np.array_equal(host_u8(q8.codes), oracle.tile_codes_fp8(ref8.codes))
    assert np.array_equal(host_u8(q8.scales), oracle.tile_scales(ref8.scales, 2048))


def test_quantize_axis1_walk_with_slice_wrap(mx):
    """20000 x 608: 5 K slices (the last one ragged) and 6320 tiles, more than
    the resident waves, and a wave stride that is not a multiple of 5, so each
    wave's (row group, K slice) pair wraps the slice index as it walks; every
    byte checked."""
    rng = np.random.default_rng(62)
    x = _rand_bits(rng, (20000, 608))
    q = mx.quantize(to_dev(x), axis=1, rotate="hadamard", round="rne")
    _sync()
    _check_q(q, oracle.quantize_ref(x, 1, rotate="hadamard"), "walk with slice wrap")


@pytest.mark.parametrize("rot", ROTS)
@pytest.mark.parametrize("shape,ld", [((160, 100), 100), ((256, 64), 64), ((96, 516), 520),
                                      ((32, 4), 8)])
def test_quantize_axis0_sr_quad_shared_philox(mx, rot, shape, ld):
    """Axis-0 stochastic rounding with cols % 4 == 0, where the four lanes of a
    quad share each Philox call: ragged and aligned column counts, padded
    rows, a row stride above cols; bit-exact against the oracle."""
    rng = np.random.default_rng(71 + shape[1])
    x = _rand_bits(rng, shape, 1.5)
    t = to_dev(x) if ld == shape[1] else to_dev_strided(x, ld=ld)
    seed = 0xBEEF | (1 << 32)
    q = mx.quantize(t, axis=0, rotate=rot, round="sr", seed=seed)
    _sync()
    _check_q(q, oracle.quantize_ref(x, 0, rotate=rot, rounding="sr", seed=seed),
             f"rot={rot} shape={shape} ld={ld}")


# ------------------------------------------------------- size limit
def _sampled_operand_rows(q, rows):
    """Codes and scales of the given operand rows, read from the device
    buffers one 256-row panel at a time (a panel's codes are contiguous in
    the tiled layout)."""
    mnp, kp = oracle.padded_extents(q.mn, q.k)
    panel = 256 * kp // 2
    scales = oracle.untile_scales(host_u8(q.scales), q.mn, q.k)
    codes = np.empty((len(rows), q.k), np.uint8)
    cache = {}
    for i, m in enumerate(rows):
        p = int(m) // 256
        if p not in cache:
            cache[p] = oracle.untile_codes(host_u8(q.codes[p * panel:(p + 1) * panel]), 256, q.k)
        codes[i] = cache[p][int(m) % 256]
    return codes, scales[rows]


def _host_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def test_operands_at_the_size_limit(mx):
    """A 130816 x 16384 source, whose operands in either orientation hold
    1 GiB - 2 MiB of codes (the largest the host accepts is just under
    1 GiB), quantized with random signs and stochastic rounding along both
    axes; sampled operand rows (the first and the last included) bit-exact
    against the oracle, then an Fprop over 130816 rows and a Wgrad over a
    130816-long reduction, sampled output rows within the GEMM bound; the
    dual quantizer's two outputs equal the two single launches byte for
    byte."""
    import torch
    R, C = 130816, 16384
    mnp, kp = oracle.padded_extents(R, C)
    assert mnp * kp // 2 == (1 << 30) - (1 << 21)
    g = torch.Generator(device="cuda")
    g.manual_seed(0x51CE)
    x = torch.randn((R, C), generator=g, device="cuda", dtype=torch.bfloat16)
    w = torch.randn((256, C), generator=g, device="cuda", dtype=torch.bfloat16)
    x2 = torch.randn((R, 64), generator=g, device="cuda", dtype=torch.bfloat16)
    rot, rnd, s = "rand_sign_hadamard", "sr", 0x3C3C
    sa, sb = s, s | (1 << 32)

    # Fprop: A = q(x, axis 1) over all 130816 rows, B = q(w, axis 1)
    qa = mx.quantize(x, 1, rot, rnd, seed=sa)
    qb = mx.quantize(w, 1, rot, rnd, seed=sb)
    y = mx.linear("fprop", qa, qb, "f32")
    _sync()
    rng = np.random.default_rng(9)
    ms = np.unique(np.r_[0, R - 1, rng.choice(R, 30, replace=False)])
    ra = oracle.quantize_ref(_host_bits(x[torch.from_numpy(ms).cuda()]), 1, rotate=rot,
                             rounding=rnd, seed=sa, row_index=ms, total_cols=C)
    codes, scales = _sampled_operand_rows(qa, ms)
    assert np.array_equal(codes, ra.codes) and np.array_equal(scales, ra.scales)
    rb = oracle.quantize_ref(_host_bits(w), 1, rotate=rot, rounding=rnd, seed=sb)
    got = y[torch.from_numpy(ms).cuda()].cpu().numpy()
    err = rel_fro(got, oracle.mx_gemm_ref(ra, rb))
    assert err <= GEMM_TOL, f"fprop at the limit: rel Frobenius {err:.3e}"
    del y

    # Wgrad: A = q(x, axis 0) (16384 operand rows, K = 130816), B = q(x2, axis 0)
    qa0 = mx.quantize(x, 0, rot, rnd, seed=sa)
    qb0 = mx.quantize(x2, 0, rot, rnd, seed=sb)
    dw = mx.linear("wgrad", qa0, qb0, "f32")
    _sync()
    ns = np.unique(np.r_[0, C - 1, rng.choice(C, 20, replace=False)])
    ra0 = oracle.quantize_ref(_host_bits(x[:, torch.from_numpy(ns).cuda()]), 0, rotate=rot,
                              rounding=rnd, seed=sa, col_index=ns, total_cols=C)
    codes0, scales0 = _sampled_operand_rows(qa0, ns)
    assert np.array_equal(codes0, ra0.codes) and np.array_equal(scales0, ra0.scales)
    rb0 = oracle.quantize_ref(_host_bits(x2), 0, rotate=rot, rounding=rnd, seed=sb)
    got0 = dw[torch.from_numpy(ns).cuda()].cpu().numpy()
    err0 = rel_fro(got0, oracle.mx_gemm_ref(ra0, rb0))
    assert err0 <= GEMM_TOL, f"wgrad at the limit: rel Frobenius {err0:.3e}"
    del dw

    # both orientations from one read: byte-identical to the two launches above
    qd1, qd0 = mx.quantize_dual(x, rot, rnd, seed1=sa, seed0=sa)
    _sync()
    for got_q, want_q in ((qd1, qa), (qd0, qa0)):
        assert torch.equal(got_q.codes, want_q.codes) and torch.equal(got_q.scales, want_q.scales)


# ------------------------------------------------------- two-operand launch
@pytest.mark.parametrize("ra,rb,cols", [(37, 300, 160), (1000, 256, 512), (0, 64, 96),
                                        (64, 0, 96), (20000, 5000, 608)])
@pytest.mark.parametrize("rot", ROTS)
@pytest.mark.parametrize("rnd", RNDS)
def test_quantize_pair_matches_two_launches(mx, ra, rb, cols, rot, rnd):
    """One launch over two axis-1 operands that share their column count
    (the Fprop pair X, W): both outputs byte-identical to the two single
    launches, ragged row counts, an empty side, and 7920 tiles (one per
    wave) across the boundary between the operands."""
    rng = np.random.default_rng(ra * 7 + rb + cols)
    xa, xb = to_dev(_rand_bits(rng, (ra, cols))), to_dev(_rand_bits(rng, (rb, cols)))
    sa, sb = 0x77, 0x77 | (1 << 32)
    pa, pb = mx.quantize_pair(xa, xb, rot, rnd, seed_a=sa, seed_b=sb)
    qa = mx.quantize(xa, 1, rot, rnd, seed=sa)
    qb = mx.quantize(xb, 1, rot, rnd, seed=sb)
    _sync()
    for p, q in ((pa, qa), (pb, qb)):
        assert np.array_equal(host_u8(p.codes), host_u8(q.codes))
        assert np.array_equal(host_u8(p.scales), host_u8(q.scales))


def test_quantize_pair_strided_against_oracle(mx):
    """Row-strided sources of different strides, random signs and SR, each
    output against the oracle directly."""
    rng = np.random.default_rng(31)
    a, b = _rand_bits(rng, (300, 224), 2.0), _rand_bits(rng, (77, 224), 0.5)
    ta, tb = to_dev_strided(a, ld=240), to_dev_strided(b, ld=256)
    sa, sb = 0x1D, 0x1D | (1 << 32)
    pa, pb = mx.quantize_pair(ta, tb, "rand_sign_hadamard", "sr", seed_a=sa, seed_b=sb)
    _sync()
    _check_q(pa, oracle.quantize_ref(a, 1, rotate="rand_sign_hadamard", rounding="sr", seed=sa), "A")
    _check_q(pb, oracle.quantize_ref(b, 1, rotate="rand_sign_hadamard", rounding="sr", seed=sb), "B")
