"""GPU parity of the grouped GEMM (mx_linear_batched) through the C ABI.

Each output of a grouped launch must equal, bit for bit, what mx_linear
writes for the same pair: every output element sees the same MFMAs in the
same order, only the tiles' placement on the compute units changes. One
entry per case (the last, which comes from the argument block's extra
entries) is also checked against the oracle directly: within 1e-5 relative
Frobenius error and the per-element bound of the other GEMM tests.

The cases cover the launcher's paths on a 256-compute-unit MI355X with the
entries' tile rows stacked into one grid (256 x 256 tiles): half tiles
only, whole tiles only, whole tiles then half tiles, ragged edges in M, N
and K, an fp32 and a bf16 output, strided outputs, and K = 0.
"""
import numpy as np
import pytest

import oracle
from datagen import f32_to_bf16_bits
from gpu_util import rel_fro, to_dev

pytestmark = pytest.mark.gpu

GEMM_TOL = 1e-5

# (op, M, N, K, count): tiles per entry, tiles of the grouped launch
CASES = [
    ("fprop", 300, 200, 256, 2),     # 2 tiles each, 4: all as 8 half tiles
    ("wgrad", 1024, 4096, 512, 2),   # k/v-projection Wgrad shape: 64 each, 128 -> 256 half tiles
    ("dgrad", 600, 520, 384, 3),     # 9 each, 27: half tiles, ragged M, N
    ("fprop", 2048, 2048, 256, 4),   # 64 each, 256: one round of whole tiles
    ("fprop", 4096, 2560, 128, 2),   # 160 each, 320: 256 whole, then 64 as 128 half tiles
    ("wgrad", 384, 288, 224, 4),     # 2 each, 8: half tiles; K tail (224)
]


def _rand_bits(rng, shape, scale=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _sources(op, M, N, K, rng):
    """Source tensors (A, B) of one entry in the shapes the op quantizes."""
    if op == "fprop":      # X [T=M, in=K], W [out=N, in=K]
        return _rand_bits(rng, (M, K)), _rand_bits(rng, (N, K), 0.02)
    if op == "dgrad":      # dY [T=M, out=K], W [out=K, in=N]
        return _rand_bits(rng, (M, K), 1e-2), _rand_bits(rng, (K, N), 0.02)
    return _rand_bits(rng, (K, M), 1e-2), _rand_bits(rng, (K, N))   # dY [T=K, out=M], X [T=K, in=N]


@pytest.mark.parametrize("op,M,N,K,count", CASES)
def test_batched_equals_single_and_oracle(mx, op, M, N, K, count):
    import torch
    print(f"[batched] {op} {M}x{N}x{K} x{count}", flush=True)
    rng = np.random.default_rng(M + 3 * N + 7 * K + count)
    ax_a, ax_b = mx.OP_AXES[op]
    srcs, qa, qb = [], [], []
    for i in range(count):
        a, b = _sources(op, M, N, K, rng)
        srcs.append((a, b))
        seed = 5 + i
        qa.append(mx.quantize(to_dev(a), ax_a, "hadamard", "rne", seed=seed))
        qb.append(mx.quantize(to_dev(b), ax_b, "hadamard", "rne", seed=seed | (1 << 32)))
    for dt in ("f32", "bf16"):
        got = mx.linear_batched(op, qa, qb, dt)
        ref = [mx.linear(op, qa[i], qb[i], dt) for i in range(count)]
        torch.cuda.synchronize()
        for i in range(count):
            assert torch.equal(got[i], ref[i]), f"{op} {dt} entry {i}: grouped != single launch"
    # the last entry against the oracle
    a, b = srcs[-1]
    c32 = got_f32 = mx.linear_batched(op, qa, qb, "f32")[-1].cpu().numpy()
    C_ref, ra, rb = oracle.linear_ref(op, a, b, rotate="hadamard", rounding="rne", seed=5 + count - 1)
    err = rel_fro(c32, C_ref)
    assert err <= GEMM_TOL, f"{op}: rel Frobenius {err:.3e}"
    da = np.abs(oracle.dequantize_ref(ra.codes, ra.scales))
    db = np.abs(oracle.dequantize_ref(rb.codes, rb.scales))
    bound = (K / 32 + 4) * 2.0 ** -23 * (da @ db.T)
    over = np.count_nonzero(np.abs(got_f32.astype(np.float64) - C_ref) > bound)
    assert over == 0, f"{op}: {over} elements beyond the per-element bound"


def test_batched_strided_outputs_and_empty_k(mx):
    """Outputs as column slices of wider buffers (one shared leading
    dimension): equal to the contiguous results, padding untouched; K = 0
    writes zeros to every entry."""
    import torch
    rng = np.random.default_rng(77)
    M, N, K = 520, 300, 256
    qa, qb = [], []
    for i in range(3):
        a, b = _sources("fprop", M, N, K, rng)
        qa.append(mx.quantize(to_dev(a), 1, "hadamard", "rne", seed=i))
        qb.append(mx.quantize(to_dev(b), 1, "hadamard", "rne", seed=i | (1 << 32)))
    for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        ref = mx.linear_batched("fprop", qa, qb, dt)
        bigs = [torch.full((M, N + 5), 3.0, dtype=tdt, device="cuda") for _ in range(3)]
        mx.linear_batched("fprop", qa, qb, dt, outs=[g[:, :N] for g in bigs])
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(bigs[i][:, :N], ref[i]), f"{dt} entry {i}: strided output differs"
            assert torch.all(bigs[i][:, N:] == 3.0), f"{dt} entry {i}: pad columns written"
    za = [mx.quantize(to_dev(np.zeros((64, 0), np.uint16)), 1, "hadamard", "rne", seed=0)
          for _ in range(2)]
    zb = [mx.quantize(to_dev(np.zeros((96, 0), np.uint16)), 1, "hadamard", "rne", seed=1 << 32)
          for _ in range(2)]
    outs = [torch.full((64, 96), 9.0, dtype=torch.float32, device="cuda") for _ in range(2)]
    mx.linear_batched("fprop", za, zb, "f32", outs=outs)
    torch.cuda.synchronize()
    assert all(torch.all(o == 0.0) for o in outs), "K = 0 must write zeros"


def test_batched_entries_with_different_quantizations(mx):
    """Each entry keeps its own operands' quantization: entries quantized
    with different rotations and roundings (each pair consistent) give the
    single launches' outputs bit for bit, and the SR entry matches the
    oracle."""
    import torch
    rng = np.random.default_rng(515)
    M, N, K = 384, 320, 256
    variants = [("hadamard", "rne", 3), ("none", "sr", 9), ("rand_sign_hadamard", "rne", 11),
                ("hadamard16", "sr", 4)]
    qa, qb, srcs = [], [], []
    for rot, rnd, seed in variants:
        a, b = _sources("wgrad", M, N, K, rng)
        srcs.append((a, b))
        qa.append(mx.quantize(to_dev(a), 0, rot, rnd, seed=seed))
        qb.append(mx.quantize(to_dev(b), 0, rot, rnd, seed=seed | (1 << 32)))
    got = mx.linear_batched("wgrad", qa, qb, "f32")
    torch.cuda.synchronize()
    for i in range(len(variants)):
        ref = mx.linear("wgrad", qa[i], qb[i], "f32")
        torch.cuda.synchronize()
        assert torch.equal(got[i], ref), f"entry {i} {variants[i]}: grouped != single launch"
    a, b = srcs[1]
    C_ref, _, _ = oracle.linear_ref("wgrad", a, b, rotate="none", rounding="sr", seed=9)
    err = rel_fro(got[1].cpu().numpy(), C_ref)
    assert err <= GEMM_TOL, f"SR entry: rel Frobenius {err:.3e}"
