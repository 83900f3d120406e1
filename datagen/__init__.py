"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no part of the quantization method: it only draws random
numbers and rounds them to bfloat16 so that the inputs have the shapes and
value distributions of Llama-3.1-8B linear layers (the workload the pages
train on: 36Kr article "Neue Studie von AMD durchbricht die bestehende
Erkenntnis ...", section "Fehlerdiagnoseexperiment": Llama 3.1-8B, MLPerf C4).
C4 and Llama weights are not available; these tensors stand in for them.

Recipe (every tensor):
  * draw fp32 values from numpy.random.Generator(PCG64(...)), then round each
    value to bfloat16 with round-to-nearest-even on the fp32 bit pattern;
  * activations X ~ N(0, 1), optionally with round(0.001 * cols) outlier
    channels (columns chosen without replacement) multiplied by 50 before the
    bfloat16 rounding;
  * weights W ~ N(0, 0.02^2);
  * output gradients dY = 1e-4 * Student-t(nu = 3).

Streams. The tiny Wgrad workload draws its tensors in the listed order from
one PCG64(data_seed) stream. The larger workloads (up to 1.5e9 elements for
the Llama block at 16384 tokens; one stream would take minutes on one core)
draw each tensor in chunks of CHUNK_ROWS rows: chunk j of the tensor listed
t-th comes from PCG64(SeedSequence([data_seed, t, j])) (the outlier columns
of an activation from PCG64(SeedSequence([data_seed, t, OUTLIER_STREAM]))),
and the chunks are drawn on a thread pool. The values depend only on the
seeds, not on the thread count.

Arrays are returned as numpy uint16 bfloat16 bit patterns, row-major.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "normal_bf16",
    "student_t_bf16",
    "activations_bf16",
    "Workload",
    "LinearShape",
    "LLAMA_BLOCK_LINEARS",
    "BLOCK_INPUT_OF",
    "workload",
    "WORKLOADS",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); NaN stays NaN
    (sign and payload kept, quiet bit set).

    For every non-NaN pattern u (at most 0xFF800000), u + 0x7FFF + bit 16 of
    u stays below 2^32, so the sum is formed in uint32 in place.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                                   # wraps for NaN patterns only
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x.reshape(-1))
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def student_t_bf16(rng: np.random.Generator, shape, nu: float = 3.0,
                   scale: float = 1e-4) -> np.ndarray:
    x = rng.standard_t(nu, size=shape).astype(np.float32)
    x *= np.float32(scale)
    return f32_to_bf16_bits(x)


def activations_bf16(rng: np.random.Generator, shape, outlier_frac: float = 0.0,
                     outlier_gain: float = 50.0) -> np.ndarray:
    """N(0,1) activations; a fraction of channels (columns) scaled by outlier_gain."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * shape[1]))
        if n_out > 0:
            cols = rng.choice(shape[1], size=n_out, replace=False)
            x[:, cols] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(x)


@dataclasses.dataclass(frozen=True)
class LinearShape:
    name: str
    out_features: int
    in_features: int


# Llama-3.1-8B linear layers of one transformer block (d = 4096).
LLAMA_BLOCK_LINEARS: Tuple[LinearShape, ...] = (
    LinearShape("q_proj", 4096, 4096),
    LinearShape("k_proj", 1024, 4096),
    LinearShape("v_proj", 1024, 4096),
    LinearShape("o_proj", 4096, 4096),
    LinearShape("gate_proj", 14336, 4096),
    LinearShape("up_proj", 14336, 4096),
    LinearShape("down_proj", 4096, 14336),
)

# Linears that read another linear's input activation in the block: q, k and
# v project the same normalised hidden state, gate and up the same one after
# the attention. The follower's X is the leader's tensor.
BLOCK_INPUT_OF: Dict[str, str] = {"k_proj": "q_proj", "v_proj": "q_proj", "up_proj": "gate_proj"}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One GEMM of the linear-layer triple with its two source tensors.

    op: "fprop" (Y = X W^T), "dgrad" (dX = dY W) or "wgrad" (dW = dY^T X).
    tensors: name -> (rows, cols, kind) in draw order; kind is one of
      "act" (N(0,1) + outliers), "act_plain" (N(0,1)), "weight" (N(0,0.02^2)),
      "grad" (1e-4 * t_3). A fifth entry, in chunked workloads only, is the
      data seed that tensor is drawn with instead of the workload's (a tensor
      shared with another workload).
    """
    name: str
    op: str
    tokens: int
    out_features: int
    in_features: int
    data_seed: int
    tensors: Tuple[tuple, ...]
    variants: Tuple[Tuple[str, str, str, int], ...]  # (label, rotate, round, seed)
    out_dtype: str = "f32"
    chunk_rows: int = 0      # > 0: chunked multi-stream recipe (module docstring)

    def gemm_mnk(self) -> Tuple[int, int, int]:
        t, o, i = self.tokens, self.out_features, self.in_features
        if self.op == "fprop":
            return t, o, i
        if self.op == "dgrad":
            return t, i, o
        if self.op == "wgrad":
            return o, i, t
        raise ValueError(self.op)

    def flops(self) -> int:
        m, n, k = self.gemm_mnk()
        return 2 * m * n * k


def _values(rng: np.random.Generator, shape, kind: str) -> np.ndarray:
    """fp32 values of one tensor (or row chunk) before the bf16 rounding."""
    if kind in ("act", "act_plain"):
        return rng.standard_normal(size=shape, dtype=np.float32)
    if kind == "weight":
        x = rng.standard_normal(size=shape, dtype=np.float32)
        x *= np.float32(0.02)
        return x
    if kind == "grad":
        x = rng.standard_t(3.0, size=shape).astype(np.float32)
        x *= np.float32(1e-4)
        return x
    raise ValueError(kind)


def _draw(rng: np.random.Generator, rows: int, cols: int, kind: str) -> np.ndarray:
    if kind == "act":
        return activations_bf16(rng, (rows, cols), outlier_frac=0.001)
    if kind == "act_plain":
        return normal_bf16(rng, (rows, cols), 1.0)
    if kind == "weight":
        return normal_bf16(rng, (rows, cols), 0.02)
    if kind == "grad":
        return student_t_bf16(rng, (rows, cols), 3.0, 1e-4)
    raise ValueError(kind)


OUTLIER_STREAM = 1 << 20     # SeedSequence word of an activation's outlier columns
CHUNK_ROWS = 512


def _gen_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_chunked(data_seed: int, t: int, rows: int, cols: int, kind: str,
                  chunk_rows: int, pool: ThreadPoolExecutor) -> np.ndarray:
    """Tensor t of a chunked workload: row chunk j from
    PCG64(SeedSequence([data_seed, t, j])); outlier columns of an activation
    from PCG64(SeedSequence([data_seed, t, OUTLIER_STREAM]))."""
    out = np.empty((rows, cols), np.uint16)
    cols_x = None
    if kind == "act":
        n_out = int(round(0.001 * cols))
        if n_out > 0:
            r = np.random.Generator(np.random.PCG64(
                np.random.SeedSequence([data_seed, t, OUTLIER_STREAM])))
            cols_x = r.choice(cols, size=n_out, replace=False)

    def chunk(j):
        lo, hi = j * chunk_rows, min(rows, (j + 1) * chunk_rows)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([data_seed, t, j])))
        x = _values(rng, (hi - lo, cols), kind)
        if cols_x is not None:
            x[:, cols_x] *= np.float32(50.0)
        out[lo:hi] = f32_to_bf16_bits(x)

    list(pool.map(chunk, range(-(-rows // chunk_rows))))
    return out


def workload_tensors(w: Workload) -> Dict[str, np.ndarray]:
    """Draw the workload's tensors: in their listed order from one PCG64
    stream, or (chunk_rows > 0) chunk by chunk from per-chunk streams."""
    if w.chunk_rows > 0:
        with ThreadPoolExecutor(_gen_threads()) as pool:
            return {spec[0]: _draw_chunked(spec[4] if len(spec) > 4 else w.data_seed, t,
                                           spec[1], spec[2], spec[3], w.chunk_rows, pool)
                    for t, spec in enumerate(w.tensors)}
    if any(len(spec) > 4 for spec in w.tensors):
        raise ValueError("a per-tensor data seed needs a chunked workload")
    rng = np.random.Generator(np.random.PCG64(w.data_seed))
    return {name: _draw(rng, r, c, kind) for (name, r, c, kind) in w.tensors}


DET = ("det_hadamard", "hadamard", "rne", 0)

WORKLOADS: Dict[str, Workload] = {
    # Tiny Wgrad: dY 256x128 and X 256x96, both N(0,1), seed 0, 32-point
    # Hadamard along the 256-token reduction axis, RNE; dW 128x96 fp32.
    "tiny_wgrad": Workload(
        "tiny_wgrad", "wgrad", 256, 128, 96, 0,
        (("dY", 256, 128, "act_plain"), ("X", 256, 96, "act_plain")),
        (DET,), "f32"),
    # Fprop, q_proj: X 8192x4096 (0.1% outlier channels x50), W 4096x4096.
    "fprop_q_proj": Workload(
        "fprop_q_proj", "fprop", 8192, 4096, 4096, 2,
        (("X", 8192, 4096, "act"), ("W", 4096, 4096, "weight")),
        (DET, ("det_hadamard16", "hadamard16", "rne", 0)), "bf16", CHUNK_ROWS),
    # Wgrad, gate/up: dY 8192x14336 (1e-4 t_3), X 8192x4096 N(0,1).
    "wgrad_gate_proj": Workload(
        "wgrad_gate_proj", "wgrad", 8192, 14336, 4096, 3,
        (("dY", 8192, 14336, "grad"), ("X", 8192, 4096, "act_plain")),
        (("no_rotation", "none", "rne", 0), DET), "f32", CHUNK_ROWS),
    # Dgrad, down_proj: dY 8192x4096 (1e-4 t_3), W 4096x14336.
    "dgrad_down_proj": Workload(
        "dgrad_down_proj", "dgrad", 8192, 4096, 14336, 4,
        (("dY", 8192, 4096, "grad"), ("W", 4096, 14336, "weight")),
        (DET, ("det_hadamard_sr7", "hadamard", "sr", 7)), "bf16", CHUNK_ROWS),
}

BLOCK_TOKENS = 16384
BLOCK_VARIANTS = (
    DET,
    ("rand_sign_hadamard11", "rand_sign_hadamard", "rne", 11),
    ("no_rotation_sr11", "none", "sr", 11),
)


def block_workloads(tokens: int = BLOCK_TOKENS) -> List[Workload]:
    """All 21 GEMMs of one Llama-3.1-8B block (7 linears x fprop/dgrad/wgrad).

    Each linear draws its own W (out x in) and dY (T x out) with data seed
    5 * 100 + linear index, in row chunks of CHUNK_ROWS (the chunked recipe
    of the module docstring). X (T x in, with outliers) is the block's input
    activation of that linear: q, k and v share the one drawn with q's seed,
    gate and up the one drawn with gate's (BLOCK_INPUT_OF); o and down draw
    their own. X is tensor 0 of every linear, so a shared X is the same
    array.
    """
    out: List[Workload] = []
    index = {lin.name: li for li, lin in enumerate(LLAMA_BLOCK_LINEARS)}
    for li, lin in enumerate(LLAMA_BLOCK_LINEARS):
        x_seed = 500 + index[BLOCK_INPUT_OF.get(lin.name, lin.name)]
        tensors = (("X", tokens, lin.in_features, "act", x_seed),
                   ("W", lin.out_features, lin.in_features, "weight"),
                   ("dY", tokens, lin.out_features, "grad"))
        for op in ("fprop", "dgrad", "wgrad"):
            out.append(Workload(f"block_{lin.name}_{op}", op, tokens,
                                lin.out_features, lin.in_features, 500 + li,
                                tensors, BLOCK_VARIANTS,
                                "bf16" if op != "wgrad" else "f32", CHUNK_ROWS))
    return out


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def operands_for(w: Workload, tensors: Dict[str, np.ndarray]):
    """The (A source, A axis, B source, B axis) of the workload's GEMM.

    Fprop: A = X (blocks along in, axis 1), B = W (axis 1).
    Dgrad: A = dY (blocks along out, axis 1), B = W (blocks along out, axis 0).
    Wgrad: A = dY (blocks along tokens, axis 0), B = X (axis 0).
    """
    if w.op == "fprop":
        return tensors["X"], 1, tensors["W"], 1
    if w.op == "dgrad":
        return tensors["dY"], 1, tensors["W"], 0
    if w.op == "wgrad":
        return tensors["dY"], 0, tensors["X"], 0
    raise ValueError(w.op)
