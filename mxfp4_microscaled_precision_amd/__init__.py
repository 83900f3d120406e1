"""MXFP4 linear layers on MI355X (gfx950): Python binding of libmxfp4.so.

The binding only marshals arguments: PyTorch provides device memory and the
current HIP stream, and every step of the computation runs in the library's
HIP kernels. There is no CPU fallback; if the library is missing, loading it
raises.

    q_x = quantize(x_bf16, axis=1, rotate="hadamard", round="rne", seed=0)
    q_w = quantize(w_bf16, axis=1, rotate="hadamard", seed=1 << 32)
    y = linear("fprop", q_x, q_w, out_dtype="bf16")

The three GEMMs and their operand axes (36Kr article "Neue Studie von AMD
durchbricht die bestehende Erkenntnis ...", section "Fehlerdiagnoseexperiment"):
    fprop: A = X  [T, in]  axis 1, B = W [out, in] axis 1 -> Y  [T, out]
    dgrad: A = dY [T, out] axis 1, B = W [out, in] axis 0 -> dX [T, in]
    wgrad: A = dY [T, out] axis 0, B = X [T, in]   axis 0 -> dW [out, in]
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "LIB_PATH", "MxError", "QTensorDesc", "QTensor", "load_library", "library_symbols",
    "status_string", "version", "last_hip_error", "quantize_sizes", "quantize", "quantize_dual",
    "quantize_pair",
    "quantize_fp8_sizes", "quantize_fp8", "linear", "linear_batched", "dequantize",
    "ROTATE", "ROUND", "FORMATS", "OPS", "OUT_DTYPES", "OP_AXES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp4.so")

ROTATE = {"none": 0, "hadamard": 1, "rand_sign_hadamard": 2, "hadamard16": 3}
ROUND = {"rne": 0, "sr": 1}
FORMATS = {"fp4_e2m1": 0, "fp8_e4m3": 1}
OPS = {"fprop": 0, "dgrad": 1, "wgrad": 2}
OUT_DTYPES = {"f32": 0, "bf16": 1}
# (A axis, B axis) each op needs
OP_AXES = {"fprop": (1, 1), "dgrad": (1, 0), "wgrad": (0, 0)}

MX_OK = 0


class MxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_string(status)} ({status})"
        if status == -7:
            msg += f" [{load_library().mx_last_hip_error().decode()}]"
        super().__init__(msg)


class QTensorDesc(ctypes.Structure):
    """Mirror of struct mx_qtensor in include/mxfp4.h."""
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("axis", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("rotate", ctypes.c_int32),
        ("round", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
        ("format", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None

_SIGNATURES = {
    "mx_quantize_sizes": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t),
                                         ctypes.POINTER(ctypes.c_size_t)]),
    "mx_quantize_fp8_sizes": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t),
                                             ctypes.POINTER(ctypes.c_size_t)]),
    "mx_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64,
                                   ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.POINTER(QTensorDesc), ctypes.c_void_p]),
    "mx_quantize_dual": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.POINTER(QTensorDesc),
                                        ctypes.POINTER(QTensorDesc), ctypes.c_void_p]),
    "mx_quantize_pair": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.POINTER(QTensorDesc),
                                        ctypes.POINTER(QTensorDesc), ctypes.c_void_p]),
    "mx_quantize_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.POINTER(QTensorDesc),
                                       ctypes.c_void_p]),
    "mx_linear": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(QTensorDesc),
                                 ctypes.POINTER(QTensorDesc), ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_int32, ctypes.c_void_p]),
    "mx_linear_batched": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32,
                                         ctypes.POINTER(QTensorDesc), ctypes.POINTER(QTensorDesc),
                                         ctypes.POINTER(ctypes.c_void_p), ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_void_p]),
    "mx_dequantize": (ctypes.c_int, [ctypes.POINTER(QTensorDesc), ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_void_p]),
    "mx_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "mx_version": (ctypes.c_char_p, []),
    "mx_last_hip_error": (ctypes.c_char_p, []),
}


def library_symbols() -> Tuple[str, ...]:
    return tuple(_SIGNATURES)


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as fh:
            return sorted({ln.split()[-1] for ln in fh if "libamdhip64" in ln})
    except OSError:
        return []


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmxfp4.so (built by mxfp4_microscaled_precision_amd.build).

    torch is imported first: PyTorch-ROCm ships its own HIP runtime under the
    same soname, and the library must bind to that one so that torch's streams
    and allocations are valid for its launches. Two HIP runtimes in one process
    is refused with an error.
    """
    global _lib
    if _lib is not None and path is None:
        return _lib
    import torch  # noqa: F401  (binds libamdhip64 to torch's runtime first)
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m mxfp4_microscaled_precision_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(p)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError("two HIP runtimes are loaded in this process (%s); load torch "
                           "before libmxfp4.so" % ", ".join(runtimes))
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mx_status_string(int(status)).decode()


def version() -> str:
    return load_library().mx_version().decode()


def last_hip_error() -> str:
    return load_library().mx_last_hip_error().decode()


def _check(status: int, where: str) -> None:
    if status != MX_OK:
        raise MxError(status, where)


def quantize_sizes(rows: int, cols: int, axis: int, block: int = 32) -> Tuple[int, int]:
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().mx_quantize_sizes(rows, cols, axis, block, ctypes.byref(cb),
                                            ctypes.byref(sb)), "mx_quantize_sizes")
    return cb.value, sb.value


def quantize_fp8_sizes(rows: int, cols: int, axis: int, block: int = 32) -> Tuple[int, int]:
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().mx_quantize_fp8_sizes(rows, cols, axis, block, ctypes.byref(cb),
                                                ctypes.byref(sb)), "mx_quantize_fp8_sizes")
    return cb.value, sb.value


def _stream_handle(device, stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


class QTensor:
    """A quantized operand: flat uint8 buffers holding the tiled codes and
    scales (layout in include/mxfp4.h, struct mx_qtensor) plus the C
    descriptor that points at them."""

    def __init__(self, codes, scales, desc: QTensorDesc):
        self.codes = codes
        self.scales = scales
        self.desc = desc

    @property
    def axis(self) -> int:
        return self.desc.axis

    @property
    def source_shape(self) -> Tuple[int, int]:
        return (self.desc.rows, self.desc.cols)

    @property
    def format(self) -> str:
        return {v: k for k, v in FORMATS.items()}[self.desc.format]

    @property
    def mn(self) -> int:
        return self.desc.rows if self.desc.axis == 1 else self.desc.cols

    @property
    def k(self) -> int:
        return self.desc.cols if self.desc.axis == 1 else self.desc.rows


def _source_extents(x) -> Tuple[int, int, int]:
    """(rows, cols, ld) of a 2-D bf16 CUDA source; raises for anything else."""
    import torch
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    if not x.is_cuda:
        raise ValueError("x must be a CUDA (HIP) tensor; there is no CPU path")
    if x.numel() > 0 and x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else max(cols, 8 * ((cols + 7) // 8))
    return rows, cols, ld


def quantize(x, axis: int, rotate: str = "hadamard", round: str = "rne", seed: int = 0,
             codes=None, scales=None, stream=None) -> QTensor:
    """Rotate + quantize a 2-D bf16 CUDA tensor along `axis` (see mx_quantize).

    x may be a row-strided view (stride(1) == 1). codes / scales may be
    preallocated uint8 tensors of at least the sizes quantize_sizes returns.
    """
    import torch
    lib = load_library()
    rows, cols, ld = _source_extents(x)
    cb, sb = quantize_sizes(rows, cols, axis)
    if codes is None:
        codes = torch.empty((cb,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((sb,), dtype=torch.uint8, device=x.device)
    if codes.numel() < cb or scales.numel() < sb:
        raise ValueError("codes / scales buffers too small")
    desc = QTensorDesc()
    st = lib.mx_quantize(x.data_ptr() if x.numel() else None, rows, cols, ld, axis, 32,
                         ROTATE[rotate], ROUND[round], seed & 0xFFFFFFFFFFFFFFFF,
                         codes.data_ptr() if codes.numel() else None,
                         scales.data_ptr() if scales.numel() else None,
                         ctypes.byref(desc), _stream_handle(x.device, stream))
    _check(st, "mx_quantize")
    return QTensor(codes, scales, desc)


def quantize_pair(xa, xb, rotate: str = "hadamard", round: str = "rne", seed_a: int = 0,
                  seed_b: int = 0, stream=None) -> Tuple[QTensor, QTensor]:
    """Axis-1 quantizations of two 2-D bf16 CUDA tensors with the same column
    count in one launch (see mx_quantize_pair): returns (A operand, B operand),
    byte-identical to quantize(xa, 1, ...) and quantize(xb, 1, ...)."""
    import torch
    lib = load_library()
    ra, cols, lda = _source_extents(xa)
    rb, cols_b, ldb = _source_extents(xb)
    if cols != cols_b:
        raise ValueError("quantize_pair needs sources with the same column count")
    out = []
    for rows in (ra, rb):
        cb, sb = quantize_sizes(rows, cols, 1)
        out.append((torch.empty((cb,), dtype=torch.uint8, device=xa.device),
                    torch.empty((sb,), dtype=torch.uint8, device=xa.device)))
    (ca, sa), (cb_, sb_) = out
    da, db = QTensorDesc(), QTensorDesc()
    ptr = lambda t: t.data_ptr() if t.numel() else None  # noqa: E731
    st = lib.mx_quantize_pair(ptr(xa), ra, lda, ptr(xb), rb, ldb, cols, 32, ROTATE[rotate],
                              ROUND[round], seed_a & 0xFFFFFFFFFFFFFFFF,
                              seed_b & 0xFFFFFFFFFFFFFFFF, ptr(ca), ptr(sa), ptr(cb_), ptr(sb_),
                              ctypes.byref(da), ctypes.byref(db), _stream_handle(xa.device, stream))
    _check(st, "mx_quantize_pair")
    return QTensor(ca, sa, da), QTensor(cb_, sb_, db)


def quantize_dual(x, rotate: str = "hadamard", round: str = "rne", seed1: int = 0,
                  seed0: int = 0, stream=None) -> Tuple[QTensor, QTensor]:
    """Both orientations of a 2-D bf16 CUDA tensor from one read of it (see
    mx_quantize_dual): returns (axis-1 operand, axis-0 operand)."""
    import torch
    lib = load_library()
    rows, cols, ld = _source_extents(x)
    out = []
    for axis in (1, 0):
        cb, sb = quantize_sizes(rows, cols, axis)
        out.append((torch.empty((cb,), dtype=torch.uint8, device=x.device),
                    torch.empty((sb,), dtype=torch.uint8, device=x.device)))
    (c1, s1), (c0, s0) = out
    d1, d0 = QTensorDesc(), QTensorDesc()
    ptr = lambda t: t.data_ptr() if t.numel() else None  # noqa: E731
    st = lib.mx_quantize_dual(ptr(x), rows, cols, ld, 32, ROTATE[rotate], ROUND[round],
                              seed1 & 0xFFFFFFFFFFFFFFFF, seed0 & 0xFFFFFFFFFFFFFFFF,
                              ptr(c1), ptr(s1), ptr(c0), ptr(s0), ctypes.byref(d1),
                              ctypes.byref(d0), _stream_handle(x.device, stream))
    _check(st, "mx_quantize_dual")
    return QTensor(c1, s1, d1), QTensor(c0, s0, d0)


def quantize_fp8(x, axis: int, rotate: str = "hadamard", seed: int = 0, codes=None,
                 scales=None, stream=None) -> QTensor:
    """Rotate + quantize into MXFP8 with E4M3 elements, the FP8 comparator
    (see mx_quantize_fp8; nearest rounding only). Arguments as for quantize."""
    import torch
    lib = load_library()
    rows, cols, ld = _source_extents(x)
    cb, sb = quantize_fp8_sizes(rows, cols, axis)
    if codes is None:
        codes = torch.empty((cb,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((sb,), dtype=torch.uint8, device=x.device)
    if codes.numel() < cb or scales.numel() < sb:
        raise ValueError("codes / scales buffers too small")
    desc = QTensorDesc()
    st = lib.mx_quantize_fp8(x.data_ptr() if x.numel() else None, rows, cols, ld, axis, 32,
                             ROTATE[rotate], seed & 0xFFFFFFFFFFFFFFFF,
                             codes.data_ptr() if codes.numel() else None,
                             scales.data_ptr() if scales.numel() else None,
                             ctypes.byref(desc), _stream_handle(x.device, stream))
    _check(st, "mx_quantize_fp8")
    return QTensor(codes, scales, desc)


def linear(op: str, A: QTensor, B: QTensor, out_dtype: str = "f32", out=None,
           stream=None):
    """One GEMM of the triple (see mx_linear); returns C [M, N] (fp32 or bf16).
    Two MXFP8 operands (quantize_fp8) run the E4M3 comparator GEMM."""
    import torch
    lib = load_library()
    M, N = A.mn, B.mn
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=A.codes.device)
    if out.dtype != dt or out.dim() != 2 or tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong dtype or shape")
    if out.numel() and out.stride(1) != 1:
        raise ValueError("out must have unit column stride")
    ldc = out.stride(0) if M > 1 else max(N, 4)
    st = lib.mx_linear(OPS[op], ctypes.byref(A.desc), ctypes.byref(B.desc),
                       out.data_ptr() if out.numel() else None, ldc, OUT_DTYPES[out_dtype],
                       _stream_handle(A.codes.device, stream))
    _check(st, "mx_linear")
    return out


def linear_batched(op: str, As, Bs, out_dtype: str = "f32", outs=None, stream=None):
    """Several GEMMs of one op and one shape in one launch (see
    mx_linear_batched): C[i] = linear(op, As[i], Bs[i]); returns the list of
    C [M, N] (fp32 or bf16), bitwise identical to separate linear calls."""
    import torch
    lib = load_library()
    n = len(As)
    if len(Bs) != n:
        raise ValueError("As and Bs differ in length")
    M, N = As[0].mn, Bs[0].mn
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    if outs is None:
        outs = [torch.empty((M, N), dtype=dt, device=As[0].codes.device) for _ in range(n)]
    if len(outs) != n:
        raise ValueError("outs differs in length")
    lds = set()
    for o in outs:
        if o.dtype != dt or o.dim() != 2 or tuple(o.shape) != (M, N):
            raise ValueError("an output has the wrong dtype or shape")
        if o.numel() and o.stride(1) != 1:
            raise ValueError("outputs must have unit column stride")
        lds.add(o.stride(0) if M > 1 else max(N, 4))
    if len(lds) != 1:
        raise ValueError("outputs must share one leading dimension")
    da = (QTensorDesc * n)(*[q.desc for q in As])
    db = (QTensorDesc * n)(*[q.desc for q in Bs])
    cs = (ctypes.c_void_p * n)(*[o.data_ptr() if o.numel() else None for o in outs])
    st = lib.mx_linear_batched(OPS[op], n, da, db, cs, lds.pop(), OUT_DTYPES[out_dtype],
                               _stream_handle(As[0].codes.device, stream))
    _check(st, "mx_linear_batched")
    return outs


def dequantize(q: QTensor, out=None, stream=None):
    """fp32 values of a quantized operand in its source's shape [rows, cols]
    (see mx_dequantize): sign * E2M1 (or E4M3) value * 2^(scale - 127)."""
    import torch
    lib = load_library()
    rows, cols = q.source_shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=q.codes.device)
    if out.dtype != torch.float32 or out.dim() != 2 or tuple(out.shape) != (rows, cols):
        raise ValueError("out must be a float32 tensor of the source's shape")
    if out.numel() and out.stride(1) != 1:
        raise ValueError("out must have unit column stride")
    ld = out.stride(0) if rows > 1 else max(cols, 1)
    st = lib.mx_dequantize(ctypes.byref(q.desc), out.data_ptr() if out.numel() else None, ld,
                           _stream_handle(q.codes.device, stream))
    _check(st, "mx_dequantize")
    return out
