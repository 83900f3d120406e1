"""C-ABI checks that need no GPU: every declared symbol is exported, and every
invalid argument is rejected on the host before any HIP call."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (the library must bind to torch's HIP runtime)

import mxfp4_microscaled_precision_amd as mx

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mxfp4.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(mx.library_symbols())


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mx.LIB_PATH)
    assert len(mx._hip_runtimes_mapped()) <= 1
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert mx.version().startswith("mxfp4-gfx950")
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert mx.status_string(s).startswith("MX_")
    assert mx.last_hip_error() == "hipSuccess"
    assert "unknown" in mx.status_string(42)


def test_quantize_sizes():
    assert mx.quantize_sizes(8192, 4096, 1) == (8192 * 4096 // 2, 8192 * 4096 // 32)
    # tiled layout: MN padded to 256, K to 128
    assert mx.quantize_sizes(256, 96, 0) == (256 * 256 // 2, 256 * 256 // 32)
    assert mx.quantize_sizes(37, 160, 1) == (256 * 256 // 2, 256 * 256 // 32)
    assert mx.quantize_sizes(160, 37, 0) == (256 * 256 // 2, 256 * 256 // 32)
    assert mx.quantize_sizes(300, 128, 1) == (512 * 128 // 2, 512 * 128 // 32)
    assert mx.quantize_sizes(0, 0, 1) == (0, 0)
    assert mx.quantize_sizes(0, 64, 1) == (0, 0)
    for args, code in [((64, 48, 1), -2), ((48, 64, 0), -2), ((64, 64, 2), -4),
                       ((-1, 64, 1), -2)]:
        with pytest.raises(mx.MxError) as ei:
            mx.quantize_sizes(*args)
        assert ei.value.status == code
    with pytest.raises(mx.MxError) as ei:
        mx.quantize_sizes(64, 64, 1, block=16)
    assert ei.value.status == -4


def test_quantize_fp8_sizes():
    # one code byte per element, scales as for MXFP4
    assert mx.quantize_fp8_sizes(8192, 4096, 1) == (8192 * 4096, 8192 * 4096 // 32)
    assert mx.quantize_fp8_sizes(37, 160, 1) == (256 * 256, 256 * 256 // 32)
    assert mx.quantize_fp8_sizes(160, 37, 0) == (256 * 256, 256 * 256 // 32)
    assert mx.quantize_fp8_sizes(0, 64, 1) == (0, 0)
    with pytest.raises(mx.MxError) as ei:
        mx.quantize_fp8_sizes(64, 48, 1)
    assert ei.value.status == -2


def _q8(lib, x, rows, cols, ld, axis=1, block=32, rot=1, codes=4096, scales=4096):
    desc = mx.QTensorDesc()
    return lib.mx_quantize_fp8(x, rows, cols, ld, axis, block, rot, 0, codes, scales,
                               ctypes.byref(desc), None)


def test_quantize_fp8_rejects_before_launch():
    lib = mx.load_library()
    P = 4096
    assert _q8(lib, P, 64, 64, 64, block=16) == -4
    assert _q8(lib, P, 64, 64, 64, axis=2) == -4
    assert _q8(lib, P, 64, 64, 64, rot=4) == -4
    assert _q8(lib, P, 64, 48, 64) == -2
    assert _q8(lib, P, 64, 64, 68) == -3
    assert _q8(lib, P + 2, 64, 64, 64) == -3
    assert _q8(lib, P, 64, 64, 64, codes=P + 8) == -3
    # 1 GiB of E4M3 codes is reached at half the FP4 element count
    assert _q8(lib, P, 1 << 16, 1 << 14, 1 << 14) == -6
    assert _q(lib, P, 1 << 16, 1 << 14, 1 << 14, codes=None) == -1   # FP4: within the limit
    assert _q8(lib, None, 64, 64, 64) == -1


def test_quantize_fp8_empty_fills_descriptor():
    lib = mx.load_library()
    desc = mx.QTensorDesc()
    assert lib.mx_quantize_fp8(None, 0, 64, 64, 1, 32, 3, 9, None, None, ctypes.byref(desc),
                               None) == 0
    assert (desc.format, desc.round, desc.rotate, desc.seed) == (1, 0, 3, 9)


def _q(lib, x, rows, cols, ld, axis=1, block=32, rot=1, rnd=0, codes=16, scales=16):
    desc = mx.QTensorDesc()
    return lib.mx_quantize(x, rows, cols, ld, axis, block, rot, rnd, 0, codes, scales,
                           ctypes.byref(desc), None)


def test_quantize_rejects_before_launch():
    """Host pointers are never dereferenced: validation fails before any HIP call."""
    lib = mx.load_library()
    P = 4096  # a fake, 16-byte-aligned address; never touched
    assert _q(lib, P, 64, 64, 64, block=16) == -4
    assert _q(lib, P, 64, 64, 64, axis=2) == -4
    assert _q(lib, P, 64, 64, 64, rot=4) == -4
    assert _q(lib, P, 64, 64, 64, rnd=2) == -4
    assert _q(lib, P, 64, 48, 64, axis=1) == -2          # cols % 32
    assert _q(lib, P, 48, 64, 64, axis=0) == -2          # rows % 32
    assert _q(lib, P, 64, 64, 32) == -2                  # ld < cols
    assert _q(lib, P, 64, 64, 68) == -3                  # ld % 8 (axis 1)
    assert _q(lib, P + 2, 64, 64, 64) == -3              # x misaligned (axis 1)
    assert _q(lib, P + 1, 64, 64, 64, axis=0) == -3      # x odd address (axis 0)
    assert _q(lib, P, 64, 64, 64, codes=P + 4) == -3     # codes misaligned
    assert _q(lib, P, 64, 64, 64, scales=P + 2) == -3    # scales misaligned
    assert _q(lib, P, 1 << 17, 1 << 14, 1 << 14) == -6   # codes of 1 GiB: unsupported
    assert _q(lib, None, 64, 64, 64) == -1
    assert _q(lib, P, 64, 64, 64, codes=None) == -1
    assert _q(lib, P, 64, 64, 64, scales=None) == -1
    assert _q(lib, P, -1, 64, 64) == -2


def test_quantize_rejects_extents_that_overflow():
    """Extents whose padded product (or source span) would overflow int64
    are refused on the host; they used to wrap around the 1 GiB check and
    reach a launch."""
    lib = mx.load_library()
    P = 4096
    assert _q(lib, P, 1 << 36, 1 << 36, 1 << 36) == -6            # product wraps to 0
    assert _q(lib, P, 1 << 36, 1 << 36, 1 << 36, axis=0) == -6
    assert _q(lib, P, (1 << 31) + 32, 64, 64) == -6               # an extent above 2^31
    assert _q(lib, P, 1 << 20, 64, 1 << 60) == -6                 # rows * ld * 2 above 2^62
    assert _q(lib, P, 1 << 20, 64, 1 << 60, axis=0) == -6
    assert _q8(lib, P, 1 << 36, 1 << 36, 1 << 36) == -6
    assert _qd(lib, P, 1 << 36, 1 << 36, 1 << 36) == -6
    assert _qd(lib, P, 1 << 20, 64, 1 << 60) == -6
    assert _qp(lib, P, 1 << 20, 1 << 60, P, 64, 64, 64) == -6
    assert _qp(lib, P, 64, 64, P, 1 << 36, 64, 64) == -6                 # B rows above 2^31
    for sizes in (mx.quantize_sizes, mx.quantize_fp8_sizes):
        with pytest.raises(mx.MxError) as ei:
            sizes(1 << 36, 1 << 36, 1)
        assert ei.value.status == -6
        assert sizes(1 << 40, 0, 1) == (0, 0)                     # empty stays valid
    # the span limit's edge (2^20 rows of 2^41 bf16 elements = 2^62 bytes): the
    # largest ld passes it and stops at the next check, a misaligned source
    assert _q(lib, P + 2, 1 << 20, 64, 1 << 41) == -3
    assert _q(lib, P + 2, 1 << 20, 64, (1 << 41) + 8) == -6


def _qp(lib, xa, ra, lda, xb, rb, ldb, cols, block=32, rot=1, rnd=0, ca=16, sa=16, cb=4096,
        sb=4096, da=None, db=None):
    return lib.mx_quantize_pair(xa, ra, lda, xb, rb, ldb, cols, block, rot, rnd, 5, 6, ca, sa,
                                cb, sb, da, db, None)


def test_quantize_pair_rejects_before_launch():
    """Both operands are validated as mx_quantize would, A first, before any HIP call."""
    lib = mx.load_library()
    P = 4096
    assert _qp(lib, P, 64, 64, P, 64, 64, 64, block=16) == -4
    assert _qp(lib, P, 64, 64, P, 64, 64, 64, rot=7) == -4
    assert _qp(lib, P, 64, 64, P, 64, 64, 48) == -2            # K % 32
    assert _qp(lib, P, 64, 32, P, 64, 64, 64) == -2            # lda < cols
    assert _qp(lib, P, 64, 64, P, 64, 32, 64) == -2            # ldb < cols
    assert _qp(lib, P + 2, 64, 64, P, 64, 64, 64) == -3        # A misaligned
    assert _qp(lib, P, 64, 64, P + 2, 64, 64, 64) == -3        # B misaligned
    assert _qp(lib, P, 64, 64, P, 64, 68, 64) == -3            # ldb % 8
    assert _qp(lib, P, 64, 64, None, 64, 64, 64) == -1
    assert _qp(lib, P, 64, 64, P, 64, 64, 64, cb=None) == -1
    assert _qp(lib, P, 64, 1 << 14, P, 1 << 17, 1 << 14, 1 << 14) == -6   # B codes of 1 GiB


def test_quantize_pair_empty_fills_both_descriptors():
    lib = mx.load_library()
    da, db = mx.QTensorDesc(), mx.QTensorDesc()
    assert _qp(lib, None, 0, 64, None, 0, 64, 64, rot=2, rnd=1, ca=None, sa=None, cb=None,
               sb=None, da=ctypes.byref(da), db=ctypes.byref(db)) == 0
    assert (da.rows, da.cols, da.axis, da.rotate, da.round, da.seed) == (0, 64, 1, 2, 1, 5)
    assert (db.rows, db.cols, db.axis, db.rotate, db.round, db.seed) == (0, 64, 1, 2, 1, 6)


def test_quantize_empty_is_a_noop_and_fills_descriptor():
    lib = mx.load_library()
    desc = mx.QTensorDesc()
    assert lib.mx_quantize(None, 0, 64, 64, 1, 32, 2, 1, 77, None, None, ctypes.byref(desc),
                           None) == 0
    assert (desc.rows, desc.cols, desc.axis, desc.rotate, desc.round, desc.seed) == (0, 64, 1, 2, 1, 77)


def _desc(rows, cols, axis, rot=1, rnd=0, seed=0, codes=4096, scales=4096, fmt=0):
    d = mx.QTensorDesc()
    d.codes, d.scales = codes, scales
    d.rows, d.cols, d.axis, d.block, d.rotate, d.round, d.seed = rows, cols, axis, 32, rot, rnd, seed
    d.format = fmt
    return d


def _lin(lib, op, A, B, C=4096, ldc=None, out=0):
    ldc = ldc if ldc is not None else (B.rows if B.axis == 1 else B.cols)
    return lib.mx_linear(op, ctypes.byref(A), ctypes.byref(B), C, ldc, out, None)


def _qd(lib, x, rows, cols, ld, block=32, rot=1, rnd=0, c1=None, s1=None, c0=None, s0=None):
    P = 4096
    d1, d0 = mx.QTensorDesc(), mx.QTensorDesc()
    return lib.mx_quantize_dual(x, rows, cols, ld, block, rot, rnd, 0, 0,
                                P if c1 is None else c1, P if s1 is None else s1,
                                P if c0 is None else c0, P if s0 is None else s0,
                                ctypes.byref(d1), ctypes.byref(d0), None)


def test_quantize_dual_rejects_before_launch():
    """Validation of mx_quantize_dual fails before any HIP call."""
    lib = mx.load_library()
    P = 4096
    assert _qd(lib, P, 64, 64, 64, block=16) == -4
    assert _qd(lib, P, 64, 64, 64, rot=4) == -4
    assert _qd(lib, P, 64, 64, 64, rnd=2) == -4
    assert _qd(lib, P, 64, 48, 64) == -2                 # cols % 32
    assert _qd(lib, P, 48, 64, 64) == -2                 # rows % 32
    assert _qd(lib, P, 64, 64, 32) == -2                 # ld < cols
    assert _qd(lib, P, 64, 64, 68) == -3                 # ld % 8
    assert _qd(lib, P + 2, 64, 64, 64) == -3             # x misaligned
    assert _qd(lib, P, 64, 64, 64, c0=P + 4) == -3       # axis-0 codes misaligned
    assert _qd(lib, P, 64, 64, 64, s1=P + 2) == -3       # axis-1 scales misaligned
    assert _qd(lib, None, 64, 64, 64) == -1
    assert _qd(lib, P, 64, 64, 64, c1=0) == -1
    assert _qd(lib, P, 1 << 17, 1 << 14, 1 << 14) == -6  # codes of 1 GiB


def test_quantize_dual_empty_fills_both_descriptors():
    lib = mx.load_library()
    d1, d0 = mx.QTensorDesc(), mx.QTensorDesc()
    st = lib.mx_quantize_dual(None, 0, 64, 64, 32, 3, 1, 5, 6, None, None, None, None,
                              ctypes.byref(d1), ctypes.byref(d0), None)
    assert st == 0
    assert (d1.axis, d1.rotate, d1.round, d1.seed, d1.cols) == (1, 3, 1, 5, 64)
    assert (d0.axis, d0.rotate, d0.round, d0.seed, d0.cols) == (0, 3, 1, 6, 64)


def test_linear_rejects_before_launch():
    lib = mx.load_library()
    X, W = _desc(64, 128, 1), _desc(96, 128, 1)
    assert _lin(lib, 3, X, W) == -4                       # bad op
    assert _lin(lib, 0, X, W, out=2) == -4                # bad dtype
    assert _lin(lib, 1, X, W) == -4                       # dgrad needs B on axis 0
    assert _lin(lib, 2, X, W) == -4                       # wgrad needs axis 0 for both
    assert _lin(lib, 0, X, _desc(96, 160, 1)) == -2       # K mismatch
    assert _lin(lib, 0, X, _desc(96, 128, 1, rot=0)) == -5
    assert _lin(lib, 0, _desc(64, 128, 1, rot=2, seed=1), _desc(96, 128, 1, rot=2, seed=2)) == -5
    # same low 32 bits, different role in the high bits: accepted by validation
    # (so pass a NULL C to stop at the pointer check instead of launching)
    assert _lin(lib, 0, _desc(64, 128, 1, rot=2, seed=1), _desc(96, 128, 1, rot=2, seed=1 | 1 << 32),
                C=None) == -1
    assert _lin(lib, 0, X, W, ldc=95) == -2               # ldc < N
    assert _lin(lib, 0, X, W, C=4096 + 2) == -3           # fp32 C not 4-byte aligned
    assert _lin(lib, 0, X, W, C=4096 + 1, out=1) == -3    # bf16 C not 2-byte aligned
    assert _lin(lib, 0, X, W, C=None) == -1
    assert _lin(lib, 0, _desc(64, 128, 1, codes=None), W) == -1
    assert _lin(lib, 0, _desc(64, 128, 1, codes=4100), W) == -3
    bad = _desc(64, 128, 1)
    bad.block = 16
    assert _lin(lib, 0, bad, W) == -4
    assert _lin(lib, 0, _desc(64, 128, 1, fmt=2), _desc(96, 128, 1, fmt=2)) == -4  # bad format
    assert _lin(lib, 0, _desc(64, 128, 1, fmt=1, rnd=1), _desc(96, 128, 1, fmt=1, rnd=1)) == -4
    assert _lin(lib, 0, _desc(64, 128, 1, fmt=1), W) == -5                # E4M3 with E2M1
    assert _lin(lib, 0, X, _desc(96, 128, 1, fmt=1)) == -5
    assert _lin(lib, 0, _desc(64, 128, 1, fmt=1), _desc(96, 128, 1, fmt=1), C=None) == -1
    assert lib.mx_linear(0, None, ctypes.byref(W), 4096, 96, 0, None) == -1
    # descriptors not filled by a quantize call, with extents that would overflow
    assert _lin(lib, 0, _desc(1 << 36, 1 << 36, 1), _desc(96, 1 << 36, 1)) == -6
    assert _lin(lib, 0, X, W, ldc=1 << 60) == -6          # M * ldc * 4 bytes above 2^62
    assert _lin(lib, 0, X, W, ldc=1 << 60, out=1) == -6


def test_linear_empty_is_a_noop():
    lib = mx.load_library()
    assert _lin(lib, 0, _desc(0, 128, 1), _desc(96, 128, 1), C=None) == 0
    assert _lin(lib, 2, _desc(64, 0, 0), _desc(64, 32, 0), C=None) == 0


def _linb(lib, op, As, Bs, Cs=None, ldc=None, out=0, count=None):
    n = len(As)
    da = (mx.QTensorDesc * n)(*As)
    db = (mx.QTensorDesc * n)(*Bs)
    Cs = [4096 * (i + 1) for i in range(n)] if Cs is None else Cs
    cs = (ctypes.c_void_p * n)(*Cs)
    ldc = ldc if ldc is not None else (Bs[0].rows if Bs[0].axis == 1 else Bs[0].cols)
    return lib.mx_linear_batched(op, n if count is None else count, da, db, cs, ldc, out, None)


def test_linear_batched_rejects_before_launch():
    """Validation of mx_linear_batched fails before any HIP call; every entry
    is checked as mx_linear checks it."""
    lib = mx.load_library()
    X, W = _desc(64, 128, 1), _desc(96, 128, 1)
    assert _linb(lib, 0, [X, X], [W, W], count=0) == -4
    assert _linb(lib, 0, [X] * 4, [W] * 4, count=5) == -4
    assert lib.mx_linear_batched(0, 1, None, None, None, 96, 0, None) == -1
    assert _linb(lib, 0, [X, _desc(32, 128, 1)], [W, W]) == -2           # entry rows differ
    assert _linb(lib, 0, [X, X], [W, _desc(64, 128, 1)]) == -2           # entry N differs
    assert _linb(lib, 0, [X, X], [W, _desc(96, 160, 1)]) == -2           # entry K differs
    assert _linb(lib, 0, [X, X], [W, _desc(96, 128, 1, rot=0)]) == -5    # second pair's rotations
    assert _linb(lib, 1, [X, X], [W, W]) == -4                           # dgrad needs B on axis 0
    assert _linb(lib, 0, [X, X], [W, W], Cs=[4096, None]) == -1
    assert _linb(lib, 0, [X, X], [W, W], Cs=[4096, 4098]) == -3          # fp32 C misaligned
    assert _linb(lib, 0, [X, X], [W, W], ldc=95) == -2
    assert _linb(lib, 0, [X, X], [W, W], out=2) == -4
    E = _desc(64, 128, 1, fmt=1)
    assert _linb(lib, 0, [E, E], [_desc(96, 128, 1, fmt=1)] * 2, Cs=[4096, 8192]) == -6  # MXFP8
    # empty problem: nothing launched
    assert _linb(lib, 0, [_desc(0, 128, 1)] * 2, [W, W], Cs=[None, None]) == 0


def test_dequantize_rejects_before_launch():
    lib = mx.load_library()
    deq = lambda d, out=4096, ld=None: lib.mx_dequantize(  # noqa: E731
        ctypes.byref(d), out, d.cols if ld is None else ld, None)
    assert lib.mx_dequantize(None, 4096, 128, None) == -1
    assert deq(_desc(64, 128, 1), ld=127) == -2           # ld < cols
    assert deq(_desc(64, 128, 1), out=None) == -1
    assert deq(_desc(64, 128, 1), out=4098) == -3         # fp32 out not 4-byte aligned
    assert deq(_desc(64, 48, 1)) == -2                    # K % 32
    assert deq(_desc(64, 128, 2)) == -4                   # bad axis
    assert deq(_desc(64, 128, 1, codes=None)) == -1
    assert deq(_desc(64, 128, 1, fmt=3)) == -4
    assert deq(_desc(1 << 17, 1 << 14, 1)) == -6          # beyond the size limit
    assert deq(_desc(1 << 36, 1 << 36, 0)) == -6          # padded product would wrap
    assert deq(_desc(64, 128, 1), ld=1 << 60) == -6       # rows * ld * 4 bytes above 2^62
    assert deq(_desc(0, 128, 1), out=None) == 0           # empty: nothing launched
