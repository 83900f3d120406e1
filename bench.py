#!/usr/bin/env python3
"""Throughput of the MXFP4 linear-layer hot path on one MI355X.

One step = rotate + quantize operand A, rotate + quantize operand B, MXFP4 GEMM
(fp32 accumulation), i.e. the whole hot path of one GEMM of the triple, with
the inputs already resident in HBM. The headline workload is the Fprop of a
Llama-3.1-8B q_proj layer: X 8192x4096 bf16 (0.1% of channels x50), W
4096x4096 bf16, 32-point Hadamard + RNE along K = 4096, bf16 output.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--variant V]
                    [--all] [--no-cpu-baseline]

Prints ONE JSON line. `value` is TFLOP/s including the two quantizations
(2*M*N*K / step time). The inputs are replicated so that consecutive steps
read different copies and the working set exceeds the last-level cache.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MXFP4 linear TFLOP/s incl. Hadamard+quant, Llama-3.1-8B shapes; % MFMA peak"
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense MXFP8 MFMA (the E4M3 comparator)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
LLC_BYTES = 256 << 20          # MI355X Infinity Cache
CSRC = "mxfp4_microscaled_precision_amd/csrc/"
GEMM_SRC = (CSRC + "mx_gemm.hip", CSRC + "mx_gemm_common.h")
GEMM_E4M3_SRC = (CSRC + "mx_gemm_e4m3.hip", CSRC + "mx_gemm_common.h")
WORKLOADS_REF = None
GEMM_TRAFFIC = "profiles/gemm_{}_traffic.md"
GEMM_E4M3_TRAFFIC = "profiles/gemm_e4m3_{}_traffic.md"
QUANT_SRC = (CSRC + "mx_quant.hip", CSRC + "mx_device.h")
QUANT_TRAFFIC = "profiles/quant_{}_traffic.md"
QUANT_E4M3_TRAFFIC = "profiles/quant_e4m3_{}_traffic.md"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # about 40 ms of back-to-back steps: the clock settles under sustained load
    # (measured: 10 warmup steps time the step ~15% slow, 400 and more agree)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="fprop_q_proj")
    ap.add_argument("--variant", default=None)
    ap.add_argument("--format", default="fp4_e2m1", choices=("fp4_e2m1", "fp8_e4m3"),
                    help="element format of the timed path (fp8_e4m3: the MXFP8 comparator)")
    ap.add_argument("--all", action="store_true",
                    help="also time every other workload/variant and the full block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--structural", action="store_true",
                    help="also run the repeated-Wgrad structural-error harness")
    ap.add_argument("--cpu-reps", type=int, default=3,
                    help="repetitions of the whole-workload oracle run (cpu_baseline)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB three "
                         "times (reference for HBM byte counters)")
    return ap.parse_args()


class Runner:
    """Pre-marshalled C-ABI calls for one workload variant (no torch calls in
    the timed loop)."""

    def __init__(self, mx, w, variant, tensors=None, min_bytes=2 * LLC_BYTES, device="cuda",
                 fmt="fp4_e2m1"):
        import numpy as np
        import torch
        from datagen import operands_for, workload_tensors

        self.w = w
        self.fmt = fmt
        label, rot, rnd, seed = [v for v in w.variants if v[0] == variant][0]
        if fmt == "fp8_e4m3" and rnd != "rne":
            raise ValueError("the E4M3 comparator rounds to nearest only")
        self.variant, self.rot, self.rnd, self.seed = label, rot, rnd, seed
        t = tensors if tensors is not None else workload_tensors(w)
        a_src, self.ax_a, b_src, self.ax_b = operands_for(w, t)
        self.a_shape, self.b_shape = a_src.shape, b_src.shape
        self.a_src, self.b_src = a_src, b_src
        per_copy = 2 * (a_src.size + b_src.size)
        self.ncopy = max(1, math.ceil(min_bytes / per_copy))
        lib = mx.load_library()
        self.lib = lib

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
                torch.bfloat16).to(device)

        a0, b0 = dev(a_src), dev(b_src)
        self.A = [a0] + [a0.clone() for _ in range(self.ncopy - 1)]
        self.B = [b0] + [b0.clone() for _ in range(self.ncopy - 1)]
        stream = torch.cuda.current_stream().cuda_stream
        self.stream = stream
        seed_a = seed & 0xFFFFFFFF
        seed_b = seed_a | (1 << 32)
        self.qa, self.qb, self.qcalls_a, self.qcalls_b = [], [], [], []
        fp8 = fmt == "fp8_e4m3"
        self.qfn = lib.mx_quantize_fp8 if fp8 else lib.mx_quantize
        for i in range(self.ncopy):
            if fp8:
                qa = mx.quantize_fp8(self.A[i], self.ax_a, rot, seed=seed_a)
                qb = mx.quantize_fp8(self.B[i], self.ax_b, rot, seed=seed_b)
            else:
                qa = mx.quantize(self.A[i], self.ax_a, rot, rnd, seed=seed_a)
                qb = mx.quantize(self.B[i], self.ax_b, rot, rnd, seed=seed_b)
            self.qa.append(qa)
            self.qb.append(qb)
            for q, src, lst in ((qa, self.A[i], self.qcalls_a), (qb, self.B[i], self.qcalls_b)):
                r, c = src.shape
                head = (src.data_ptr(), r, c, src.stride(0), q.desc.axis, 32, mx.ROTATE[rot])
                tail = (q.desc.seed, q.codes.data_ptr(), q.scales.data_ptr(), None, stream)
                lst.append(head + tail if fp8 else head + (mx.ROUND[rnd],) + tail)
        # Fprop's X and W are both quantized along `in`: one mx_quantize_pair
        # launch does both (byte-identical to the two mx_quantize calls)
        self.pcalls = None
        if not fp8 and self.ax_a == 1 and self.ax_b == 1 and a_src.shape[1] == b_src.shape[1]:
            self.pcalls = []
            for i in range(self.ncopy):
                qa, qb, sa, sb = self.qa[i], self.qb[i], self.A[i], self.B[i]
                self.pcalls.append((sa.data_ptr(), sa.shape[0], sa.stride(0), sb.data_ptr(),
                                    sb.shape[0], sb.stride(0), sa.shape[1], 32, mx.ROTATE[rot],
                                    mx.ROUND[rnd], qa.desc.seed, qb.desc.seed,
                                    qa.codes.data_ptr(), qa.scales.data_ptr(),
                                    qb.codes.data_ptr(), qb.scales.data_ptr(), None, None,
                                    stream))
        self.M, self.N = self.qa[0].mn, self.qb[0].mn
        self.K = self.qa[0].k
        self.out_dtype = w.out_dtype
        dt = torch.float32 if w.out_dtype == "f32" else torch.bfloat16
        self.C = torch.empty((self.M, self.N), dtype=dt, device=device)
        self.lcalls = [(mx.OPS[w.op], ctypes.byref(self.qa[i].desc), ctypes.byref(self.qb[i].desc),
                        self.C.data_ptr(), self.C.stride(0), mx.OUT_DTYPES[w.out_dtype], stream)
                       for i in range(self.ncopy)]
        torch.cuda.synchronize()

    def step(self, i):
        j = i % self.ncopy
        if self.pcalls is not None:
            quantized = self.lib.mx_quantize_pair(*self.pcalls[j]) == 0
        else:
            quantized = not (self.qfn(*self.qcalls_a[j]) or self.qfn(*self.qcalls_b[j]))
        if not quantized or self.lib.mx_linear(*self.lcalls[j]):
            raise RuntimeError("library call failed")

    def quant_a(self, i):
        if self.qfn(*self.qcalls_a[i % self.ncopy]):
            raise RuntimeError("quantize failed")

    def quant_b(self, i):
        if self.qfn(*self.qcalls_b[i % self.ncopy]):
            raise RuntimeError("quantize failed")

    def gemm(self, i):
        if self.lib.mx_linear(*self.lcalls[i % self.ncopy]):
            raise RuntimeError("mx_linear failed")

    # algorithmic work
    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def code_bytes(self):
        return 1.0 if self.fmt == "fp8_e4m3" else 0.5

    def quant_bytes(self, shape):
        n = shape[0] * shape[1]
        return n * (2 + self.code_bytes() + 1.0 / 32)

    def gemm_bytes(self):
        ob = 4 if self.out_dtype == "f32" else 2
        return (self.M + self.N) * self.K * (self.code_bytes() + 1.0 / 32) + self.M * self.N * ob


SETTLE_MS = 40.0   # sustained load before timing: the clock settles in about this long


def settle(fn, min_ms=SETTLE_MS):
    """Run fn(i) back to back for at least min_ms of GPU time (untimed
    warmup sized from a short first burst); returns the number of calls."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(5):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1) / 5, 1e-3)
    n = int(math.ceil(min_ms / per))
    for i in range(n):
        fn(5 + i)
    torch.cuda.synchronize()
    return 5 + n


def time_loop(fn, iters, warmup=None):
    """Average ms per call of fn(i) over `iters` back-to-back calls, between
    one pair of HIP events on the current stream (the stream the library
    launches on)."""
    import torch
    if warmup is None:
        settle(fn)
    for i in range(warmup or 0):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def measure(r, steps, warmup=None):
    """The timed region: `steps` whole steps (quantize A, quantize B, GEMM)
    back to back, after `warmup` untimed steps (None: as many as SETTLE_MS of
    load takes). Then each kernel alone, back to back, for its average
    launch duration (events between the kernels of a step would add gaps)."""
    import torch
    if warmup is None:
        settle(r.step)
    for i in range(warmup or 0):
        r.step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        r.step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    t_qa = time_loop(r.quant_a, max(steps, 10), 3)
    t_qb = time_loop(r.quant_b, max(steps, 10), 3)
    t_g = time_loop(r.gemm, max(steps, 10), 3)
    flops = r.flops()
    return {
        "ms_per_step": ms,
        "wall_ms_per_step": wall * 1e3 / steps,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "t_quant_a_us": t_qa * 1e3,
        "t_quant_b_us": t_qb * 1e3,
        "t_gemm_us": t_g * 1e3,
        "gemm_tflops": flops / (t_g * 1e-3) / 1e12,
        "quant_a_gbs": r.quant_bytes(r.a_shape) / (t_qa * 1e-3) / 1e9,
        "quant_b_gbs": r.quant_bytes(r.b_shape) / (t_qb * 1e-3) / 1e9,
    }


def cpu_baseline(r, reps):
    """The oracle as it stands, on the host cores: the whole workload
    (quantize both operands, fp64 GEMM of the dequantized operands), `reps`
    times; the value is the workload's flops over the mean time."""
    import numpy as np  # noqa: F401

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()
                            if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = None
    seed_a = r.seed & 0xFFFFFFFF
    t_q = t_g = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        qa = oracle.quantize_ref(r.a_src, r.ax_a, rotate=r.rot, rounding=r.rnd, seed=seed_a,
                                 fmt=r.fmt)
        qb = oracle.quantize_ref(r.b_src, r.ax_b, rotate=r.rot, rounding=r.rnd,
                                 seed=seed_a | (1 << 32), fmt=r.fmt)
        t1 = time.perf_counter()
        oracle.mx_gemm_ref(qa, qb)
        t2 = time.perf_counter()
        t_q += t1 - t0
        t_g += t2 - t1
        del qa, qb
    per = (t_q + t_g) / reps
    return {
        "value": round(r.flops() / per / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": blas_threads if blas_threads else len(os.sched_getaffinity(0)),
        "affinity_cores": len(os.sched_getaffinity(0)),
        "quantizer_threads": 1,
        "kind": "oracle",
        "sample": (f"whole workload {r.M}x{r.N}x{r.K} x{reps}: oracle quantize of both "
                   f"operands (NumPy, 1 thread, {t_q / reps:.2f} s) + fp64 GEMM of the "
                   f"dequantized operands (BLAS, {t_g / reps:.2f} s) per repetition"),
        "sample_seconds": round(t_q + t_g, 2),
    }


def sources_digest(paths):
    """sha256[:16] over the concatenated kernel sources (repo-relative)."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_src, summary):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel sources have changed since the counters were taken."""
    try:
        digest = sources_digest(kernel_src)
        with open(os.path.join(ROOT, summary)) as fh:
            fields = dict(ln.strip()[2:].split(": ", 1) for ln in fh
                          if ln.startswith("- ") and ": " in ln)
        if fields.get("kernel source sha256[:16]") != digest:
            return None
        return float(fields["traffic bytes per launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(sharding across GPUs is not implemented)"}))
        sys.exit(2)
    import torch

    import mxfp4_microscaled_precision_amd as mx
    from datagen import WORKLOADS, block_workloads, workload_tensors
    global WORKLOADS_REF
    WORKLOADS_REF = WORKLOADS

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    mx.load_library()
    w = WORKLOADS[args.workload]
    variant = args.variant or w.variants[0][0]
    print(f"[bench] workload {w.name} variant {variant}", file=sys.stderr, flush=True)
    fp8 = args.format == "fp8_e4m3"
    r = Runner(mx, w, variant, fmt=args.format)
    res = measure(r, args.steps, args.warmup)
    t_dom = res["t_gemm_us"]
    gemm_ach = r.flops() / (t_dom * 1e-6) / 1e12
    qa_ach = res["quant_a_gbs"]
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_FP4_TFLOPS
    gemm_src, gemm_prof = (GEMM_E4M3_SRC, GEMM_E4M3_TRAFFIC) if fp8 else (GEMM_SRC, GEMM_TRAFFIC)
    quant_prof = QUANT_E4M3_TRAFFIC if fp8 else QUANT_TRAFFIC
    out = {
        "metric": METRIC,
        "value": round(res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3xfp8_e4m3->f32" if fp8 else "fp4_e2m1xfp4_e2m1->f32",
        "data": "synthetic (seeded PCG64; Llama-3.1-8B q_proj shapes, no real weights)",
        "config": {
            "workload": (f"{w.name}: {w.op} M={r.M} N={r.N} K={r.K}, rotate={r.rot}, "
                         f"round={r.rnd}, out={w.out_dtype}"),
            "M": r.M, "N": r.N, "K": r.K, "variant": variant, "input_copies": r.ncopy,
        },
        "pct_mfma_peak": round(100.0 * res["tflops"] / peak, 2),
        "roofline": {
            "kernel": ("gemm_e4m3_kernel (MXFP8 comparator GEMM)" if fp8
                       else "gemm_tiled_kernel (MXFP4 MFMA GEMM)"),
            "bound": "mfma",
            "achieved": round(gemm_ach, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(gemm_ach / peak, 4),
            "traffic": recorded_traffic(gemm_src, gemm_prof.format(w.name)),
        },
        "quant_roofline": {
            "kernel": f"mx_quant axis {r.ax_a} (operand A)",
            "bound": "hbm",
            "achieved": round(qa_ach, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(qa_ach / PEAK_HBM_GBS, 4),
            "traffic": recorded_traffic(QUANT_SRC, quant_prof.format(w.name)),
        },
        "per_kernel_us": {k: round(res[k], 2) for k in ("t_quant_a_us", "t_quant_b_us",
                                                       "t_gemm_us")},
        "quant_b_gbs": round(res["quant_b_gbs"], 1),
        "gemm_only_tflops": round(res["gemm_tflops"], 2),
    }
    if not fp8 and r.rnd == "rne":
        out["fp8_comparator"] = fp8_comparator(mx, w, variant, max(10, args.steps // 4), res)
        print(f"[bench] fp8 comparator {out['fp8_comparator']}", file=sys.stderr, flush=True)
    if args.all:
        extra = {}
        for name, wl in WORKLOADS.items():
            if name == "tiny_wgrad":
                continue
            t = workload_tensors(wl)
            for v in wl.variants:
                if name == w.name and v[0] == variant:
                    continue
                rr = Runner(mx, wl, v[0], tensors=t)
                m = measure(rr, max(10, args.steps // 4))
                extra[f"{name}/{v[0]}"] = {k: round(val, 3) for k, val in m.items()}
                print(f"[bench] {name}/{v[0]}: {m['tflops']:.1f} TFLOP/s", file=sys.stderr,
                      flush=True)
                del rr
        out["other_workloads"] = extra
        out["dual_quantizer"] = dual_quant_bench(mx, max(10, args.steps // 2))
        print(f"[bench] dual quantizer {out['dual_quantizer']}", file=sys.stderr, flush=True)
        wg = WORKLOADS["wgrad_gate_proj"]
        out["wgrad_gate_proj_quant_error"] = output_mse(mx, wg, [v[0] for v in wg.variants])
        print(f"[bench] quant error {out['wgrad_gate_proj_quant_error']}", file=sys.stderr,
              flush=True)
        out["block"] = bench_block(mx, block_workloads(), max(5, args.steps // 20))
    if args.structural or args.all:
        out["structural_error"] = structural_error(mx)
        print("[bench] structural error done", file=sys.stderr, flush=True)
    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(r, args.cpu_reps)
    print(json.dumps(out), flush=True)


def fp8_comparator(mx, w, variant, steps, fp4_res):
    """The same workload and rotation through the MXFP8 (E4M3) comparator:
    whole-step and per-kernel times beside the MXFP4 ones measured just
    before, and the FP4 : FP8 speed ratios (the pages' context: FP4 has in
    theory twice FP8's compute; the MXFP4 training step ran about 20% faster
    than the FP8 baseline)."""
    r8 = Runner(mx, w, variant, fmt="fp8_e4m3")
    m8 = measure(r8, steps)
    fl = r8.flops()
    out = {
        "ms_per_step": round(m8["ms_per_step"], 5),
        "tflops": round(m8["tflops"], 2),
        "per_kernel_us": {k: round(m8[k], 2) for k in ("t_quant_a_us", "t_quant_b_us",
                                                      "t_gemm_us")},
        "gemm_tflops": round(fl / (m8["t_gemm_us"] * 1e-6) / 1e12, 2),
        "gemm_frac_fp8_peak": round(fl / (m8["t_gemm_us"] * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
        "quant_a_gbs": round(m8["quant_a_gbs"], 1),
        "fp4_over_fp8_step_speed": round(m8["ms_per_step"] / fp4_res["ms_per_step"], 3),
        "fp4_over_fp8_gemm_speed": round(m8["t_gemm_us"] / fp4_res["t_gemm_us"], 3),
    }
    del r8
    return out


def output_mse(mx, wl, variants):
    """Quantization error at the output of one GEMM: the fp32 MXFP4 result
    against the fp32 product of the unquantized bf16 operands (torch.matmul on
    the GPU), as mean squared error and relative Frobenius error."""
    import torch
    from datagen import operands_for, workload_tensors
    t = workload_tensors(wl)
    a_src, ax_a, b_src, ax_b = operands_for(wl, t)
    res = {}
    for label in variants:
        rr = Runner(mx, wl, label, tensors=t, min_bytes=0)
        c = torch.empty((rr.M, rr.N), dtype=torch.float32, device="cuda")
        st = rr.lib.mx_linear(mx.OPS[wl.op], ctypes.byref(rr.qa[0].desc),
                              ctypes.byref(rr.qb[0].desc), c.data_ptr(), c.stride(0),
                              mx.OUT_DTYPES["f32"], rr.stream)
        if st:
            raise RuntimeError("mx_linear failed")
        a = rr.A[0].float()
        b = rr.B[0].float()
        a = a if ax_a == 1 else a.t().contiguous()        # [M, K]
        b = b if ax_b == 1 else b.t().contiguous()        # [N, K]
        ref = torch.matmul(a, b.t().contiguous())
        d = (c - ref).double()
        res[label] = {"output_mse": float((d * d).mean()),
                      "rel_fro": float(d.norm() / ref.double().norm())}
        del rr, a, b, ref, d, c
        torch.cuda.empty_cache()
    return res


def dual_quant_bench(mx, steps):
    """The dual-output quantizer against the two single-orientation launches it
    replaces, on the Fprop activation X and the Wgrad gradient dY (H32, RNE).
    Algorithmic bytes: 2 B read + 2 x (0.5 + 1/32) B written per element."""
    import torch
    from datagen import workload_tensors
    res = {}
    for wname, tname in (("fprop_q_proj", "X"), ("wgrad_gate_proj", "dY")):
        src = workload_tensors(WORKLOADS_REF[wname])[tname]
        x = torch.from_numpy(src.view("int16")).view(torch.bfloat16).to("cuda")
        copies = [x] + [x.clone() for _ in range(max(0, (512 << 20) // (2 * x.numel())))]
        lib = mx.load_library()
        st = torch.cuda.current_stream().cuda_stream
        rows, cols = x.shape
        outs = {}
        for axis in (1, 0):
            cb, sb = mx.quantize_sizes(rows, cols, axis)
            outs[axis] = (torch.empty(cb, dtype=torch.uint8, device="cuda"),
                          torch.empty(sb, dtype=torch.uint8, device="cuda"))
        d1, d0 = mx.QTensorDesc(), mx.QTensorDesc()

        def dual(i):
            c = copies[i % len(copies)]
            if lib.mx_quantize_dual(c.data_ptr(), rows, cols, c.stride(0), 32, 1, 0, 0, 0,
                                    outs[1][0].data_ptr(), outs[1][1].data_ptr(),
                                    outs[0][0].data_ptr(), outs[0][1].data_ptr(),
                                    ctypes.byref(d1), ctypes.byref(d0), st):
                raise RuntimeError("mx_quantize_dual failed")

        def single(axis):
            def f(i):
                c = copies[i % len(copies)]
                if lib.mx_quantize(c.data_ptr(), rows, cols, c.stride(0), axis, 32, 1, 0, 0,
                                   outs[axis][0].data_ptr(), outs[axis][1].data_ptr(),
                                   ctypes.byref(d1), st):
                    raise RuntimeError("mx_quantize failed")
            return f

        t_d = time_loop(dual, steps) * 1e3
        t_1 = time_loop(single(1), steps) * 1e3
        t_0 = time_loop(single(0), steps) * 1e3
        n = rows * cols
        res[f"{wname}/{tname} {rows}x{cols}"] = {
            "dual_us": round(t_d, 2), "axis1_us": round(t_1, 2), "axis0_us": round(t_0, 2),
            "dual_gbs": round(n * (2 + 2 * (0.5 + 1 / 32)) / (t_d * 1e-6) / 1e9, 1),
            "speedup_vs_two_launches": round((t_1 + t_0) / t_d, 3)}
        del copies, outs, x
        torch.cuda.empty_cache()
    return res


STRUCTURAL_VARIANTS = (("det_hadamard", "hadamard", "rne", False),
                       ("det_hadamard16", "hadamard16", "rne", False),
                       ("rand_sign_hadamard", "rand_sign_hadamard", "rne", True),
                       ("no_rotation_sr", "none", "sr", True),
                       ("hadamard_sr", "hadamard", "sr", True))


def structural_error(mx, T=8192, n_out=2048, n_in=1024, steps=64, data_seed=3):
    """Error of Wgrad repeated over `steps` steps on fixed tensors.

    dY [T, n_out] = 1e-4 t_3 and X [T, n_in] ~ N(0, 1) (bf16, the Wgrad
    gate/up distributions) stay fixed; step k computes dW_k = dY^T X through
    the MXFP4 path (both operands quantized along T), with seed k for the
    randomized variants (random signs, stochastic rounding) and the same
    deterministic rotation every step otherwise. For K = 1, 2, 4, ... the
    relative Frobenius error of the K-step mean against the fp32 product of
    the bf16 operands is reported, with the single-step error: a fixed error
    pattern keeps the mean's error at the single-step value, a pattern that
    changes from step to step lets it fall. The reference product is a plain
    torch fp32 matmul (measurement only)."""
    import numpy as np
    import torch
    from datagen import normal_bf16, student_t_bf16
    rng = np.random.Generator(np.random.PCG64(data_seed))
    dY = student_t_bf16(rng, (T, n_out), 3.0, 1e-4)
    X = normal_bf16(rng, (T, n_in), 1.0)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda")  # noqa: E731
    dYd, Xd = dev(dY), dev(X)
    ref = torch.matmul(dYd.float().t().contiguous(), Xd.float())
    ref_norm = ref.double().norm().item()
    out = {"shape": {"T": T, "out": n_out, "in": n_in}, "steps": steps, "variants": {}}
    Ks = [k for k in (1, 2, 4, 8, 16, 32, 64, 128, 256) if k <= steps]
    for label, rot, rnd, reseed in STRUCTURAL_VARIANTS:
        acc = torch.zeros_like(ref, dtype=torch.float64)
        single = []
        curve = {}
        for k in range(1, steps + 1):
            seed = k if reseed else 0
            qa = mx.quantize(dYd, 0, rot, rnd, seed=seed)
            qb = mx.quantize(Xd, 0, rot, rnd, seed=seed | (1 << 32))
            c = mx.linear("wgrad", qa, qb, "f32")
            acc += c.double()
            if k <= 4:
                single.append(((c.double() - ref.double()).norm() / ref_norm).item())
            if k in Ks:
                curve[k] = ((acc / k - ref.double()).norm() / ref_norm).item()
        out["variants"][label] = {
            "rotate": rot, "round": rnd, "new_seed_per_step": reseed,
            "single_step_rel_err": [round(v, 6) for v in single],
            "mean_rel_err": {str(k): round(v, 6) for k, v in curve.items()},
            "mean_over_single": round(curve[Ks[-1]] / single[0], 4)}
    return out


# Linears whose input X a real block shares with an earlier one (q/k/v read
# the same normed hidden state, gate/up the same one): their X quantizations
# (Fprop operand A, axis 1; Wgrad operand B, axis 0) could be reused.
SHARED_INPUT_LINEARS = ("k_proj", "v_proj", "up_proj")


def block_dual_linear(mx, wl, tensors, steps):
    """One linear of the block as a training step runs it with the dual-output
    quantizer: X, W and dY are each quantized once into both orientations
    (mx_quantize_dual), then Fprop, Dgrad and Wgrad run on those operands.
    The operands are byte for byte those of the per-op quantizations. Returns
    {variant: ms per linear}."""
    import numpy as np
    import torch
    lib = mx.load_library()
    st = torch.cuda.current_stream().cuda_stream

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to("cuda")

    src = {k: dev(tensors[k]) for k in ("X", "W", "dY")}
    T, n_out, n_in = wl.tokens, wl.out_features, wl.in_features
    bufs, descs = {}, {}
    for k, x in src.items():
        rows, cols = x.shape
        for axis in (1, 0):
            cb, sb = mx.quantize_sizes(rows, cols, axis)
            bufs[k, axis] = (torch.empty(cb, dtype=torch.uint8, device="cuda"),
                             torch.empty(sb, dtype=torch.uint8, device="cuda"))
            descs[k, axis] = mx.QTensorDesc()
    outs = {"fprop": torch.empty((T, n_out), dtype=torch.bfloat16, device="cuda"),
            "dgrad": torch.empty((T, n_in), dtype=torch.bfloat16, device="cuda"),
            "wgrad": torch.empty((n_out, n_in), dtype=torch.float32, device="cuda")}
    # (A, B) of each op, as (tensor, axis)
    ops = {"fprop": (("X", 1), ("W", 1)), "dgrad": (("dY", 1), ("W", 0)),
           "wgrad": (("dY", 0), ("X", 0))}
    res = {}
    for label, rot, rnd, seed in wl.variants:
        sa = seed & 0xFFFFFFFF
        sb_ = sa | (1 << 32)
        # seeds by role: X is A of Fprop and B of Wgrad; W is B of both of
        # its ops; dY is A of both of its ops
        seeds = {"X": (sa, sb_), "W": (sb_, sb_), "dY": (sa, sa)}

        def step(i):
            for k, x in src.items():
                s1, s0 = seeds[k]
                if lib.mx_quantize_dual(x.data_ptr(), x.shape[0], x.shape[1], x.stride(0), 32,
                                        mx.ROTATE[rot], mx.ROUND[rnd], s1, s0,
                                        bufs[k, 1][0].data_ptr(), bufs[k, 1][1].data_ptr(),
                                        bufs[k, 0][0].data_ptr(), bufs[k, 0][1].data_ptr(),
                                        ctypes.byref(descs[k, 1]), ctypes.byref(descs[k, 0]), st):
                    raise RuntimeError("mx_quantize_dual failed")
            for op, (a, b) in ops.items():
                c = outs[op]
                if lib.mx_linear(mx.OPS[op], ctypes.byref(descs[a]), ctypes.byref(descs[b]),
                                 c.data_ptr(), c.stride(0), 1 if op != "wgrad" else 0, st):
                    raise RuntimeError("mx_linear failed")

        res[label] = time_loop(step, steps)
    del src, bufs, outs
    torch.cuda.empty_cache()
    return res


def bench_block(mx, wls, steps):
    """Full Llama-3.1-8B block: 7 linears x {fprop, dgrad, wgrad} per variant.

    Each op quantizes its own two operands (the primary figure). The
    `shared_input` figure also drops the X quantizations that k/v reuse from
    q and up from gate, using the same measured per-kernel times. The
    `dual_quantizer` figure times each linear as a training step runs it:
    X, W and dY quantized once each into both orientations, then the three
    GEMMs (block_dual_linear)."""
    import torch
    from datagen import workload_tensors
    res = {}
    cache = {}
    dual_ms = {}
    for wl in wls:
        key = wl.data_seed
        if key not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[key] = workload_tensors(wl)
            for v, ms in block_dual_linear(mx, wl, cache[key], steps).items():
                dual_ms[v] = dual_ms.get(v, 0.0) + ms
        for v in wl.variants:
            rr = Runner(mx, wl, v[0], tensors=cache[key], min_bytes=0)
            m = measure(rr, steps)
            d = res.setdefault(v[0], {"flops": 0.0, "ms": 0.0, "saved_ms": 0.0, "ops": {}})
            d["flops"] += rr.flops()
            d["ms"] += m["ms_per_step"]
            lin = wl.name[len("block_"):].rsplit("_", 1)[0]
            if lin in SHARED_INPUT_LINEARS and wl.op in ("fprop", "wgrad"):
                if wl.op == "wgrad":
                    saved = 1e-3 * m["t_quant_b_us"]
                elif rr.pcalls is not None:
                    # X and W in one launch: what X adds is the step less W's own
                    # launch and the GEMM
                    saved = max(0.0, m["ms_per_step"] - 1e-3 * (m["t_quant_b_us"] + m["t_gemm_us"]))
                else:
                    saved = 1e-3 * m["t_quant_a_us"]
                d["saved_ms"] += saved
            d["ops"][wl.name] = {"ms": round(m["ms_per_step"], 4), "tflops": round(m["tflops"], 1),
                                 "t_gemm_us": round(m["t_gemm_us"], 1)}
            del rr
        print(f"[bench] block {wl.name} done", file=sys.stderr, flush=True)
    for v, d in res.items():
        d["tflops"] = round(d["flops"] / (d["ms"] * 1e-3) / 1e12, 2)
        d["pct_mfma_peak"] = round(100 * d["tflops"] / PEAK_FP4_TFLOPS, 2)
        ms_shared = d["ms"] - d.pop("saved_ms")
        d["shared_input"] = {"ms": round(ms_shared, 4),
                             "tflops": round(d["flops"] / (ms_shared * 1e-3) / 1e12, 2)}
        if v in dual_ms:
            d["dual_quantizer"] = {"ms": round(dual_ms[v], 4),
                                   "tflops": round(d["flops"] / (dual_ms[v] * 1e-3) / 1e12, 2),
                                   "pct_mfma_peak": round(100 * d["flops"] / (dual_ms[v] * 1e-3)
                                                          / 1e12 / PEAK_FP4_TFLOPS, 2)}
    return res


if __name__ == "__main__":
    main()
