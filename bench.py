#!/usr/bin/env python3
"""Throughput of the MXFP4 linear-layer hot path on one MI355X.

Headline workload (default, --workload block): the 21 GEMMs of one
Llama-3.1-8B transformer block at 16384 tokens -- q/k/v/o (4096x4096,
1024x4096 twice, 4096x4096), gate/up (14336x4096) and down (4096x14336),
each as Fprop Y = X W^T, Dgrad dX = dY W and Wgrad dW = dY^T X -- with every
operand rotated by the 32-point Hadamard and quantized to MXFP4 (E8M0 scale
per 32 elements, E2M1 elements, round to nearest even).

One step is one training step's linear-layer work of the block, with the
inputs already resident in HBM: each distinct X, W and dY is quantized once
into both packed orientations (mx_quantize_dual; q, k and v read one input
activation X, gate and up another, as in the model), then each linear's
Fprop (bf16 out), Dgrad (bf16 out) and Wgrad (fp32 out) run on those
operands.
`value` is the 21 GEMMs' 2*M*N*K over the step time, i.e. TFLOP/s including
the Hadamard and the quantization. The block's working set (about 7 GB)
exceeds the 256 MB last-level cache many times over, so every step reads
its inputs from HBM.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--variant V]
                    [--all] [--structural] [--no-cpu-baseline]

Prints ONE JSON line. --workload fprop_q_proj (or wgrad_gate_proj,
dgrad_down_proj) times one GEMM of the triple with its two quantizations as
the step instead.
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
QUANT_SRC = (CSRC + "mx_quant.hip", CSRC + "mx_device.h")
GEMM_TRAFFIC = "profiles/gemm_{}_traffic.md"
GEMM_E4M3_TRAFFIC = "profiles/gemm_e4m3_{}_traffic.md"
QUANT_TRAFFIC = "profiles/quant_{}_traffic.md"
QUANT_E4M3_TRAFFIC = "profiles/quant_e4m3_{}_traffic.md"
BLOCK_GEMM_TRAFFIC = "profiles/gemm_bf16_block_t16384_traffic.md"
BLOCK_QUANT_TRAFFIC = "profiles/quant_dual_block_t16384_traffic.md"
SETTLE_MS = 40.0   # sustained load before timing: the clock settles in about this long
WORKLOADS_REF = None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed steps after the settle phase (at least 40 ms of steps "
                         "back to back always runs first)")
    ap.add_argument("--workload", default="block")
    ap.add_argument("--variant", default=None)
    ap.add_argument("--tokens", type=int, default=16384, help="block workload: tokens T")
    ap.add_argument("--format", default="fp4_e2m1", choices=("fp4_e2m1", "fp8_e4m3"),
                    help="element format of a single-GEMM workload (fp8_e4m3: the MXFP8 "
                         "comparator)")
    ap.add_argument("--all", action="store_true",
                    help="also time every single-GEMM workload and variant, the block with "
                         "per-op quantization, the dual quantizer and the quantization error")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="block workload: skip the q_proj Fprop and FP8-comparator figures")
    ap.add_argument("--structural", action="store_true",
                    help="also run the repeated-Wgrad structural-error harness")
    ap.add_argument("--cpu-reps", type=int, default=1,
                    help="repetitions of the oracle run (cpu_baseline)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB three "
                         "times (reference for HBM byte counters)")
    return ap.parse_args()


def _dev_bf16(bits, device="cuda"):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to(device)


# ------------------------------------------------------------------ timing
def settle(fn, min_ms=SETTLE_MS, join=None):
    """Run fn(i) back to back for at least min_ms of GPU time (untimed,
    sized from a short first burst); returns the number of calls. join()
    makes the current stream wait for work fn left on other streams."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(3):
        fn(i)
    if join is not None:
        join()
    e1.record()
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1) / 3, 1e-3)
    n = int(math.ceil(min_ms / per))
    for i in range(n):
        fn(3 + i)
    torch.cuda.synchronize()
    return 3 + n


def timed(fn, steps, warmup=0, join=None):
    """Average ms per call of fn(i): at least SETTLE_MS of calls back to back,
    then `warmup` more, then `steps` calls between one pair of HIP events on
    the current stream, bracketed by device synchronisation. A call may
    launch on other streams if it first makes them wait for the current one;
    join() then makes the current stream wait for them before the closing
    event. Returns (ms per call, wall ms per call)."""
    import torch
    settle(fn, join=join)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(i)
    if join is not None:
        join()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


# ------------------------------------------------------ the Llama block
class BlockRunner:
    """The 7 linears of one Llama-3.1-8B block at T tokens, resident on the
    GPU with their quantized operands and outputs; pre-marshalled C-ABI
    calls (no torch compute inside a step; torch only records and waits on
    HIP events).

    A step of the dual-quantizer schedule runs on two streams of default
    priority: the quantizations on one, in group order, and the GEMMs on the
    other, each group's GEMMs waiting for that group's quantizations, and
    each group's quantizations waiting for that group's GEMMs of the step
    before (they overwrite the operands those read). The quantizer of the
    next group can then start while a GEMM drains its last tiles, and a GEMM
    while the last quantizer workgroups finish. Same launches, same
    outputs; `overlap = False` (and the per-launch instrumented pass) runs
    them in order on the current stream."""

    def __init__(self, mx, tokens=16384, keep_host=("k_proj",)):
        import torch
        from datagen import BLOCK_INPUT_OF, LLAMA_BLOCK_LINEARS, block_workloads, workload_tensors
        self.mx = mx
        self.lib = mx.load_library()
        self.stream = torch.cuda.current_stream().cuda_stream
        self.side = (torch.cuda.Stream(), torch.cuda.Stream())   # quantizer, GEMM streams
        self.overlap = True
        self.plan = None
        self.T = tokens
        wls = block_workloads(tokens)
        self.variants = wls[0].variants
        self.lins = []
        self.host = {}
        for li, lin in enumerate(LLAMA_BLOCK_LINEARS):
            wl = [w for w in wls if w.data_seed == 500 + li and w.op == "fprop"][0]
            t = workload_tensors(wl)
            if lin.name in keep_host:
                self.host[lin.name] = t
            # a linear that reads another's input (k, v: q's; up: gate's)
            # takes that linear's X and its packed buffers (BLOCK_INPUT_OF)
            lead = BLOCK_INPUT_OF.get(lin.name)
            src = {k: _dev_bf16(t[k]) for k in ("X", "W", "dY") if not (lead and k == "X")}
            del t
            bufs = {}
            if lead:
                L0 = [L for L in self.lins if L["name"] == lead][0]
                src = {"X": L0["src"]["X"], **src}
                for axis in (1, 0):
                    bufs["X", axis] = L0["bufs"]["X", axis][:2] + (mx.QTensorDesc(),)
            for k, x in src.items():
                rows, cols = x.shape
                for axis in (1, 0):
                    if (k, axis) in bufs:
                        continue
                    cb, sb = mx.quantize_sizes(rows, cols, axis)
                    bufs[k, axis] = (torch.empty(cb, dtype=torch.uint8, device="cuda"),
                                     torch.empty(sb, dtype=torch.uint8, device="cuda"),
                                     mx.QTensorDesc())
            T, o, i = tokens, lin.out_features, lin.in_features
            outs = {"fprop": torch.empty((T, o), dtype=torch.bfloat16, device="cuda"),
                    "dgrad": torch.empty((T, i), dtype=torch.bfloat16, device="cuda"),
                    "wgrad": torch.empty((o, i), dtype=torch.float32, device="cuda")}
            self.lins.append({"name": lin.name, "out": o, "in": i, "src": src, "bufs": bufs,
                              "outs": outs, "x_of": lead})
            print(f"[bench] block {lin.name}: {T}x{i} -> {o} resident", file=sys.stderr,
                  flush=True)
        # Linears that see their inputs together share one grouped GEMM launch
        # per op (mx_linear_batched): k and v read the same activations, gate
        # and up too. Each (tensor, axis) descriptor feeds exactly one op, so a
        # group's descriptors live side by side in one ctypes array per
        # (tensor, axis): the quantizer fills element j, the GEMM takes the array.
        by_name = {L["name"]: L for L in self.lins}
        self.groups = []
        for names in self.GROUPS:
            ls = [by_name[n] for n in names]
            descs = {}
            for key in ls[0]["bufs"]:
                arr = (mx.QTensorDesc * len(ls))()
                for j, L in enumerate(ls):
                    c, s, _ = L["bufs"][key]
                    L["bufs"][key] = (c, s, arr[j])
                descs[key] = arr
            self.groups.append({"lins": ls, "descs": descs})
        torch.cuda.synchronize()
        self.calls = []

    GROUPS = (("q_proj",), ("k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"),
              ("down_proj",))
    # ops a group runs as grouped launches (the others as single launches): the
    # gate and up Fprop, large on their own, measured 0.2-0.3% faster per step
    # as two launches; every other op of a pair gains from one launch
    GROUPED_OPS = {("k_proj", "v_proj"): ("fprop", "dgrad", "wgrad"),
                   ("gate_proj", "up_proj"): ("dgrad", "wgrad")}

    # (A, B) of each op as (tensor, axis), and the output dtype
    OPS = (("fprop", ("X", 1), ("W", 1), "bf16"), ("dgrad", ("dY", 1), ("W", 0), "bf16"),
           ("wgrad", ("dY", 0), ("X", 0), "f32"))

    def flops(self):
        return sum(3 * 2.0 * self.T * L["out"] * L["in"] for L in self.lins)

    def _seeds(self, seed):
        """Seeds by role: X is A of Fprop (axis 1) and B of Wgrad (axis 0);
        W is B of Fprop and of Dgrad; dY is A of Dgrad and of Wgrad."""
        sa = seed & 0xFFFFFFFF
        sb = sa | (1 << 32)
        return {"X": (sa, sb), "W": (sb, sb), "dY": (sa, sa)}

    def build(self, label, per_op=False):
        """The launch list of one step of variant `label`: a list of
        (kind, info, fn, args). With per_op, each op quantizes its own two
        operands (Fprop's pair in one launch) right before its GEMM."""
        mx, lib, st = self.mx, self.lib, self.stream
        _, rot, rnd, seed = [v for v in self.variants if v[0] == label][0]
        R, D = mx.ROTATE[rot], mx.ROUND[rnd]
        seeds = self._seeds(seed)
        calls = []

        def dual(L, k):
            x, bufs = L["src"][k], L["bufs"]
            c1, s1, d1 = bufs[k, 1]
            c0, s0, d0 = bufs[k, 0]
            return ("quant_dual", {"linear": L["name"], "tensor": k, "elems": x.numel()},
                    lib.mx_quantize_dual,
                    (x.data_ptr(), x.shape[0], x.shape[1], x.stride(0), 32, R, D, seeds[k][0],
                     seeds[k][1], c1.data_ptr(), s1.data_ptr(), c0.data_ptr(), s0.data_ptr(),
                     ctypes.byref(d1), ctypes.byref(d0), st))

        def gemm_info(ls, op):
            C = ls[0]["outs"][op]
            m, n = C.shape
            L = ls[0]
            k = self.T if op == "wgrad" else (L["in"] if op == "fprop" else L["out"])
            return {"linear": "+".join(x["name"] for x in ls), "op": op, "M": m, "N": n, "K": k,
                    "count": len(ls)}

        def gemm(L, op, a, b, odt):
            C = L["outs"][op]
            bufs = L["bufs"]
            return ("gemm_" + odt, gemm_info([L], op),
                    lib.mx_linear, (mx.OPS[op], ctypes.byref(bufs[a][2]),
                                    ctypes.byref(bufs[b][2]), C.data_ptr(), C.stride(0),
                                    mx.OUT_DTYPES[odt], st))

        def gemm_group(grp, op, a, b, odt):
            ls = grp["lins"]
            cs = (ctypes.c_void_p * len(ls))(*[L["outs"][op].data_ptr() for L in ls])
            return ("gemm_" + odt, gemm_info(ls, op),
                    lib.mx_linear_batched, (mx.OPS[op], len(ls), grp["descs"][a],
                                            grp["descs"][b], cs, ls[0]["outs"][op].stride(0),
                                            mx.OUT_DTYPES[odt], st))

        if not per_op:
            # a shared X is quantized once, by the first linear that reads it;
            # the others' descriptors describe those buffers as that call does
            for L in self.lins:
                if L["x_of"]:
                    x = L["src"]["X"]
                    for axis, sd in ((1, seeds["X"][0]), (0, seeds["X"][1])):
                        c, s, d = L["bufs"]["X", axis]
                        d.codes, d.scales = c.data_ptr(), s.data_ptr()
                        d.rows, d.cols = x.shape
                        d.axis, d.block, d.rotate, d.round, d.seed = axis, 32, R, D, sd
                        d.format = mx.FORMATS["fp4_e2m1"]
            for grp in self.groups:
                for L in grp["lins"]:
                    for k in ("X", "W", "dY"):
                        if not (k == "X" and L["x_of"]):
                            calls.append(dual(L, k))
                names = tuple(L["name"] for L in grp["lins"])
                for op, a, b, odt in self.OPS:
                    if op in self.GROUPED_OPS.get(names, ()):
                        calls.append(gemm_group(grp, op, a, b, odt))
                    else:
                        calls.extend(gemm(L, op, a, b, odt) for L in grp["lins"])
        else:
            for L in self.lins:
                src, bufs = L["src"], L["bufs"]

                def qargs(k, axis):
                    x = src[k]
                    c, s, d = bufs[k, axis]
                    sd = seeds[k][0] if axis == 1 else seeds[k][1]
                    return (x.data_ptr(), x.shape[0], x.shape[1], x.stride(0), axis, 32, R, D, sd,
                            c.data_ptr(), s.data_ptr(), ctypes.byref(d), st)

                for op, a, b, odt in self.OPS:
                    if op == "fprop":
                        x, w = src["X"], src["W"]
                        cx, sx, dx = bufs["X", 1]
                        cw, sw, dw = bufs["W", 1]
                        calls.append(("quant_pair", {"linear": L["name"], "elems": x.numel() + w.numel()},
                                      lib.mx_quantize_pair,
                                      (x.data_ptr(), x.shape[0], x.stride(0), w.data_ptr(),
                                       w.shape[0], w.stride(0), x.shape[1], 32, R, D,
                                       seeds["X"][0], seeds["W"][0], cx.data_ptr(),
                                       sx.data_ptr(), cw.data_ptr(), sw.data_ptr(),
                                       ctypes.byref(dx), ctypes.byref(dw), st)))
                    else:
                        for k, axis in (a, b):
                            calls.append(("quant_single", {"linear": L["name"], "tensor": k,
                                                           "axis": axis,
                                                           "elems": src[k].numel()},
                                          lib.mx_quantize, qargs(k, axis)))
                    calls.append(gemm(L, op, a, b, odt))
        self.calls = calls
        self.plan = None if per_op else self._two_stream_plan(calls)
        return calls

    def _two_stream_plan(self, calls):
        """Per group: (its quantizer calls on the quantizer stream, its GEMM
        calls on the GEMM stream, quantized event, GEMMs-done event)."""
        import torch
        qs, gs = (s.cuda_stream for s in self.side)
        plan = []
        for kind, _, fn, args in calls:
            if kind == "quant_dual":
                if not plan or plan[-1][1]:
                    plan.append(([], [], torch.cuda.Event(), torch.cuda.Event()))
                plan[-1][0].append((fn, tuple(args[:-1]) + (qs,)))
            else:
                plan[-1][1].append((fn, tuple(args[:-1]) + (gs,)))
        self._gemms_recorded = False
        return plan

    def step(self, i=0):
        if self.plan is None or not self.overlap:
            for kind, _, fn, args in self.calls:
                if fn(*args):
                    raise RuntimeError(f"library call {fn.__name__} failed")
            return
        import torch
        qs, gs = self.side
        cur = torch.cuda.current_stream()
        qs.wait_stream(cur)
        gs.wait_stream(cur)
        if not self._gemms_recorded:
            qs.wait_stream(gs)     # GEMMs of an earlier plan may still read the operands
        for duals, gemms, quantized, gemms_done in self.plan:
            if self._gemms_recorded:
                qs.wait_event(gemms_done)
            for fn, args in duals:
                if fn(*args):
                    raise RuntimeError(f"library call {fn.__name__} failed")
            quantized.record(qs)
            gs.wait_event(quantized)
            for fn, args in gemms:
                if fn(*args):
                    raise RuntimeError(f"library call {fn.__name__} failed")
            gemms_done.record(gs)
        self._gemms_recorded = True

    def join(self):
        """Make the current stream wait for everything the steps launched."""
        import torch
        cur = torch.cuda.current_stream()
        for s in self.side:
            cur.wait_stream(s)

    def instrumented(self, steps):
        """`steps` steps with a HIP event before every launch and after the
        last: per-launch durations (ms), summed over the steps, in launch
        order, and the instrumented ms per step."""
        import torch
        n = len(self.calls)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        tot = [0.0] * n
        step_ms = 0.0
        for s in range(steps):
            for j, (kind, _, fn, args) in enumerate(self.calls):
                ev[j].record()
                if fn(*args):
                    raise RuntimeError("library call failed")
            ev[n].record()
            torch.cuda.synchronize()
            for j in range(n):
                tot[j] += ev[j].elapsed_time(ev[j + 1])
            step_ms += ev[0].elapsed_time(ev[n])
        return [t / steps for t in tot], step_ms / steps


def gemm_bytes(M, N, K, out_bytes, code_bytes=0.5):
    return (M + N) * K * (code_bytes + 1.0 / 32) + M * N * out_bytes


def block_bench(mx, args):
    """The headline: the block under every variant (dual quantizer), the
    det. Hadamard one instrumented per launch."""
    br = BlockRunner(mx, args.tokens)
    flops = br.flops()
    labels = [v[0] for v in br.variants]
    head = args.variant or labels[0]
    res = {}
    for label in [head] + [lb for lb in labels if lb != head]:
        br.build(label)
        ms, wall = timed(br.step, args.steps, args.warmup, join=br.join)
        res[label] = {"ms_per_step": ms, "wall_ms_per_step": wall,
                      "tflops": flops / (ms * 1e-3) / 1e12}
        print(f"[bench] block {label}: {ms:.3f} ms/step, {res[label]['tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
    # the headline variant with every launch in order on one stream
    calls = br.build(head)
    br.overlap = False
    ms, _ = timed(br.step, args.steps, args.warmup)
    res[head]["serial_ms_per_step"] = ms
    print(f"[bench] block {head}, one stream: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    # per-launch split of the headline variant (in order, one stream)
    per_launch, inst_ms = br.instrumented(args.steps)
    br.overlap = True
    split = {}
    per_op = {}
    for (kind, info, _, _), ms in zip(calls, per_launch):
        d = split.setdefault(kind, {"us": 0.0, "launches": 0, "flops": 0.0, "bytes": 0.0})
        d["us"] += ms * 1e3
        d["launches"] += 1
        if kind.startswith("gemm"):
            f = 2.0 * info["M"] * info["N"] * info["K"] * info["count"]
            d["flops"] += f
            d["bytes"] += info["count"] * gemm_bytes(info["M"], info["N"], info["K"],
                                                     2 if kind == "gemm_bf16" else 4)
            per_op[f"{info['linear']}/{info['op']}"] = {
                "M": info["M"], "N": info["N"], "K": info["K"], "gemms": info["count"],
                "us": round(ms * 1e3, 2), "tflops": round(f / (ms * 1e-3) / 1e12, 1)}
        else:
            d["bytes"] += info["elems"] * (2 + 2 * (0.5 + 1.0 / 32))
    return br, res, head, split, per_op, inst_ms


def cpu_baseline_block(br, seed, reps):
    """The oracle as it stands, on the host cores, on a bounded sample of the
    block: the k_proj linear's whole training-step work (X 16384x4096,
    W 1024x4096, dY 16384x1024 each quantized along both axes with the
    det. Hadamard, then the three fp64 GEMMs of the dequantized operands),
    `reps` times; the value is that sample's flops over its mean time."""
    import oracle
    t = br.host["k_proj"]
    X, W, dY = t["X"], t["W"], t["dY"]
    sa = seed & 0xFFFFFFFF
    sb = sa | (1 << 32)
    T, n_in = X.shape
    n_out = W.shape[0]
    flops = 3 * 2.0 * T * n_in * n_out
    t_q = t_g = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        q = {("X", 1): oracle.quantize_ref(X, 1, seed=sa), ("X", 0): oracle.quantize_ref(X, 0, seed=sb),
             ("W", 1): oracle.quantize_ref(W, 1, seed=sb), ("W", 0): oracle.quantize_ref(W, 0, seed=sb),
             ("dY", 1): oracle.quantize_ref(dY, 1, seed=sa),
             ("dY", 0): oracle.quantize_ref(dY, 0, seed=sa)}
        t1 = time.perf_counter()
        oracle.mx_gemm_ref(q["X", 1], q["W", 1])
        oracle.mx_gemm_ref(q["dY", 1], q["W", 0])
        oracle.mx_gemm_ref(q["dY", 0], q["X", 0])
        t2 = time.perf_counter()
        t_q += t1 - t0
        t_g += t2 - t1
        del q
    per = (t_q + t_g) / reps
    return {
        "value": round(flops / per / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": _blas_threads() or len(os.sched_getaffinity(0)),
        "affinity_cores": len(os.sched_getaffinity(0)),
        "quantizer_threads": 1,
        "kind": "oracle",
        "sample": (f"k_proj linear of the block (T={T}, in={n_in}, out={n_out}), det. Hadamard: "
                   f"oracle quantization of X, W, dY along both axes (NumPy, 1 thread, "
                   f"{t_q / reps:.2f} s) + the three fp64 GEMMs of the dequantized operands "
                   f"(BLAS, {t_g / reps:.2f} s), x{reps}; {flops / 1e9:.1f} GFLOP of the "
                   f"block's {br.flops() / 1e9:.1f}"),
        "sample_seconds": round(t_q + t_g, 2),
    }


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()
                    if p.get("user_api") == "blas"] or [1])
    except Exception:
        return None


# --------------------------------------------------- one GEMM of the triple
class Runner:
    """Pre-marshalled C-ABI calls for one single-GEMM workload variant (no
    torch calls in the timed loop). The inputs are replicated so that
    consecutive steps read different copies (min_bytes of sources)."""

    def __init__(self, mx, w, variant, tensors=None, min_bytes=2 * LLC_BYTES, device="cuda",
                 fmt="fp4_e2m1"):
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
        a0, b0 = _dev_bf16(a_src, device), _dev_bf16(b_src, device)
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

    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def code_bytes(self):
        return 1.0 if self.fmt == "fp8_e4m3" else 0.5

    def quant_bytes(self, shape):
        return shape[0] * shape[1] * (2 + self.code_bytes() + 1.0 / 32)

    def gemm_bytes(self):
        ob = 4 if self.out_dtype == "f32" else 2
        return gemm_bytes(self.M, self.N, self.K, ob, self.code_bytes())


def measure(r, steps, warmup=0):
    """The timed region: `steps` whole steps (quantize A, quantize B, GEMM)
    back to back after the settle phase and `warmup` more steps. Then each
    kernel alone, settled and back to back, for its average launch
    duration (events between the kernels of a step would add gaps)."""
    ms, wall = timed(r.step, steps, warmup)
    n = max(steps, 10)
    t_qa = timed(r.quant_a, n)[0]
    t_qb = timed(r.quant_b, n)[0]
    t_g = timed(r.gemm, n)[0]
    flops = r.flops()
    return {
        "ms_per_step": ms,
        "wall_ms_per_step": wall,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "t_quant_a_us": t_qa * 1e3,
        "t_quant_b_us": t_qb * 1e3,
        "t_gemm_us": t_g * 1e3,
        "gemm_tflops": flops / (t_g * 1e-3) / 1e12,
        "quant_a_gbs": r.quant_bytes(r.a_shape) / (t_qa * 1e-3) / 1e9,
        "quant_b_gbs": r.quant_bytes(r.b_shape) / (t_qb * 1e-3) / 1e9,
    }


def cpu_baseline(r, reps):
    """The oracle as it stands, on the host cores: the whole single-GEMM
    workload (quantize both operands, fp64 GEMM of the dequantized
    operands), `reps` times; the value is the workload's flops over the mean
    time."""
    import oracle
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
        "cores": _blas_threads() or len(os.sched_getaffinity(0)),
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


def single_workload_line(mx, args, w, variant):
    """The bench line of a single-GEMM workload (--workload other than
    block)."""
    fp8 = args.format == "fp8_e4m3"
    r = Runner(mx, w, variant, fmt=args.format)
    res = measure(r, args.steps, args.warmup)
    t_dom = res["t_gemm_us"]
    gemm_ach = r.flops() / (t_dom * 1e-6) / 1e12
    qa_ach = res["quant_a_gbs"]
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_FP4_TFLOPS
    gemm_src, gemm_prof = (GEMM_E4M3_SRC, GEMM_E4M3_TRAFFIC) if fp8 else (GEMM_SRC, GEMM_TRAFFIC)
    quant_prof = QUANT_E4M3_TRAFFIC if fp8 else QUANT_TRAFFIC
    elem = "fp8_e4m3" if fp8 else "fp4_e2m1"
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
        "dtype": elem,
        "out_dtype": w.out_dtype,
        "data": "synthetic (seeded PCG64; Llama-3.1-8B layer shapes, no real weights or data)",
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
        "per_kernel_us_alone": {k: round(res[k], 2) for k in ("t_quant_a_us", "t_quant_b_us",
                                                             "t_gemm_us")},
        "quant_b_gbs": round(res["quant_b_gbs"], 1),
        "gemm_only_tflops": round(res["gemm_tflops"], 2),
    }
    return r, res, out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(sharding across GPUs is not implemented)"}))
        sys.exit(2)
    import torch

    import mxfp4_microscaled_precision_amd as mx
    from datagen import WORKLOADS, workload_tensors
    global WORKLOADS_REF
    WORKLOADS_REF = WORKLOADS

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    mx.load_library()
    print(f"[bench] workload {args.workload}", file=sys.stderr, flush=True)

    if args.workload == "block":
        br, res, head, split, per_op, inst_ms = block_bench(mx, args)
        h = res[head]
        flops = br.flops()
        dom = split["gemm_bf16"]
        dom_ach = dom["flops"] / (dom["us"] * 1e-6) / 1e12
        q = split["quant_dual"]
        q_ach = q["bytes"] / (q["us"] * 1e-6) / 1e9
        g_all_us = split["gemm_bf16"]["us"] + split["gemm_f32"]["us"]
        g_all_fl = split["gemm_bf16"]["flops"] + split["gemm_f32"]["flops"]
        out = {
            "metric": METRIC,
            "value": round(h["tflops"], 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(h["ms_per_step"], 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "fp4_e2m1",
            "out_dtype": "bf16 (Fprop, Dgrad), f32 (Wgrad); fp32 accumulation",
            "data": ("synthetic (seeded PCG64, chunked streams; Llama-3.1-8B block shapes, "
                     "no real weights or data)"),
            "config": {
                "workload": (f"Llama-3.1-8B block T={br.T}: 7 linears x Fprop/Dgrad/Wgrad "
                             f"(21 MXFP4 GEMMs; k/v ops and gate/up Dgrad and Wgrad as grouped "
                             f"launches), {head}; q/k/v read one input activation and "
                             f"gate/up another, as in the model; each distinct X, W and dY "
                             f"quantized once into both orientations; quantizations and GEMMs "
                             f"on two streams, each group's GEMMs after its quantizations"),
                "tokens": br.T, "variant": head, "gemms": 21,
                "gflop_per_step": round(flops / 1e9, 1),
                "launches_per_step": len(br.calls),
            },
            "pct_mfma_peak": round(100.0 * h["tflops"] / PEAK_FP4_TFLOPS, 2),
            "roofline": {
                "kernel": "gemm_tiled_kernel<1, 0, false|true> (MXFP4 GEMM, bf16 out: the 14 "
                          "Fprop and Dgrad GEMMs of a step in 11 launches, 8 single and 3 "
                          "grouped: k+v Fprop and Dgrad, gate+up Dgrad)",
                "bound": "mfma",
                "achieved": round(dom_ach, 2),
                "peak": PEAK_FP4_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(dom_ach / PEAK_FP4_TFLOPS, 4),
                "traffic": recorded_traffic(GEMM_SRC, BLOCK_GEMM_TRAFFIC),
                "launches": dom["launches"],
                "avg_gflop_per_launch": round(dom["flops"] / dom["launches"] / 1e9, 3),
                "avg_us_per_launch": round(dom["us"] / dom["launches"], 2),
                "algorithmic_bytes_per_launch": round(dom["bytes"] / dom["launches"]),
                # measured limiter: the shader clock under this load (in-kernel
                # s_memtime over s_memrealtime on a timing build of the same kernel)
                "limited_by": "clock under load: 1.6-1.7 GHz against the 2.4 GHz of the peak; "
                              "in cycles within 8-10% of an MFMA-only build (profiles/"
                              "gemm_fprop_q_proj_mfma_counters.md)",
            },
            "quant_roofline": {
                "kernel": "quant_dual_kernel (both orientations from one read)",
                "bound": "hbm",
                "achieved": round(q_ach, 1),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(q_ach / PEAK_HBM_GBS, 4),
                "traffic": recorded_traffic(QUANT_SRC, BLOCK_QUANT_TRAFFIC),
                "avg_us_per_launch": round(q["us"] / q["launches"], 2),
                "algorithmic_bytes_per_launch": round(q["bytes"] / q["launches"]),
                # measured limiter (rocprofv3 SQ_INSTS_VALU / SQ_WAVES of the H32 + RNE
                # instance): vector-instruction issue, not HBM
                "limited_by": "VALU issue: 326 VALU instructions per wave (4 cycles each on a "
                              "16-lane SIMD), issued for 82-93% of the launch "
                              "(profiles/quant_dual_block_t16384_counters.md)",
            },
            "gemm_all": {"tflops": round(g_all_fl / (g_all_us * 1e-6) / 1e12, 2),
                         "frac": round(g_all_fl / (g_all_us * 1e-6) / 1e12 / PEAK_FP4_TFLOPS, 4)},
            # the step's time split over the kernel classes in proportion to
            # their event-timed durations in the one-stream pass (so the split
            # sums to ms_per_step); the raw event-timed sums are
            # per_kernel_us_events: an event between every two launches adds a
            # few us to each
            "per_kernel_us": {k: round(v["us"] * h["ms_per_step"] / inst_ms, 1)
                              for k, v in split.items()},
            "per_kernel_us_events": {k: round(v["us"], 1) for k, v in split.items()},
            "instrumented_ms_per_step": round(inst_ms, 5),
            # the same launches in order on one stream (no overlap between a
            # GEMM's last tiles and the next quantizer)
            "serial_ms_per_step": round(h["serial_ms_per_step"], 5),
            "per_op": per_op,
            "variants": {lb: {"ms_per_step": round(v["ms_per_step"], 5),
                              "tflops": round(v["tflops"], 2),
                              "pct_mfma_peak": round(100 * v["tflops"] / PEAK_FP4_TFLOPS, 2)}
                         for lb, v in res.items()},
        }
        if args.all:
            per = {}
            for label in [v[0] for v in br.variants]:
                br.build(label, per_op=True)
                ms, _ = timed(br.step, args.steps, args.warmup)
                per[label] = {"ms_per_step": round(ms, 5),
                              "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
                print(f"[bench] block per-op {label}: {ms:.3f} ms", file=sys.stderr, flush=True)
            out["per_op_quantization"] = per
        if not args.no_secondary:
            w = WORKLOADS["fprop_q_proj"]
            r, sres, _ = single_workload_line(mx, args, w, "det_hadamard")
            out["secondary"] = {"fprop_q_proj": {
                "tflops": round(sres["tflops"], 2), "ms_per_step": round(sres["ms_per_step"], 5),
                "gemm_us_alone": round(sres["t_gemm_us"], 2),
                "gemm_frac": round(sres["gemm_tflops"] / PEAK_FP4_TFLOPS, 4),
                "quant_a_gbs": round(sres["quant_a_gbs"], 1)}}
            out["secondary"]["fp8_comparator"] = fp8_comparator(mx, w, "det_hadamard",
                                                                max(10, args.steps), sres)
            del r
            wg = WORKLOADS["wgrad_gate_proj"]
            out["secondary"]["wgrad_gate_proj_quant_error"] = quant_error(
                mx, wg, [v[0] for v in wg.variants])
            print(f"[bench] quant error {out['secondary']['wgrad_gate_proj_quant_error']}",
                  file=sys.stderr, flush=True)
        if args.all:
            add_all(mx, args, out, skip=None)
        if args.structural or args.all:
            out["structural_error"] = structural_error(mx)
            print("[bench] structural error done", file=sys.stderr, flush=True)
        copy_calibration(args, out)
        if not args.no_cpu_baseline:
            print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
            out["cpu_baseline"] = cpu_baseline_block(br, 0, args.cpu_reps)
        print(json.dumps(out), flush=True)
        return

    w = WORKLOADS[args.workload]
    variant = args.variant or w.variants[0][0]
    r, res, out = single_workload_line(mx, args, w, variant)
    if args.format != "fp8_e4m3" and r.rnd == "rne":
        out["fp8_comparator"] = fp8_comparator(mx, w, variant, max(10, args.steps), res)
    if args.all:
        add_all(mx, args, out, skip=(w.name, variant))
    if args.structural or args.all:
        out["structural_error"] = structural_error(mx)
    copy_calibration(args, out)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(r, args.cpu_reps)
    print(json.dumps(out), flush=True)


def copy_calibration(args, out):
    import torch
    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n


def add_all(mx, args, out, skip):
    """--all: every single-GEMM workload and variant, the dual quantizer
    alone, and the quantization error of the Wgrad gate/up workload."""
    from datagen import WORKLOADS, workload_tensors
    extra = {}
    for name, wl in WORKLOADS.items():
        if name == "tiny_wgrad":
            continue
        t = workload_tensors(wl)
        for v in wl.variants:
            if skip is not None and (name, v[0]) == skip:
                continue
            rr = Runner(mx, wl, v[0], tensors=t)
            m = measure(rr, max(10, args.steps))
            extra[f"{name}/{v[0]}"] = {k: round(val, 3) for k, val in m.items()}
            print(f"[bench] {name}/{v[0]}: {m['tflops']:.1f} TFLOP/s", file=sys.stderr,
                  flush=True)
            del rr
    out["other_workloads"] = extra
    out["dual_quantizer"] = dual_quant_bench(mx, max(10, args.steps))
    print(f"[bench] dual quantizer {out['dual_quantizer']}", file=sys.stderr, flush=True)
    if "secondary" not in out:
        wg = WORKLOADS["wgrad_gate_proj"]
        out["wgrad_gate_proj_quant_error"] = quant_error(mx, wg, [v[0] for v in wg.variants])


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
        "per_kernel_us_alone": {k: round(m8[k], 2) for k in ("t_quant_a_us", "t_quant_b_us",
                                                            "t_gemm_us")},
        "gemm_tflops": round(fl / (m8["t_gemm_us"] * 1e-6) / 1e12, 2),
        "gemm_frac_fp8_peak": round(fl / (m8["t_gemm_us"] * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
        "quant_a_gbs": round(m8["quant_a_gbs"], 1),
        "fp4_over_fp8_step_speed": round(m8["ms_per_step"] / fp4_res["ms_per_step"], 3),
        "fp4_over_fp8_gemm_speed": round(m8["t_gemm_us"] / fp4_res["t_gemm_us"], 3),
    }
    del r8
    return out


def quant_error(mx, wl, variants):
    """Quantization error of one GEMM's operands and output (the Wgrad
    gate/up workload, rotation off and on).

    Operand level: mean((deq - y)^2) over each operand, where deq is the
    library's dequantization (mx_dequantize) of the quantized operand and y
    the rotated source, y = R x with R the same block rotation applied in
    fp32 by a torch matmul with the 32 x 32 matrix (measurement only; R is
    orthonormal, so this equals the error in the source's own domain up to
    fp32 rounding).
    Output level: the fp32 MXFP4 result against the fp32 product of the
    unquantized bf16 operands (torch.matmul), as mean squared error and
    relative Frobenius error."""
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
        entry = {"output_mse": float((d * d).mean()),
                 "rel_fro": float(d.norm() / ref.double().norm())}
        del d, ref, c
        for name, q, xs, ax in (("A", rr.qa[0], rr.A[0], ax_a), ("B", rr.qb[0], rr.B[0], ax_b)):
            deq = mx.dequantize(q)                          # the source's shape, fp32
            x = xs.float()
            if ax == 0:                                     # reduction along the rows
                deq, x = deq.t().contiguous(), x.t().contiguous()
            y = rotate_rows(x, rr.rot)                      # [MN, K], rotated along K
            e = (deq - y).double()
            entry[f"operand_{name}_mse"] = float((e * e).mean())
            entry[f"operand_{name}_rel_fro"] = float(e.norm() / y.double().norm())
            del deq, x, y, e
        res[label] = entry
        del rr, a, b
        torch.cuda.empty_cache()
    return res


def rotate_rows(x, rot):
    """y = x with every 32-element block of each row multiplied by the
    rotation R = H / sqrt(32) (H the Sylvester Hadamard matrix), in fp32 on
    the GPU with torch (measurement only); rot 'none' returns x."""
    import torch
    if rot == "none":
        return x
    if rot != "hadamard":
        raise ValueError(rot)
    i = torch.arange(32, device=x.device)
    pc = torch.zeros((32, 32), dtype=torch.int64, device=x.device)
    v = i[:, None] & i[None, :]
    for b in range(5):
        pc += (v >> b) & 1
    H = torch.where(pc % 2 == 0, 1.0, -1.0).to(torch.float32) / math.sqrt(32.0)
    m, k = x.shape
    return torch.matmul(x.reshape(m * (k // 32), 32), H.t().contiguous()).reshape(m, k)


def dual_quant_bench(mx, steps):
    """The dual-output quantizer against the two single-orientation launches it
    replaces, on the Fprop activation X and the Wgrad gradient dY (H32, RNE).
    Algorithmic bytes: 2 B read + 2 x (0.5 + 1/32) B written per element."""
    import torch
    from datagen import workload_tensors
    res = {}
    for wname, tname in (("fprop_q_proj", "X"), ("wgrad_gate_proj", "dY")):
        src = workload_tensors(WORKLOADS_REF[wname])[tname]
        x = _dev_bf16(src)
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

        t_d = timed(dual, steps)[0] * 1e3
        t_1 = timed(single(1), steps)[0] * 1e3
        t_0 = timed(single(0), steps)[0] * 1e3
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


def structural_inputs(T, n_out, n_in, data_seed=3):
    """The harness's fixed tensors (bf16 bits): dY [T, n_out] = 1e-4 t_3 and
    X [T, n_in] ~ N(0, 1), the Wgrad gate/up distributions."""
    import numpy as np
    from datagen import normal_bf16, student_t_bf16
    rng = np.random.Generator(np.random.PCG64(data_seed))
    dY = student_t_bf16(rng, (T, n_out), 3.0, 1e-4)
    X = normal_bf16(rng, (T, n_in), 1.0)
    return dY, X


def structural_step_seed(k, reseed):
    """Seed of step k (1-based): k for the randomized variants, 0 otherwise;
    operand A (dY) takes it, operand B (X) takes it | 1 << 32."""
    return k if reseed else 0


def structural_error(mx, T=8192, n_out=2048, n_in=1024, steps=64, data_seed=3, keep_steps=0):
    """Error of Wgrad repeated over `steps` steps on fixed tensors.

    dY and X (structural_inputs) stay fixed; step k computes
    dW_k = dY^T X through the MXFP4 path (both operands quantized along T),
    with seed k for the randomized variants (random signs, stochastic
    rounding) and the same deterministic rotation every step otherwise. For
    K = 1, 2, 4, ... the relative Frobenius error of the K-step mean against
    the exact product of the bf16 operands is reported, with the single-step
    error: a fixed error pattern keeps the mean's error at the single-step
    value, a pattern that changes from step to step lets it fall. The
    reference product is formed in fp64 on the host from the bf16 values
    (exact up to fp64 summation). keep_steps > 0 also returns, under
    "_steps", the first keep_steps steps' quantized operands and dW (host
    copies) of every variant."""
    import numpy as np
    import torch
    dY, X = structural_inputs(T, n_out, n_in, data_seed)
    dYd, Xd = _dev_bf16(dY), _dev_bf16(X)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    ref = f(dY).T @ f(X)
    ref_norm = float(np.linalg.norm(ref))
    ref_d = torch.from_numpy(ref).to("cuda")
    out = {"shape": {"T": T, "out": n_out, "in": n_in}, "steps": steps, "variants": {}}
    kept = {}
    Ks = [k for k in (1, 2, 4, 8, 16, 32, 64, 128, 256) if k <= steps]
    for label, rot, rnd, reseed in STRUCTURAL_VARIANTS:
        acc = torch.zeros_like(ref_d)
        single = []
        curve = {}
        for k in range(1, steps + 1):
            seed = structural_step_seed(k, reseed)
            qa = mx.quantize(dYd, 0, rot, rnd, seed=seed)
            qb = mx.quantize(Xd, 0, rot, rnd, seed=seed | (1 << 32))
            c = mx.linear("wgrad", qa, qb, "f32")
            acc += c.double()
            if k <= keep_steps:
                kept.setdefault(label, []).append({
                    "seed": seed, "a_codes": qa.codes.cpu().numpy(),
                    "a_scales": qa.scales.cpu().numpy(), "b_codes": qb.codes.cpu().numpy(),
                    "b_scales": qb.scales.cpu().numpy(), "dW": c.cpu().numpy()})
            if k <= 4:
                single.append(((c.double() - ref_d).norm() / ref_norm).item())
            if k in Ks:
                curve[k] = ((acc / k - ref_d).norm() / ref_norm).item()
        out["variants"][label] = {
            "rotate": rot, "round": rnd, "new_seed_per_step": reseed,
            "single_step_rel_err": [round(v, 6) for v in single],
            "mean_rel_err": {str(k): round(v, 6) for k, v in curve.items()},
            "mean_over_single": round(curve[Ks[-1]] / single[0], 4)}
    if keep_steps:
        out["_steps"] = kept
    return out


if __name__ == "__main__":
    main()
