"""Test-side helpers around the oracle: quantize selected operand rows of a
large source in parallel slices (the oracle itself is unchanged; each slice
is one quantize_ref call with global row / column indices, so random signs
and stochastic rounding draw the same Philox words as for the whole
tensor)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def oracle_rows(src, axis, idx, rot, rnd, seed, chunk=256, fmt="fp4_e2m1"):
    """QuantRef of operand rows `idx` of src quantized along `axis`: for
    axis 1 the operand rows are source rows, for axis 0 source columns."""
    idx = np.asarray(idx, dtype=np.int64)

    def part(lo):
        sel = idx[lo:lo + chunk]
        if axis == 1:
            return oracle.quantize_ref(src[sel], 1, rotate=rot, rounding=rnd, seed=seed,
                                       row_index=sel, total_cols=src.shape[1], fmt=fmt)
        return oracle.quantize_ref(np.ascontiguousarray(src[:, sel]), 0, rotate=rot,
                                   rounding=rnd, seed=seed, col_index=sel,
                                   total_cols=src.shape[1], fmt=fmt)

    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as pool:
        parts = list(pool.map(part, range(0, len(idx), chunk)))
    return oracle.QuantRef(np.concatenate([r.codes for r in parts]),
                           np.concatenate([r.scales for r in parts]),
                           np.empty((0, 0), np.float32), axis, parts[0].fmt)


def oracle_operand(src, axis, rot, rnd, seed, fmt="fp4_e2m1"):
    """The oracle's whole operand [MN, K]."""
    mn = src.shape[0] if axis == 1 else src.shape[1]
    return oracle_rows(src, axis, np.arange(mn), rot, rnd, seed, fmt=fmt)
