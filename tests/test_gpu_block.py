"""GPU parity of the Llama-3.1-8B block at 16384 tokens against the oracle.

The 7 linears (q/k/v/o, gate/up, down) x Fprop/Dgrad/Wgrad under the three
variants of the block workload: deterministic 32-point Hadamard with nearest
rounding, random-sign Hadamard (seed 11) with nearest rounding, and no
rotation with stochastic rounding (seed 11) -- 36Kr article "Neue Studie von
AMD durchbricht die bestehende Erkenntnis ...", section
"Fehlerdiagnoseexperiment": the three GEMMs of every linear, the
deterministic rotation against its two randomized comparators.

Each linear's X (q, k and v read one input activation, gate and up another,
as in the model), W and dY are quantized as the benchmark's step quantizes
them: once into both orientations (mx_quantize_dual), seeds by role (A of an
op s, B s | 1 << 32). For every op:
  * the dual outputs equal the two single-orientation launches byte for byte;
  * operand rows -- all rows of the first and the last 256-row panel and 16
    sampled ones, of A and of B -- are bit-exact against the oracle
    (quantize_ref on the gathered rows with their global indices, so random
    signs and stochastic rounding draw the same Philox words);
  * the output on those rows x columns (four whole 256 x 256 tiles, the
    corners of C, and the sampled rows and columns) lies within the
    per-element bound |C - C_ref| <= (K/32 + 4) 2^-23 sum_k |a b| and within
    1e-5 relative Frobenius error of the fp64 oracle product; the bf16
    output (Fprop, Dgrad) equals the round-to-nearest-even of the fp32 one.
"""
import numpy as np
import pytest

import oracle
from datagen import LLAMA_BLOCK_LINEARS, block_workloads, workload_tensors
from gpu_util import host_u8, rel_fro, to_dev
from oracle_util import oracle_rows

pytestmark = pytest.mark.gpu

TOKENS = 16384
GEMM_TOL = 1e-5
WLS = block_workloads(TOKENS)
VARIANTS = WLS[0].variants
OPS = (("fprop", ("X", 1), ("W", 1), "bf16"), ("dgrad", ("dY", 1), ("W", 0), "bf16"),
       ("wgrad", ("dY", 0), ("X", 0), "f32"))

_cache = {}


def _tensors(li):
    """Host tensors of linear li (one linear cached at a time)."""
    if li not in _cache:
        _cache.clear()
        wl = [w for w in WLS if w.data_seed == 500 + li][0]
        _cache[li] = workload_tensors(wl)
    return _cache[li]


def _operand_rows(mn, rng):
    """The first and last 256-row panels and 16 sampled rows of an operand."""
    last = (mn - 1) // 256 * 256
    rows = np.r_[np.arange(256), np.arange(last, mn), rng.choice(mn, 16, replace=False)]
    return np.unique(rows)


def _gpu_rows(q, idx):
    """Codes [len(idx), K] and scales of the given operand rows, read from
    the device one 256-row panel at a time."""
    mnp, kp = oracle.padded_extents(q.mn, q.k)
    panel = 256 * kp // 2
    scales = oracle.untile_scales(host_u8(q.scales), q.mn, q.k)
    codes = np.empty((len(idx), q.k), np.uint8)
    cache = {}
    for i, m in enumerate(idx):
        p = int(m) // 256
        if p not in cache:
            cache[p] = oracle.untile_codes(host_u8(q.codes[p * panel:(p + 1) * panel]), 256, q.k)
        codes[i] = cache[p][int(m) % 256]
    return codes, scales[idx]


def _elementwise_bound(ra, rb):
    """(K/32 + 4) 2^-23 sum_k |a b| per output element."""
    da = np.abs(oracle.dequantize_ref(ra.codes, ra.scales))
    db = np.abs(oracle.dequantize_ref(rb.codes, rb.scales))
    k = ra.codes.shape[1]
    return (k / 32 + 4) * 2.0 ** -23 * (da @ db.T)


@pytest.mark.parametrize("variant", [v[0] for v in VARIANTS])
@pytest.mark.parametrize("li", range(len(LLAMA_BLOCK_LINEARS)),
                         ids=[lin.name for lin in LLAMA_BLOCK_LINEARS])
def test_block_linear(mx, li, variant):
    import torch
    lin = LLAMA_BLOCK_LINEARS[li]
    print(f"[block] {lin.name} {variant}", flush=True)
    _, rot, rnd, seed = [v for v in VARIANTS if v[0] == variant][0]
    sa = seed & 0xFFFFFFFF
    sb = sa | (1 << 32)
    # seeds by role, as the benchmark step passes them: (axis 1, axis 0)
    seeds = {"X": (sa, sb), "W": (sb, sb), "dY": (sa, sa)}
    host = _tensors(li)
    dev = {k: to_dev(host[k]) for k in ("X", "W", "dY")}
    q = {}
    for k, x in dev.items():
        q1, q0 = mx.quantize_dual(x, rot, rnd, seed1=seeds[k][0], seed0=seeds[k][1])
        q[k, 1], q[k, 0] = q1, q0
        for axis, qq in ((1, q1), (0, q0)):
            s = mx.quantize(x, axis, rot, rnd, seed=seeds[k][1 - axis])
            assert torch.equal(s.codes, qq.codes) and torch.equal(s.scales, qq.scales), \
                f"{k} axis {axis}: dual != single launch"
            del s
    rng = np.random.default_rng(1000 * li + len(variant))
    for op, a, b, odt in OPS:
        qa, qb = q[a], q[b]
        ia, ib = _operand_rows(qa.mn, rng), _operand_rows(qb.mn, rng)
        ra = oracle_rows(host[a[0]], a[1], ia, rot, rnd, seeds[a[0]][1 - a[1]])
        rb = oracle_rows(host[b[0]], b[1], ib, rot, rnd, seeds[b[0]][1 - b[1]])
        for rq, qq, idx, name in ((ra, qa, ia, "A"), (rb, qb, ib, "B")):
            codes, scales = _gpu_rows(qq, idx)
            nb = np.count_nonzero(codes != rq.codes)
            ns = np.count_nonzero(scales != rq.scales)
            assert nb == 0 and ns == 0, f"{lin.name} {op} {name}: {nb} codes, {ns} scales differ"
        c32 = mx.linear(op, qa, qb, "f32")
        ta, tb = torch.from_numpy(ia).cuda(), torch.from_numpy(ib).cuda()
        got = c32[ta][:, tb].cpu().numpy().astype(np.float64)
        C_ref = oracle.mx_gemm_ref(ra, rb)
        err = rel_fro(got, C_ref)
        assert err <= GEMM_TOL, f"{lin.name} {op} {variant}: rel Frobenius {err:.3e}"
        bound = _elementwise_bound(ra, rb)
        over = np.count_nonzero(np.abs(got - C_ref) > bound)
        assert over == 0, f"{lin.name} {op} {variant}: {over} elements beyond the bound"
        if odt == "bf16":
            c16 = mx.linear(op, qa, qb, "bf16")
            g16 = c16[ta][:, tb].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(g16, oracle.bf16_round_ref(got.astype(np.float32))), \
                f"{lin.name} {op}: bf16 != RNE(fp32)"
            del c16
        del c32
        torch.cuda.synchronize()
    del q, dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pair", [("k_proj", "v_proj"), ("gate_proj", "up_proj")],
                         ids=["k_v", "gate_up"])
def test_block_grouped_gemms_equal_single(mx, pair):
    """The benchmark step runs k/v and gate/up as one grouped launch per op
    (mx_linear_batched). At full size, under the deterministic H32 variant,
    every grouped output equals the single launch's bit for bit; the single
    launches are the ones test_block_linear checks against the oracle."""
    import torch
    print(f"[block] grouped {pair}", flush=True)
    names = [lin.name for lin in LLAMA_BLOCK_LINEARS]
    _, rot, rnd, seed = VARIANTS[0]
    sa = seed & 0xFFFFFFFF
    sb = sa | (1 << 32)
    seeds = {"X": (sa, sb), "W": (sb, sb), "dY": (sa, sa)}
    q = []
    for name in pair:
        host = _tensors(names.index(name))
        qq = {}
        for k in ("X", "W", "dY"):
            q1, q0 = mx.quantize_dual(to_dev(host[k]), rot, rnd, seed1=seeds[k][0],
                                      seed0=seeds[k][1])
            qq[k, 1], qq[k, 0] = q1, q0
        q.append(qq)
    for op, a, b, odt in OPS:
        got = mx.linear_batched(op, [qq[a] for qq in q], [qq[b] for qq in q], odt)
        for i, qq in enumerate(q):
            ref = mx.linear(op, qq[a], qq[b], odt)
            torch.cuda.synchronize()
            assert torch.equal(got[i], ref), f"{pair[i]} {op}: grouped != single launch"
            del ref
        del got
    del q
    torch.cuda.empty_cache()
