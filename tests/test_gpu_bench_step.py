"""The benchmark's block step computes what the library's single calls do.

At a small token count, after steps of bench.BlockRunner -- each distinct X,
W and dY quantized once into both orientations (q, k and v share one input
activation, gate and up another, so the followers' descriptors describe the
leader's buffers), k/v and gate/up ops as grouped launches, quantizations and
GEMMs on two streams -- every linear's Fprop, Dgrad and Wgrad output equals,
bit for bit, separate mx_quantize and mx_linear calls on the same tensors
with the same seeds by role; so does the same step in order on one stream.
The single calls are checked against the oracle by the other GPU tests (the
three GEMMs of every linear: 36Kr article "Neue Studie von AMD durchbricht
die bestehende Erkenntnis ...", section "Fehlerdiagnoseexperiment").
"""
import pytest
import torch

from datagen import BLOCK_VARIANTS

pytestmark = pytest.mark.gpu

TOKENS = 512


@pytest.fixture(scope="module")
def runner(mx):
    import bench
    return bench.BlockRunner(mx, tokens=TOKENS, keep_host=())


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _single_calls(mx, L, rot, rnd, seed):
    sa = seed & 0xFFFFFFFF
    sb = sa | (1 << 32)
    X, W, dY = L["src"]["X"], L["src"]["W"], L["src"]["dY"]

    def q(x, axis, s):
        return mx.quantize(x, axis, rot, rnd, seed=s)

    return {"fprop": mx.linear("fprop", q(X, 1, sa), q(W, 1, sb), "bf16"),
            "dgrad": mx.linear("dgrad", q(dY, 1, sa), q(W, 0, sb), "bf16"),
            "wgrad": mx.linear("wgrad", q(dY, 0, sa), q(X, 0, sb), "f32")}


@pytest.mark.parametrize("label", [v[0] for v in BLOCK_VARIANTS])
def test_block_step_equals_single_calls(mx, runner, label):
    br = runner
    _, rot, rnd, seed = [v for v in br.variants if v[0] == label][0]
    br.build(label)
    assert len(br.calls) == 34                      # 18 quantizations, 16 GEMM calls
    shared = [L["name"] for L in br.lins if L["x_of"]]
    assert shared == ["k_proj", "v_proj", "up_proj"]
    ref = {L["name"]: _single_calls(mx, L, rot, rnd, seed) for L in br.lins}
    try:
        for overlap in (True, False):
            for L in br.lins:
                for o in L["outs"].values():
                    o.fill_(float("nan"))
            br.overlap = overlap
            br.step(0)
            br.step(1)                              # the second waits on the first's GEMMs
            br.join()
            torch.cuda.synchronize()
            for L in br.lins:
                for op, c in ref[L["name"]].items():
                    assert torch.equal(_bits(L["outs"][op]), _bits(c)), (label, overlap,
                                                                        L["name"], op)
    finally:
        br.overlap = True
