"""The seeded input generators (no part of the method): the Llama block's
linears that read one input activation in the model get the same X array."""
import dataclasses

import numpy as np
import pytest

from datagen import (BLOCK_INPUT_OF, LLAMA_BLOCK_LINEARS, WORKLOADS, block_workloads,
                     workload_tensors)


def test_block_inputs_are_shared_as_in_the_model():
    wls = {w.name: w for w in block_workloads(64)}
    t = {lin.name: workload_tensors(wls[f"block_{lin.name}_fprop"]) for lin in LLAMA_BLOCK_LINEARS}
    assert BLOCK_INPUT_OF == {"k_proj": "q_proj", "v_proj": "q_proj", "up_proj": "gate_proj"}
    for follower, leader in BLOCK_INPUT_OF.items():
        assert np.array_equal(t[follower]["X"], t[leader]["X"])
    # distinct inputs elsewhere, and every linear's own W and dY
    assert not np.array_equal(t["q_proj"]["X"], t["o_proj"]["X"])
    assert not np.array_equal(t["gate_proj"]["X"][:, :4096], t["q_proj"]["X"])
    assert not np.array_equal(t["k_proj"]["W"], t["v_proj"]["W"])
    assert not np.array_equal(t["gate_proj"]["dY"], t["up_proj"]["dY"])
    # the three ops of a linear draw the same tensors
    for lin in LLAMA_BLOCK_LINEARS:
        for op in ("dgrad", "wgrad"):
            u = workload_tensors(wls[f"block_{lin.name}_{op}"])
            assert all(np.array_equal(u[k], t[lin.name][k]) for k in ("X", "W", "dY"))


def test_per_tensor_seed_needs_the_chunked_recipe():
    w = WORKLOADS["tiny_wgrad"]
    spec = w.tensors[0]
    bad = dataclasses.replace(w, tensors=((*spec, 7),) + w.tensors[1:])
    with pytest.raises(ValueError):
        workload_tensors(bad)
