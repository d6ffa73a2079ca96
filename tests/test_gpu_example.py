"""The end-to-end example of the package runs and its outputs hang
together: the copied-out bf16 weights are the bf16 of the updated master
(the step's fused copy-in followed by the copy-out), the layout is the
oracle's, and the clipping coefficient follows the norm."""
import math

import torch
import pytest

import oracle
from gpu_harness import log
from sharded_state_raggedshard_amd import example

pytestmark = pytest.mark.gpu


def test_example_runs_and_outputs_agree():
    log("example")
    r = example.main(steps=3)
    plan = r["plan"]
    L = oracle.Layout(plan.specs, plan.m, 16)
    assert r["S"] == L.S and plan.offsets == L.offsets
    assert r["padding"] == [0, 0]
    for i, s in enumerate(plan.specs):
        master = r["theta"][plan.pos[i]:plan.pos[i] + s.numel]
        assert torch.equal(r["weights"][i], master.to(torch.bfloat16).float())
    assert r["grad_norm"] > 0.0
    assert math.isclose(r["clip"], min(1.0, 1.0 / (r["grad_norm"] + 1e-6)), rel_tol=1e-6)
    plan.free()
