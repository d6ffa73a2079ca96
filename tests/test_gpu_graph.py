"""The hot path under HIP graph capture: the per-step entry points launch
kernels only (no allocation, copy or memset), so a step captured once
replays.  Captured here: the allocation-free L2 norm, the clipping
coefficient and the step with bf16 and FP8 output, on a layout with split
blocks (cross-workgroup waits inside the graph in the one-launch modes, two
launches in the two-pass mode); and a distributed-Muon step.  Every replay
is compared bit for bit with the same sequence run eagerly on a twin of
the state, with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
from gpu_harness import DevState, host_state, log, make_plan
from synth import ROWS, TensorSpec
from test_gpu_step import CASES

pytestmark = pytest.mark.gpu


class _Run:
    def __init__(self, hs, L):
        self.d = DevState(hs, with_out=True)
        self.codes = torch.zeros(L.total, dtype=torch.uint8, device="cuda")
        self.scale8 = torch.zeros(L.n_blocks, dtype=torch.float32, device="cuda")
        self.sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
        self.clip = torch.zeros(1, dtype=torch.float32, device="cuda")

    def sequence(self, plan, t):
        d = self.d
        rs.rs_group_l2norm_static(plan.h, rs.RS_ALL, rs.RS_ALL, d.grad, rs.RS_BF16, self.sumsq)
        rs.rs_clip_coef(self.sumsq, 0.05, self.clip)
        rs.rs_adam8_step_fp8(plan.h, rs.RS_ALL, rs.RS_ALL, d.theta, d.grad, d.qm, d.qv, d.am,
                             d.av, self.codes, self.scale8, step=t, grad_scale=self.clip,
                             bf16_out=d.out)

    def snapshot(self):
        torch.cuda.synchronize()
        d = self.d
        return [x.cpu().numpy().copy() for x in (d.theta, d.qm, d.qv, d.am, d.av, d.out,
                                                 self.codes, self.scale8, self.sumsq, self.clip)]


@pytest.mark.parametrize("mode", [rs.RS_SPLIT_COOPERATIVE, rs.RS_SPLIT_ORDERED,
                                  rs.RS_SPLIT_TWO_PASS])
def test_captured_step_replays_like_eager_calls(mode):
    specs, m, g, sigma = CASES["mixed"]()
    log(f"graph capture mode={mode}")
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g, chunk=1024, mode=mode)
    hs = host_state(L, specs, seed=21, sigma=sigma, warm=True)
    eager, graphed = _Run(hs, L), _Run(hs, L)
    t = 9  # the step count is captured with the launch arguments
    expected = []
    for _ in range(3):
        eager.sequence(plan, t)
        expected.append(eager.snapshot())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed.sequence(plan, t)
    torch.cuda.synchronize()
    # capture ran nothing
    assert not graphed.codes.any() and not graphed.sumsq.any()
    other = torch.zeros(1 << 20, device="cuda")
    for k, exp in enumerate(expected):
        graph.replay()
        torch.cuda.synchronize()
        got = graphed.snapshot()
        for name, a, b in zip(("theta", "qm", "qv", "amax_m", "amax_v", "bf16", "fp8", "fp8 scale",
                               "sumsq", "clip"), got, exp):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (k, name)
        other.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
    assert float(expected[0][9][0]) < 1.0  # the clip coefficient is active
    if mode != rs.RS_SPLIT_TWO_PASS:
        rs.rs_plan_check_device(plan.h)
    del graph
    plan.free()


def test_captured_muon_step_replays_like_eager_calls():
    """Distributed Muon (gather, Newton-Schulz, apply over every root)
    captured once and replayed three times, against eager calls on a twin."""
    specs = [TensorSpec("a", (136, 200), ROWS, 8), TensorSpec("b", (200, 136), ROWS, 8),
             TensorSpec("c", (256, 512), ROWS, 32)]
    m, g = 3, 16
    log("graph capture muon")
    plan = make_plan(specs, m, g)
    mu = rs.Muon(plan, [0, 1, 2]).upload()
    gen = torch.Generator(device="cuda").manual_seed(3)
    theta0 = torch.rand(plan.total, device="cuda", generator=gen) * 0.2 - 0.1
    grad = (torch.randn(plan.total, device="cuda", generator=gen) * 1e-3).to(
        torch.bfloat16).view(torch.int16)

    def twin():
        return {"theta": theta0.clone(), "mom": torch.zeros(plan.total, device="cuda"),
                "root": torch.zeros(mu.root_elems, dtype=torch.int16, device="cuda")}

    def sequence(st):
        rs.rs_muon_gather(mu.h, rs.RS_ALL, st["mom"], grad, st["root"], momentum=0.95)
        rs.rs_muon_orthogonalize(mu.h, rs.RS_ALL, st["root"])
        rs.rs_muon_apply(mu.h, rs.RS_ALL, st["theta"], st["root"], lr=1e-3, weight_decay=0.01)

    eager, graphed = twin(), twin()
    expected = []
    for _ in range(3):
        sequence(eager)
        torch.cuda.synchronize()
        expected.append({k: v.cpu().numpy().copy() for k, v in eager.items()})
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sequence(graphed)
    torch.cuda.synchronize()
    assert not graphed["mom"].any()  # capture ran nothing
    for k, exp in enumerate(expected):
        graph.replay()
        torch.cuda.synchronize()
        for name, v in graphed.items():
            assert np.array_equal(v.cpu().numpy().view(np.uint8), exp[name].view(np.uint8)), (k, name)
    del graph
    mu.free()
    plan.free()
