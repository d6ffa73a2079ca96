"""The hot path under HIP graph capture: the entry points launch kernels
only (no allocation, copy or memset), so a step captured once replays.
Captured here: the allocation-free L2 norm, the clipping coefficient and
the step with bf16 and FP8 output, on a layout with split blocks in the
cooperative mode (cross-workgroup waits inside the graph).  Every replay
is compared bit for bit with the same sequence run eagerly on a twin of
the state, with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
from gpu_harness import DevState, host_state, log, make_plan
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


@pytest.mark.parametrize("mode", [rs.RS_SPLIT_COOPERATIVE, rs.RS_SPLIT_ORDERED])
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
    rs.rs_plan_check_device(plan.h)
    del graph
    plan.free()
