"""The allocation-free L2 norm (rs_group_l2norm_static), through the C-ABI:
the same result as rs_group_l2norm bit for bit (same kernels; partial sums
in the library's own device array instead of the plan's workspace), on two
calls in a row, the second with a smaller input, and without an uploaded
plan."""
import math

import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
import synth
from gpu_harness import log, make_plan

pytestmark = pytest.mark.gpu


def _grads(L, specs, seed):
    g = torch.zeros(L.total, dtype=torch.int16, device="cuda")
    for i, s in enumerate(specs):
        g[L.pos[i]:L.pos[i] + s.numel] = synth.normal_bf16(s.numel, 1e-3, seed, i,
                                                            device="cuda").view(torch.int16)
    return g


def test_static_l2norm_matches_workspace_l2norm_on_two_calls():
    big = synth.llama_layer_2048()           # 51.4M elements: 2048 partial sums
    small = synth.tiny()                     # 20,480 elements: 3 partial sums
    out_ws = torch.zeros(1, dtype=torch.float64, device="cuda")
    out_st = torch.zeros(1, dtype=torch.float64, device="cuda")
    for k, w in enumerate((big, small)):
        log(f"static l2norm call {k + 1}: {w.name}")
        L = oracle.Layout(w.specs, w.m, w.g_coll)
        g = _grads(L, w.specs, 40 + k)
        bare = rs.Plan(w.specs, w.m, w.g_coll)        # never uploaded
        rs.rs_group_l2norm_static(bare.h, rs.RS_ALL, rs.RS_ALL, g, rs.RS_BF16, out_st)
        up = make_plan(w.specs, w.m, w.g_coll)
        rs.rs_group_l2norm(up.h, rs.RS_ALL, rs.RS_ALL, g, rs.RS_BF16, out_ws)
        torch.cuda.synchronize()
        assert out_st.item() == out_ws.item()          # bit for bit
        exp = L.group_sumsq(-1, -1, g.cpu().numpy().view(np.uint16))
        assert math.isclose(math.sqrt(out_st.item()), math.sqrt(exp), rel_tol=1e-5)
        # one rank's slice, fp32 data
        x = torch.randn(L.total, generator=torch.Generator(device="cuda").manual_seed(k),
                        device="cuda")
        r = w.m - 1
        rs.rs_group_l2norm_static(bare.h, 0, r, x, rs.RS_F32, out_st)
        rs.rs_group_l2norm(up.h, 0, r, x, rs.RS_F32, out_ws)
        torch.cuda.synchronize()
        assert out_st.item() == out_ws.item()
        bare.free()
        up.free()


def test_static_l2norm_rejects_bad_arguments():
    w = synth.tiny()
    plan = rs.Plan(w.specs, w.m, w.g_coll)
    out = torch.zeros(1, dtype=torch.float64, device="cuda")
    g = torch.zeros(1 << 16, dtype=torch.int16, device="cuda")
    with pytest.raises(rs.RaggedShardError) as ei:
        rs.rs_group_l2norm_static(plan.h, 0, w.m, g, rs.RS_BF16, out)
    assert ei.value.status == rs.RS_EINVAL
    with pytest.raises(rs.RaggedShardError) as ei:
        rs.rs_group_l2norm_static(plan.h, 0, 0, g, 7, out)
    assert ei.value.status == rs.RS_EINVAL
    plan.free()
