"""Degenerate selections on the GPU, through the C ABI, against the oracle:
ranks whose slices hold no tensor data (only padding, or nothing at all),
and a bucket set where one bucket leaves several ranks empty.  Every op
must leave everything outside its selection untouched, write the
selection's padding as its definition says (zeros for the copy-ins and the
zero op), and change no state on a rank without blocks."""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
from synth import ELEMENT, ROWS, TILE, TensorSpec
from gpu_harness import (DevState, assert_step_close, dev_to_u16, host_state, log, make_plan,
                         padding_mask, u16_to_dev)

pytestmark = pytest.mark.gpu


def _layout():
    # bucket 0: three 32-row blocks of 512 elements over m = 5 ranks -> ranks
    # 3 and 4 hold padding only; bucket 1: a tile tensor and a vector that
    # fill the first ranks only
    specs = [TensorSpec("a", (96, 16), ROWS, 32, bucket=0),
             TensorSpec("t", (64, 32), TILE, 32, 32, bucket=1),
             TensorSpec("v", (40,), ELEMENT, bucket=1)]
    return specs, 5, 16


def _empty_ranks(plan, L):
    out = []
    for b in range(L.nb):
        for r in range(plan.m):
            if rs.rs_plan_rank_blocks(plan.h, b, r)[1] == 0:
                out.append((b, r))
    return out


def test_layout_has_empty_ranks():
    specs, m, g = _layout()
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    empty = _empty_ranks(plan, L)
    assert (0, 3) in empty and (0, 4) in empty and len(empty) >= 3
    plan.free()


@pytest.mark.parametrize("mode", [rs.RS_SPLIT_COOPERATIVE, rs.RS_SPLIT_ORDERED,
                                  rs.RS_SPLIT_TWO_PASS])
def test_step_on_ranks_without_blocks_changes_nothing(mode):
    specs, m, g = _layout()
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g, mode=mode)
    h = host_state(L, specs, seed=3, sigma=1e-3, warm=True)
    for b, r in _empty_ranks(plan, L):
        log(f"empty step bucket {b} rank {r} mode {mode}")
        d = DevState(h, with_out=True)
        d.step(plan, b, r, 2)
        got = d.host()
        for name in ("theta", "grad", "qm", "qv", "am", "av"):
            assert np.array_equal(getattr(got, name).view(np.uint8),
                                  getattr(h, name).view(np.uint8)), (b, r, name)
        assert not d.out.any()  # the bf16 output is not touched either
    if mode != rs.RS_SPLIT_TWO_PASS:
        rs.rs_plan_check_device(plan.h)
    plan.free()


def test_fp8_output_step_on_ranks_without_blocks_writes_nothing():
    specs, m, g = _layout()
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    h = host_state(L, specs, seed=5, sigma=1e-3, warm=True)
    for b, r in _empty_ranks(plan, L):
        log(f"empty fp8-output step bucket {b} rank {r}")
        d = DevState(h, with_out=True)
        codes = torch.full((L.total,), 0x5A, dtype=torch.uint8, device="cuda")
        scale = torch.full((L.n_blocks,), -1.0, dtype=torch.float32, device="cuda")
        rs.rs_adam8_step_fp8(plan.h, b, r, d.theta, d.grad, d.qm, d.qv, d.am, d.av, codes,
                             scale, step=2, bf16_out=d.out)
        got = d.host()
        for name in ("theta", "qm", "qv", "am", "av"):
            assert np.array_equal(getattr(got, name).view(np.uint8),
                                  getattr(h, name).view(np.uint8)), (b, r, name)
        assert not d.out.any()
        assert bool((codes == 0x5A).all()) and bool((scale == -1.0).all())
    rs.rs_plan_check_device(plan.h)
    plan.free()


def test_copy_ins_and_group_ops_on_ranks_without_blocks():
    specs, m, g = _layout()
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    hv = [np.arange(s.numel, dtype=np.float32) * np.float32(0.25) - 3 for s in specs]
    dv = [torch.from_numpy(v).cuda() for v in hv]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dv)
    for b, r in _empty_ranks(plan, L):
        log(f"empty copy-ins bucket {b} rank {r}")
        # bf16 copy-in: the slice becomes zeros, nothing else moves
        buf = torch.full((L.total,), 0x3C3C, dtype=torch.int16, device="cuda")
        rs.rs_pack_shard(plan.h, b, r, buf)
        exp = np.full(L.total, 0x3C3C, dtype=np.uint16)
        L.pack(b, r, hv, exp)
        assert np.array_equal(dev_to_u16(buf), exp)
        lo = L.base[b] + r * L.S[b]
        assert not exp[lo:lo + L.S[b]].any()
        # FP8 copy-in: zero codes in the slice, no scale written
        b8 = torch.full((L.total,), 0x5A, dtype=torch.uint8, device="cuda")
        sc = torch.full((L.n_blocks,), -1.0, dtype=torch.float32, device="cuda")
        rs.rs_pack_shard_fp8(plan.h, b, r, b8, sc)
        e8 = np.full(L.total, 0x5A, dtype=np.uint8)
        esc = np.full(L.n_blocks, -1.0, dtype=np.float32)
        L.pack_fp8(b, r, hv, e8, esc)
        assert np.array_equal(b8.cpu().numpy(), e8)
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), esc.view(np.uint32))
        # group ops over the slice: the norm of a zero slice is 0; zero and
        # scale touch only the slice
        grad = np.full(L.total, 0x3F80, dtype=np.uint16)  # 1.0 everywhere
        grad[lo:lo + L.S[b]] = 0
        dg = u16_to_dev(grad)
        ss = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
        rs.rs_group_l2norm(plan.h, b, r, dg, rs.RS_BF16, ss)
        assert ss.item() == 0.0 == L.group_sumsq(b, r, grad)
        ones = u16_to_dev(np.full(L.total, 0x3F80, dtype=np.uint16))
        rs.rs_group_zero(plan.h, b, r, ones, rs.RS_BF16)
        z = dev_to_u16(ones)
        assert not z[lo:lo + L.S[b]].any()
        assert (np.delete(z, np.s_[lo:lo + L.S[b]]) == 0x3F80).all()
    rs.rs_plan_check_device(plan.h)
    plan.free()


def test_whole_set_with_empty_ranks_matches_oracle():
    """The all-rank step over the layout with empty ranks."""
    specs, m, g = _layout()
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    h = host_state(L, specs, seed=4, sigma=1e-3, warm=False)
    d = DevState(h)
    d.step(plan, rs.RS_ALL, rs.RS_ALL, 1)
    got = d.host()
    exp = h.copy()
    L.adam8_step(-1, -1, exp.theta, exp.grad, exp.qm, exp.qv, exp.am, exp.av,
                 oracle.HParams(step=1))
    pad = padding_mask(L)
    assert_step_close(got, exp, mask=~pad, what="empty-rank layout")
    assert np.array_equal(got.qm, exp.qm) and np.array_equal(got.qv, exp.qv)
    assert (got.theta[pad] == 7.0).all()
    rs.rs_plan_check_device(plan.h)
    plan.free()
