"""GPU parity of the DBuffer copy-in / copy-out and group ops against the
oracle (bit-exact; the L2 norm to 1e-5 relative).  Runs through the C-ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
import synth
from synth import ELEMENT, ROWS, TILE, TensorSpec
from gpu_harness import check_plan_matches, dev_to_u16, log, make_plan, u16_to_dev

pytestmark = pytest.mark.gpu


def _odd_specs():
    # starts and sizes that are not multiples of 8 exercise the element-wise
    # head/tail and the scalar path (g_coll = 1)
    return [TensorSpec("a", (37, 5), ROWS, 3), TensorSpec("b", (101,), ELEMENT),
            TensorSpec("c", (19, 24), TILE, 4, 8), TensorSpec("d", (3, 7, 9), ROWS, 2)]


def _multi_bucket_specs():
    out = []
    for b in range(3):
        out += [TensorSpec(f"w{b}", (96, 64), TILE, 32, 32, b),
                TensorSpec(f"r{b}", (50, 48), ROWS, 8, 0, b),
                TensorSpec(f"n{b}", (200,), ROWS, 32, 0, b)]
    return out


LAYOUTS = {
    "tiny": lambda: (synth.tiny().specs, 4, 16),
    "llama_layer": lambda: (synth.llama_layer_2048().specs, 8, 16),
    "odd_g1": lambda: (_odd_specs(), 3, 1),
    "multi_bucket": lambda: (_multi_bucket_specs(), 5, 16),
    "one_layer_tiles": lambda: (synth.llama8b_tiles(layers=1).specs, 64, 16),
}


@pytest.mark.parametrize("name", list(LAYOUTS))
def test_pack_bitexact(name):
    specs, m, g = LAYOUTS[name]()
    log(f"pack {name}")
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    check_plan_matches(plan, L)
    hv = [synth.uniform_params(s.numel, 3, i).numpy() for i, s in enumerate(specs)]
    hv[0][:3] = [np.inf, -np.inf, 1e38]          # overflow / infinities round like the oracle
    dv = [torch.from_numpy(v).cuda() for v in hv]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dv)
    buf = torch.full((L.total,), 0x1234, dtype=torch.int16, device="cuda")
    rs.rs_pack_shard(plan.h, rs.RS_ALL, rs.RS_ALL, buf)
    exp = np.full(L.total, 0x1234, dtype=np.uint16)
    L.pack(-1, -1, hv, exp)
    assert np.array_equal(dev_to_u16(buf), exp)
    # one slice at a time touches only that slice
    ranks = sorted({0, m // 2, m - 1})
    for b in range(min(L.nb, 2)):
        for r in ranks:
            buf.fill_(0x4321)
            rs.rs_pack_shard(plan.h, b, r, buf)
            exp = np.full(L.total, 0x4321, dtype=np.uint16)
            L.pack(b, r, hv, exp)
            assert np.array_equal(dev_to_u16(buf), exp), (b, r)
    plan.free()


@pytest.mark.parametrize("name", list(LAYOUTS))
@pytest.mark.parametrize("alias", [False, True])
def test_unpack_bitexact(name, alias):
    specs, m, g = LAYOUTS[name]()
    log(f"unpack {name} alias={alias}")
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    hbuf = oracle.bf16(np.random.default_rng(1).standard_normal(L.total).astype(np.float32))
    buf = u16_to_dev(hbuf)
    views = []
    aliased = set()
    for i, s in enumerate(specs):
        if alias and i % 2 == 0 and L.pos[i] % 8 == 0:
            views.append(buf[L.pos[i]:L.pos[i] + s.numel])   # zero-copy view into the buffer
            aliased.add(i)
        else:
            views.append(torch.full((s.numel,), 0x7777, dtype=torch.int16, device="cuda"))
    rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, views)
    rs.rs_unpack_full(plan.h, rs.RS_ALL, buf)
    exp = [np.zeros(s.numel, dtype=np.uint16) for s in specs]
    L.unpack(-1, exp, hbuf)
    for i, v in enumerate(views):
        assert np.array_equal(dev_to_u16(v), exp[i]), i
    assert np.array_equal(dev_to_u16(buf), hbuf)            # the buffer is never written
    if L.nb > 1:
        # one bucket only: views of other buckets untouched
        for i in range(len(specs)):
            if i not in aliased:
                views[i].fill_(0x7777)
        rs.rs_unpack_full(plan.h, 1, buf)
        for i, s in enumerate(specs):
            if i in aliased:
                continue
            got = dev_to_u16(views[i])
            if s.bucket == 1:
                assert np.array_equal(got, exp[i])
            else:
                assert (got == 0x7777).all()
    plan.free()


@pytest.mark.parametrize("name", ["tiny", "odd_g1", "multi_bucket", "llama_layer"])
@pytest.mark.parametrize("dtype", [rs.RS_BF16, rs.RS_F32])
def test_group_ops(name, dtype):
    specs, m, g = LAYOUTS[name]()
    log(f"group ops {name} dtype={dtype}")
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    rng = np.random.default_rng(2)
    x32 = rng.standard_normal(L.total).astype(np.float32)
    host = oracle.bf16(x32) if dtype == rs.RS_BF16 else x32
    dev = u16_to_dev(host) if dtype == rs.RS_BF16 else torch.from_numpy(x32.copy()).cuda()
    back = (lambda t: dev_to_u16(t)) if dtype == rs.RS_BF16 else (lambda t: t.cpu().numpy())
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    sels = [(rs.RS_ALL, rs.RS_ALL), (0, 0), (0, m - 1), (rs.RS_ALL, m // 2)]
    if L.nb > 1:
        sels.append((L.nb - 1, rs.RS_ALL))
    for b, r in sels:
        rs.rs_group_l2norm(plan.h, b, r, dev, dtype, sumsq)
        exp = L.group_sumsq(b, r, host)
        got = float(sumsq.item())
        assert math.isclose(math.sqrt(got), math.sqrt(exp), rel_tol=1e-5), (b, r)
        # deterministic reduction order: repeat gives the same bits
        rs.rs_group_l2norm(plan.h, b, r, dev, dtype, sumsq)
        assert float(sumsq.item()) == got
    for b, r in sels:
        for s in (0.37, 2.0 ** -3, 1.0):
            rs.rs_group_scale(plan.h, b, r, dev, dtype, s)
            L.group_scale(b, r, host, s)
            assert np.array_equal(back(dev), host), (b, r, s)
    rs.rs_group_zero(plan.h, 0, m - 1, dev, dtype)
    L.group_zero(0, m - 1, host)
    assert np.array_equal(back(dev), host)
    rs.rs_group_zero(plan.h, rs.RS_ALL, rs.RS_ALL, dev, dtype)
    assert not back(dev).any()
    plan.free()


def _clip_formula(sumsq: float, max_norm: float) -> float:
    return float(np.float32(min(1.0, max_norm / (math.sqrt(sumsq) + 1e-6))))


def test_l2norm_and_clip_coefficient():
    specs, m, g = LAYOUTS["llama_layer"]()
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    for sigma in (1e-3, 1.0):
        host = np.zeros(L.total, dtype=np.uint16)
        for i, s in enumerate(specs):
            host[L.pos[i]:L.pos[i] + s.numel] = synth.normal_bf16(
                s.numel, sigma, 5, i).view(torch.int16).numpy().view(np.uint16)
        dev = u16_to_dev(host)
        sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
        scale = torch.zeros(1, dtype=torch.float32, device="cuda")
        rs.rs_group_l2norm(plan.h, rs.RS_ALL, rs.RS_ALL, dev, rs.RS_BF16, sumsq)
        rs.rs_clip_coef(sumsq, 1.0, scale)
        got = float(sumsq.item())
        exp = L.group_sumsq(-1, -1, host)
        assert math.isclose(math.sqrt(got), math.sqrt(exp), rel_tol=1e-5)
        # the coefficient: the oracle's, from the oracle's sum, to the sum's
        # tolerance; and exactly the formula (binary64, one rounding) applied
        # to the device's own sum
        assert math.isclose(scale.item(), oracle.clip_coef(exp, 1.0), rel_tol=1e-5)
        assert scale.item() == _clip_formula(got, 1.0)
        # the fused norm-and-clip launch gives both bit for bit, for a
        # threshold that clips (sigma = 1) and one that does not
        for max_norm in (1.0, 1e6):
            s2 = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
            c2 = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
            rs.rs_group_l2norm_clip(plan.h, rs.RS_ALL, rs.RS_ALL, dev, rs.RS_BF16, max_norm, s2, c2)
            assert s2.cpu().numpy().view(np.uint64)[0] == sumsq.cpu().numpy().view(np.uint64)[0]
            assert c2.item() == _clip_formula(got, max_norm)
            assert math.isclose(c2.item(), oracle.clip_coef(exp, max_norm), rel_tol=1e-5)
        # per-rank partial sums add up to the global sum
        parts = 0.0
        for r in range(m):
            rs.rs_group_l2norm(plan.h, 0, r, dev, rs.RS_BF16, sumsq)
            parts += float(sumsq.item())
        assert math.isclose(parts, got, rel_tol=1e-12)
    plan.free()


def test_l2norm_propagates_nonfinite():
    specs, m, g = LAYOUTS["tiny"]()
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    x = np.zeros(L.total, dtype=np.float32)
    x[L.pos[1] + 5] = np.inf
    dev = torch.from_numpy(x).cuda()
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    rs.rs_group_l2norm(plan.h, rs.RS_ALL, rs.RS_ALL, dev, rs.RS_F32, sumsq)
    assert math.isinf(sumsq.item())
    plan.free()


@pytest.mark.parametrize("options", [rs.RS_ORDER_BY_SIZE, rs.RS_ORDER_BY_BLOCK | rs.RS_ALIGN_CUT_UNIT])
@pytest.mark.parametrize("name", ["odd_g1", "multi_bucket", "tiny"])
def test_pack_unpack_with_planner_orders(name, options):
    """Reordered plans: the copy kernels walk the tensors in buffer order."""
    specs, m, g = LAYOUTS[name]()
    log(f"pack/unpack {name} options={options:#x}")
    L = oracle.Layout(specs, m, g, order=options & rs.RS_ORDER_MASK,
                      align_unit=bool(options & rs.RS_ALIGN_CUT_UNIT))
    plan = make_plan(specs, m, g, options=options)
    check_plan_matches(plan, L)
    hv = [synth.uniform_params(s.numel, 5, i).numpy() for i, s in enumerate(specs)]
    dv = [torch.from_numpy(v).cuda() for v in hv]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dv)
    buf = torch.full((L.total,), 0x1234, dtype=torch.int16, device="cuda")
    rs.rs_pack_shard(plan.h, rs.RS_ALL, rs.RS_ALL, buf)
    exp = np.full(L.total, 0x1234, dtype=np.uint16)
    L.pack(-1, -1, hv, exp)
    assert np.array_equal(dev_to_u16(buf), exp)
    outs = [torch.zeros(s.numel, dtype=torch.int16, device="cuda") for s in specs]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, outs)
    rs.rs_unpack_full(plan.h, rs.RS_ALL, buf)
    hexp = [np.zeros(s.numel, dtype=np.uint16) for s in specs]
    L.unpack(-1, hexp, exp)
    for o, e in zip(outs, hexp):
        assert np.array_equal(dev_to_u16(o), e)
    plan.free()
