"""GPU parity of the step with FP8 output (rs_adam8_step_fp8): the int8
AdamW step and, in the same pass, the FP8 copy-in of the new master.

Three checks per call:
- the step's own outputs (master, codes, absmax, bf16 output) are bit for
  bit those of rs_adam8_step on the same state;
- the FP8 codes and scales are bit for bit those rs_pack_shard_fp8 gives
  for views holding the new master (the contract of the entry point;
  rs_pack_shard_fp8 itself is pinned to the oracle bit for bit in
  test_gpu_fp8.py), and padding and unselected slices are not written;
- against the oracle run on its own (its step, then its FP8 copy-in of its
  own master): scales to the relative 2e-6 that the master tolerance
  allows, codes equal except where the two masters straddle a rounding
  boundary, and there at most one E4M3 step apart."""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
import synth
from gpu_harness import (DevState, assert_step_close, check_plan_matches, dev_to_u16,
                         fresh_grads, host_state, log, make_plan, padding_mask, u16_to_dev)
from test_gpu_step import CASES

pytestmark = pytest.mark.gpu

TWO, COOP, ORD = rs.RS_SPLIT_TWO_PASS, rs.RS_SPLIT_COOPERATIVE, rs.RS_SPLIT_ORDERED
SENT8 = 0x5A


class Fp8Out:
    def __init__(self, L):
        self.codes = torch.full((L.total,), SENT8, dtype=torch.uint8, device="cuda")
        self.scale = torch.full((L.n_blocks,), -1.0, dtype=torch.float32, device="cuda")


def _fused_step(plan, ds: DevState, f8: Fp8Out, bucket, rank, t, gscale=None):
    rs.rs_adam8_step_fp8(plan.h, bucket, rank, ds.theta, ds.grad, ds.qm, ds.qv, ds.am, ds.av,
                         f8.codes, f8.scale, step=t, grad_scale=gscale, bf16_out=ds.out)


def _same_step(a: DevState, b: DevState):
    torch.cuda.synchronize()
    for x, y in ((a.theta, b.theta), (a.qm, b.qm), (a.qv, b.qv), (a.am, b.am), (a.av, b.av),
                 (a.out, b.out)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def _pack_of_master(plan, L, specs, ds: DevState, bucket, rank):
    """rs_pack_shard_fp8 of views holding the device master."""
    views = [ds.theta[L.pos[i]:L.pos[i] + s.numel] for i, s in enumerate(specs)]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, views)
    ref = Fp8Out(L)
    rs.rs_pack_shard_fp8(plan.h, bucket, rank, ref.codes, ref.scale)
    return ref


def _check_against_pack(L, pad, fused: Fp8Out, packed: Fp8Out):
    torch.cuda.synchronize()
    fc, pc = fused.codes.cpu().numpy(), packed.codes.cpu().numpy()
    real = ~pad
    bad = np.nonzero(fc[real] != pc[real])[0]
    assert bad.size == 0, f"{bad.size} codes differ from the copy-in of the new master"
    # padding is never written by the step (the copy-in writes zeros there)
    assert (fc[pad] == SENT8).all()
    fs, ps = fused.scale.cpu().numpy(), packed.scale.cpu().numpy()
    assert np.array_equal(fs.view(np.uint32), ps.view(np.uint32))


def _e4m3_values(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()


def _check_against_oracle(L, specs, pad, ref_theta, fused: Fp8Out, what=""):
    hv = [ref_theta[L.pos[i]:L.pos[i] + s.numel].copy() for i, s in enumerate(specs)]
    ec = np.zeros(L.total, dtype=np.uint8)
    es = np.zeros(L.n_blocks, dtype=np.float32)
    L.pack_fp8(rs.RS_ALL, rs.RS_ALL, hv, ec, es)
    gc, gs = fused.codes.cpu().numpy(), fused.scale.cpu().numpy()
    assert np.allclose(gs, es, rtol=2e-6, atol=1e-12), f"{what}: scales"
    real = ~pad
    g, e = _e4m3_values(gc[real]), _e4m3_values(ec[real])
    diff = g != e
    n = int(diff.sum())
    assert n <= max(2, int(1e-3 * real.sum())), f"{what}: {n} codes differ"
    if n:
        # neighbours on the E4M3 grid: at most one step (2^-3 relative, or
        # the subnormal step 2^-9) apart
        gd, ed = g[diff], e[diff]
        step = np.maximum(np.maximum(np.abs(gd), np.abs(ed)) * 0.125, 2.0 ** -9)
        assert (np.abs(gd - ed) <= step).all(), f"{what}: codes more than one step apart"


def _run(name, mode, chunk, steps=3, per_rank=False, warm=False, gscale=None, options=0):
    specs, m, g, sigma = CASES[name]()
    L = oracle.Layout(specs, m, g, order=options & rs.RS_ORDER_MASK,
                      align_unit=bool(options & rs.RS_ALIGN_CUT_UNIT))
    plan = make_plan(specs, m, g, chunk=chunk, mode=mode, options=options)
    check_plan_matches(plan, L)
    hs = host_state(L, specs, seed=5, sigma=sigma, warm=warm)
    ds = DevState(hs, with_out=True)      # fused step
    dp = DevState(hs, with_out=True)      # plain step
    f8 = Fp8Out(L)
    ref = hs.copy()
    pad = padding_mask(L)
    gs_dev = None if gscale is None else torch.tensor([gscale], dtype=torch.float32,
                                                      device="cuda")
    for t in range(1, steps + 1):
        if t > 1:
            gr = fresh_grads(L, specs, 5, sigma, t)
            ref.grad = gr
            ds.grad.copy_(u16_to_dev(gr))
            dp.grad.copy_(u16_to_dev(gr))
        sel = [(b, r) for b in range(L.nb) for r in range(m)] if per_rank else \
            [(rs.RS_ALL, rs.RS_ALL)]
        for b, r in sel:
            _fused_step(plan, ds, f8, b, r, t, gs_dev)
            dp.step(plan, b, r, t, gscale=gs_dev)
        _same_step(ds, dp)
        _check_against_pack(L, pad, f8, _pack_of_master(plan, L, specs, ds, rs.RS_ALL,
                                                        rs.RS_ALL))
        L.adam8_step(-1, -1, ref.theta, ref.grad, ref.qm, ref.qv, ref.am, ref.av,
                     oracle.HParams(step=t), gscale=1.0 if gscale is None else gscale)
        got = ds.host()
        assert_step_close(got, ref, mask=~pad, what=f"{name} step {t}")
        _check_against_oracle(L, specs, pad, ref.theta, f8, what=f"{name} step {t}")
    if mode != TWO:
        rs.rs_plan_check_device(plan.h)
    plan.free()


@pytest.mark.parametrize("mode", [TWO, COOP, ORD])
@pytest.mark.parametrize("chunk", [None, 1024, 64])
@pytest.mark.parametrize("name", ["mixed", "multi_bucket", "tiny"])
def test_step_fp8_free_running(name, chunk, mode):
    log(f"step fp8 {name} chunk={chunk} mode={mode}")
    _run(name, mode, chunk)


@pytest.mark.parametrize("mode", [TWO, COOP])
def test_step_fp8_per_rank_calls_warm_and_grad_scale(mode):
    log(f"step fp8 per-rank warm mode={mode}")
    _run("mixed", mode, 1024, steps=2, per_rank=True, warm=True, gscale=0.5)
    _run("multi_bucket", mode, None, steps=2, per_rank=True, warm=True)


@pytest.mark.parametrize("options", [rs.RS_ORDER_BY_BLOCK, rs.RS_ORDER_BY_SIZE,
                                     rs.RS_ALIGN_CUT_UNIT | rs.RS_ORDER_BY_SIZE])
def test_step_fp8_with_planner_orders(options):
    """Reordered plans: block ids (absmax and FP8 scales) follow buffer order."""
    log(f"step fp8 planner options={options:#x}")
    _run("mixed", COOP, 1024, steps=2, options=options)
    _run("multi_bucket", COOP, None, steps=2, options=options)


def test_step_fp8_touches_only_its_slice():
    """One rank's call writes codes and scales of that rank's blocks only."""
    specs, m, g, sigma = CASES["mixed"]()
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g, chunk=1024)
    hs = host_state(L, specs, seed=6, sigma=sigma, warm=True)
    pad = padding_mask(L)
    for r in (0, m - 1):
        log(f"step fp8 slice rank {r}")
        ds = DevState(hs)
        f8 = Fp8Out(L)
        _fused_step(plan, ds, f8, 0, r, 3)
        codes = f8.codes.cpu().numpy()
        scale = f8.scale.cpu().numpy()
        lo, hi = L.base[0] + r * L.S[0], L.base[0] + (r + 1) * L.S[0]
        inside = np.zeros(L.total, dtype=bool)
        inside[lo:hi] = True
        assert (codes[~inside | pad] == SENT8).all()
        b0, b1 = rs.rs_plan_rank_blocks(plan.h, 0, r)
        sel = np.zeros(L.n_blocks, dtype=bool)
        sel[b0:b0 + b1] = True
        assert (scale[~sel] == -1.0).all() and (scale[sel] >= 0.0).all()
        packed = _pack_of_master(plan, L, specs, ds, 0, r)
        pc = packed.codes.cpu().numpy()
        real_in = inside & ~pad
        assert np.array_equal(codes[real_in], pc[real_in])
        assert np.array_equal(scale[sel].view(np.uint32), packed.scale.cpu().numpy()[sel].view(np.uint32))
    rs.rs_plan_check_device(plan.h)
    plan.free()


def _set_status_word(plan, value):
    off = rs.rs_plan_status_offset(plan.h)
    torch.cuda.synchronize()
    plan.workspace[off:off + 4].view(torch.int32).fill_(value)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", [COOP, ORD])
@pytest.mark.parametrize("chunk", [1024, 64])
def test_step_fp8_status_word_path(chunk, mode):
    """With the device status word set, split blocks take the wait-free
    whole-block path (FP8 output included; there the master comes from the
    correctly rounded operations, so it may differ from the waiting path's
    by the master tolerance): step outputs against the oracle (codes and
    absmax exact), FP8 codes and scales those of the copy-in of the new
    master, every kernel ends normally and the word is reported."""
    specs, m, g, sigma = CASES["mixed"]()
    log(f"step fp8 status word chunk={chunk} mode={mode}")
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g, chunk=chunk, mode=mode)
    hs = host_state(L, specs, seed=3, sigma=sigma, warm=True)
    ds = DevState(hs, with_out=True)
    f8 = Fp8Out(L)
    pad = padding_mask(L)
    ref = hs.copy()
    _set_status_word(plan, 1)
    _fused_step(plan, ds, f8, rs.RS_ALL, rs.RS_ALL, 11)
    with pytest.raises(rs.RaggedShardError):
        rs.rs_plan_check_device(plan.h)
    rs.rs_plan_check_device(plan.h)  # cleared
    L.adam8_step(-1, -1, ref.theta, ref.grad, ref.qm, ref.qv, ref.am, ref.av,
                 oracle.HParams(step=11))
    got = ds.host()
    assert_step_close(got, ref, mask=~pad, what="status word path")
    assert np.array_equal(got.qm, ref.qm) and np.array_equal(got.qv, ref.qv)
    assert np.array_equal(got.am, ref.am) and np.array_equal(got.av, ref.av)
    _check_against_pack(L, pad, f8, _pack_of_master(plan, L, specs, ds, rs.RS_ALL, rs.RS_ALL))
    _check_against_oracle(L, specs, pad, ref.theta, f8, what="status word path")
    plan.free()


@pytest.mark.parametrize("name", ["llama_layer", "moe_rank0", "llama8b_full"])
def test_step_fp8_full_size_matches_step_and_copy_in(name):
    """Full-size workloads (the one-layer bucket, 51.4M elements; one MoE
    rank's shard of 90-chunk blocks; the 8.03e9-parameter state, positions
    past 2^32), one launch as timed: the fused outputs equal rs_adam8_step's
    and rs_pack_shard_fp8's of the new master, compared on the device
    element by element."""
    if name == "llama_layer":
        w = synth.llama_layer_2048()
        bucket, rank = rs.RS_ALL, rs.RS_ALL
    elif name == "moe_rank0":
        w = synth.moe_bucket()
        bucket, rank = 0, 0
    else:
        w = synth.llama8b_full()
        bucket, rank = rs.RS_ALL, rs.RS_ALL
    log(f"step fp8 full size {name}")
    plan = make_plan(w.specs, w.m, w.g_coll)
    total, nblk = plan.total, plan.n_blocks
    gen = torch.Generator(device="cuda").manual_seed(17)
    theta = torch.rand(total, device="cuda", generator=gen) * 2 - 1
    grad = (torch.randn(total, device="cuda", generator=gen) * w.grad_sigma).to(torch.bfloat16)
    st = [theta, grad.view(torch.int16),
          torch.zeros(total, dtype=torch.int8, device="cuda"),
          torch.zeros(total, dtype=torch.uint8, device="cuda"),
          torch.zeros(nblk, device="cuda"), torch.zeros(nblk, device="cuda")]
    plain = [x.clone() for x in st]
    codes = torch.full((total,), SENT8, dtype=torch.uint8, device="cuda")
    scale = torch.full((nblk,), -1.0, device="cuda")
    for t in (1, 2):
        rs.rs_adam8_step_fp8(plan.h, bucket, rank, *st, codes, scale, step=t)
        rs.rs_adam8_step(plan.h, bucket, rank, *plain, step=t)
        for a, b in zip(st, plain):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"step {t}"
    del plain
    torch.cuda.empty_cache()
    views = [st[0][plan.pos[i]:plan.pos[i] + s.numel] for i, s in enumerate(w.specs)]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, views)
    pc = torch.full((total,), SENT8, dtype=torch.uint8, device="cuda")
    ps = torch.full((nblk,), -1.0, device="cuda")
    rs.rs_pack_shard_fp8(plan.h, bucket, rank, pc, ps)
    # the selection's tensor elements: equal codes; everything else (padding,
    # other slices) untouched by the fused step
    real = torch.zeros(total, dtype=torch.bool, device="cuda")
    for i, s in enumerate(w.specs):
        real[plan.pos[i]:plan.pos[i] + s.numel] = True
    if rank != rs.RS_ALL:
        lo = plan.base[bucket] + rank * plan.S[bucket]
        inside = torch.zeros(total, dtype=torch.bool, device="cuda")
        inside[lo:lo + plan.S[bucket]] = True
        real &= inside
    assert int(real.sum()) > 0
    # elementwise (no boolean-mask gathers: those fail past 2^32 elements)
    assert bool(((codes == pc) | ~real).all())
    assert bool(((codes == SENT8) | real).all())
    assert torch.equal(scale.view(torch.int32), ps.view(torch.int32))
    rs.rs_plan_check_device(plan.h)
    plan.free()
    del st, theta, grad, codes, scale, views, pc, ps, real
    torch.cuda.empty_cache()
