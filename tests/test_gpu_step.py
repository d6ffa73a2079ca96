"""GPU parity of the fused blockwise-int8 AdamW step against the oracle,
free-running over several steps (both sides start from the same synthetic
state and never exchange intermediate results)."""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
import synth
from synth import ELEMENT, ROWS, TILE, TensorSpec
from gpu_harness import (SENT_CODE, DevState, assert_step_close, check_plan_matches, dev_to_u16,
                         fresh_grads, host_state, log, make_plan, padding_mask, u16_to_dev)

pytestmark = pytest.mark.gpu

TWO, COOP, ORD = rs.RS_SPLIT_TWO_PASS, rs.RS_SPLIT_COOPERATIVE, rs.RS_SPLIT_ORDERED


def _mixed_specs():
    # every chunk kind: vector tiles (split and whole), vector row blocks
    # (split, whole, runs of small blocks), scalar blocks (odd widths and
    # offsets), element runs; and ragged tails
    return [
        TensorSpec("tile", (200, 96), TILE, 32, 32),        # ragged last band
        TensorSpec("rows", (70, 512), ROWS, 32),            # 16384-element blocks + tail
        TensorSpec("odd", (45, 7), ROWS, 4),                # scalar (width 7)
        TensorSpec("bias", (300,), ELEMENT),
        TensorSpec("norm", (1000,), ROWS, 32),              # runs of 32-element blocks
        TensorSpec("wide", (33, 1040), ROWS, 16),           # 16640-element blocks, split
        TensorSpec("tt", (300, 160), TILE, 128, 64),        # tiles with clipped edge columns
        TensorSpec("vec1d", (5000,), TILE, 128, 128),       # 128x1 tiles, contiguous
    ]


def _multi_bucket_specs():
    out = []
    for b in range(3):
        out += [TensorSpec(f"w{b}", (96, 64), TILE, 32, 32, b),
                TensorSpec(f"r{b}", (50, 48), ROWS, 8, 0, b),
                TensorSpec(f"n{b}", (200,), ROWS, 32, 0, b)]
    return out


CASES = {
    "tiny": lambda: (synth.tiny().specs, 4, 16, 1e-2),
    "mixed": lambda: (_mixed_specs(), 5, 16, 1e-3),
    "mixed_g4": lambda: (_mixed_specs(), 3, 4, 1e-3),
    "multi_bucket": lambda: (_multi_bucket_specs(), 4, 16, 1e-3),
}


def _run_free(name, mode, chunk, steps=3, per_rank=False, warm=False, gscale=None, options=0):
    specs, m, g, sigma = CASES[name]()
    L = oracle.Layout(specs, m, g, order=options & rs.RS_ORDER_MASK,
                      align_unit=bool(options & rs.RS_ALIGN_CUT_UNIT))
    plan = make_plan(specs, m, g, chunk=chunk, mode=mode, options=options)
    check_plan_matches(plan, L)
    hs = host_state(L, specs, seed=0, sigma=sigma, warm=warm)
    ds = DevState(hs, with_out=True)
    ref = hs.copy()
    ref_out = np.zeros(L.total, dtype=np.uint16)
    pad = padding_mask(L)
    gs_dev = None
    if gscale is not None:
        gs_dev = torch.tensor([gscale], dtype=torch.float32, device="cuda")
    for t in range(1, steps + 1):
        if t > 1:
            gr = fresh_grads(L, specs, 0, sigma, t)
            ref.grad = gr
            ds.grad.copy_(u16_to_dev(gr))
        if per_rank:
            for b in range(L.nb):
                for r in range(m):
                    ds.step(plan, b, r, t, gscale=gs_dev)
        else:
            ds.step(plan, rs.RS_ALL, rs.RS_ALL, t, gscale=gs_dev)
        L.adam8_step(-1, -1, ref.theta, ref.grad, ref.qm, ref.qv, ref.am, ref.av,
                     oracle.HParams(step=t), gscale=1.0 if gscale is None else gscale,
                     out=ref_out)
        got = ds.host()
        assert_step_close(got, ref, mask=~pad, what=f"{name} step {t}")
        # codes and absmax come out exact; padding is never touched
        assert np.array_equal(got.qm, ref.qm) and np.array_equal(got.qv, ref.qv)
        assert np.array_equal(got.am, ref.am) and np.array_equal(got.av, ref.av)
        assert (got.qm[pad] == SENT_CODE).all() and (got.qv[pad] == SENT_CODE).all()
        assert (got.theta[pad] == 7.0).all()
        out = dev_to_u16(ds.out)
        assert (out[pad] == 0).all()
        assert np.array_equal(out[~pad], _torch_bf16(got.theta[~pad]))
    if mode != TWO:
        rs.rs_plan_check_device(plan.h)
    plan.free()
    return got


def _torch_bf16(x: np.ndarray) -> np.ndarray:
    """bf16 bits of float32 values by torch's round-to-nearest-even
    conversion: the fused output must be the bf16 of the returned master
    (a property of the kernel's own outputs; the oracle is not used on them)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("mode", [TWO, COOP, ORD])
@pytest.mark.parametrize("chunk", [None, 1024, 64])
@pytest.mark.parametrize("name", list(CASES))
def test_step_free_running(name, chunk, mode):
    log(f"step {name} chunk={chunk} mode={mode}")
    _run_free(name, mode, chunk)


@pytest.mark.parametrize("mode", [TWO, COOP, ORD])
def test_step_per_rank_calls_and_warm_states(mode):
    log(f"step per-rank warm mode={mode}")
    _run_free("mixed", mode, 1024, steps=2, per_rank=True, warm=True)
    _run_free("multi_bucket", mode, None, steps=2, per_rank=True, warm=True)


def test_step_with_device_grad_scale():
    log("step grad scale")
    _run_free("mixed", TWO, None, steps=2, gscale=0.25)
    _run_free("tiny", COOP, 64, steps=2, gscale=0.6180339)


def test_modes_and_chunk_sizes_agree_bitwise():
    specs, m, g, sigma = CASES["mixed"]()
    L = oracle.Layout(specs, m, g)
    hs = host_state(L, specs, seed=4, sigma=sigma, warm=True)
    results = []
    for mode, chunk in [(TWO, None), (COOP, None), (TWO, 256), (COOP, 64), (ORD, None), (ORD, 64)]:
        plan = make_plan(specs, m, g, chunk=chunk, mode=mode)
        ds = DevState(hs, with_out=True)
        for t in (11, 12):
            ds.step(plan, rs.RS_ALL, rs.RS_ALL, t)
        h = ds.host()
        results.append((h, dev_to_u16(ds.out)))
        plan.free()
    for h, o in results[1:]:
        for a, b in zip((h.theta, h.qm, h.qv, h.am, h.av, o),
                        (results[0][0].theta, results[0][0].qm, results[0][0].qv,
                         results[0][0].am, results[0][0].av, results[0][1])):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", [TWO, COOP, ORD])
def test_llama_layer_full_parity(mode):
    """The Llama-style layer (51.4M elements, 32-row blocks, 8 ranks): two
    free-running steps over every element."""
    w = synth.llama_layer_2048()
    log(f"llama layer full parity mode={mode}")
    L = oracle.Layout(w.specs, w.m, w.g_coll)
    plan = make_plan(w.specs, w.m, w.g_coll, mode=mode)
    check_plan_matches(plan, L)
    hs = host_state(L, w.specs, seed=0, sigma=w.grad_sigma, warm=False)
    ds = DevState(hs, with_out=True)
    ref = hs.copy()
    ref_out = np.zeros(L.total, dtype=np.uint16)
    pad = padding_mask(L)
    for t in (1, 2):
        if t > 1:
            gr = fresh_grads(L, w.specs, 0, w.grad_sigma, t)
            ref.grad = gr
            ds.grad.copy_(u16_to_dev(gr))
        ds.step(plan, rs.RS_ALL, rs.RS_ALL, t)
        L.adam8_step(-1, -1, ref.theta, ref.grad, ref.qm, ref.qv, ref.am, ref.av,
                     oracle.HParams(step=t), out=ref_out)
        got = ds.host()
        assert_step_close(got, ref, mask=~pad, what=f"llama layer step {t}")
        log(f"  step {t}: codes equal m={np.array_equal(got.qm, ref.qm)} "
            f"v={np.array_equal(got.qv, ref.qv)}; max |dtheta| "
            f"{np.abs(got.theta[~pad] - ref.theta[~pad]).max():.3e}")
    if mode != TWO:
        rs.rs_plan_check_device(plan.h)
    plan.free()


def test_step_is_deterministic():
    specs, m, g, sigma = CASES["mixed"]()
    L = oracle.Layout(specs, m, g)
    hs = host_state(L, specs, seed=9, sigma=sigma, warm=True)
    plan = make_plan(specs, m, g, chunk=512, mode=COOP)
    outs = []
    for _ in range(2):
        ds = DevState(hs)
        for t in (3, 4, 5):
            ds.step(plan, rs.RS_ALL, rs.RS_ALL, t)
        outs.append(ds.host())
    for a, b in zip((outs[0].theta, outs[0].qm, outs[0].qv, outs[0].am),
                    (outs[1].theta, outs[1].qm, outs[1].qv, outs[1].am)):
        assert np.array_equal(a, b)
    rs.rs_plan_check_device(plan.h)
    plan.free()


def test_zero_grad_zero_state_is_pure_decay():
    specs, m, g, sigma = CASES["mixed"]()
    L = oracle.Layout(specs, m, g)
    hs = host_state(L, specs, seed=1, sigma=sigma, warm=False)
    hs.grad[:] = 0
    plan = make_plan(specs, m, g)
    ds = DevState(hs)
    ds.step(plan, rs.RS_ALL, rs.RS_ALL, 7)
    got = ds.host()
    real = ~padding_mask(L)
    c = np.float32(1.0 - 1e-3 * 0.01)
    assert np.array_equal(got.theta[real], hs.theta[real] * c)
    assert not got.qm[real].any() and not got.qv[real].any() and not got.am.any()
    plan.free()


@pytest.mark.parametrize("options", [rs.RS_ORDER_BY_BLOCK, rs.RS_ORDER_BY_SIZE,
                                     rs.RS_ALIGN_CUT_UNIT | rs.RS_ORDER_BY_SIZE])
@pytest.mark.parametrize("name", ["mixed", "multi_bucket"])
def test_step_with_planner_orders(name, options):
    """Reordered plans: tensors sit in buffer order, block ids follow it."""
    log(f"step {name} options={options:#x}")
    _run_free(name, COOP, 1024, steps=2, options=options)


def _set_status_word(plan, value):
    off = rs.rs_plan_status_offset(plan.h)
    torch.cuda.synchronize()
    plan.workspace[off:off + 4].view(torch.int32).fill_(value)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", [COOP, ORD])
@pytest.mark.parametrize("name,chunk", [("mixed", 1024), ("mixed", 64), ("multi_bucket", 64)])
def test_status_word_set_takes_wait_free_path_exactly(name, chunk, mode):
    """With the device status word set before the launch (as after a wait
    that gave up), the one-launch step updates every split block whole in
    one workgroup, with no wait: results stay those of the oracle (codes
    exact), every kernel ends normally, and rs_plan_check_device reports and
    clears the word; the next steps take the waiting path again."""
    specs, m, g, sigma = CASES[name]()
    log(f"status word fallback {name} chunk={chunk} mode={mode}")
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g, chunk=chunk, mode=mode)
    hs = host_state(L, specs, seed=3, sigma=sigma, warm=True)
    ds = DevState(hs, with_out=True)
    ref = hs.copy()
    ref_out = np.zeros(L.total, dtype=np.uint16)
    pad = padding_mask(L)
    for t in (11, 12, 13):
        if t > 11:
            gr = fresh_grads(L, specs, 3, sigma, t)
            ref.grad = gr
            ds.grad.copy_(u16_to_dev(gr))
        if t < 13:
            _set_status_word(plan, 1)
        ds.step(plan, rs.RS_ALL, rs.RS_ALL, t)
        L.adam8_step(-1, -1, ref.theta, ref.grad, ref.qm, ref.qv, ref.am, ref.av,
                     oracle.HParams(step=t), out=ref_out)
        got = ds.host()
        assert_step_close(got, ref, mask=~pad, what=f"{name} step {t}")
        assert np.array_equal(got.qm, ref.qm) and np.array_equal(got.qv, ref.qv)
        assert np.array_equal(got.am, ref.am) and np.array_equal(got.av, ref.av)
        assert (got.qm[pad] == SENT_CODE).all() and (got.theta[pad] == 7.0).all()
        out = dev_to_u16(ds.out)
        assert np.array_equal(out[~pad], _torch_bf16(got.theta[~pad]))
        if t < 13:
            with pytest.raises(rs.RaggedShardError) as ei:
                rs.rs_plan_check_device(plan.h)
            assert ei.value.status == rs.RS_EHIP
        rs.rs_plan_check_device(plan.h)  # cleared
    plan.free()
