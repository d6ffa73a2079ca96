"""Full-size GPU parity on sampled blocks.

Inputs are generated on the device with torch's seeded generator; the
inputs of the sampled blocks are copied to the host before the first step,
the GPU runs two steps over the whole selection, and the oracle replays the
two steps on the sampled blocks alone (blocks never interact), so no oracle
input comes from the library."""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
import synth
from gpu_harness import HostState, assert_step_close, check_plan_matches, log, make_plan

pytestmark = pytest.mark.gpu


def _gen_full(total, nblocks, seed, sigma, warm, chunk=1 << 28):
    theta = torch.empty(total, dtype=torch.float32, device="cuda")
    grad = torch.empty(total, dtype=torch.int16, device="cuda")
    for i, lo in enumerate(range(0, total, chunk)):
        hi = min(total, lo + chunk)
        theta[lo:hi] = synth.uniform_params(hi - lo, seed, 100 + i, device="cuda")
        grad[lo:hi] = synth.normal_bf16(hi - lo, sigma, seed, 5000 + i, device="cuda").view(
            torch.int16)
    if warm:
        qm = torch.empty(total, dtype=torch.int8, device="cuda")
        qv = torch.empty(total, dtype=torch.uint8, device="cuda")
        for i, lo in enumerate(range(0, total, chunk)):
            hi = min(total, lo + chunk)
            qm[lo:hi] = synth.random_codes_m(hi - lo, seed, 9000 + i, device="cuda")
            qv[lo:hi] = synth.random_codes_v(hi - lo, seed, 9500 + i, device="cuda")
        am = synth.random_absmax(nblocks, 1e-3, seed, 77, device="cuda")
        av = synth.random_absmax(nblocks, 1e-6, seed, 78, device="cuda")
    else:
        qm = torch.zeros(total, dtype=torch.int8, device="cuda")
        qv = torch.zeros(total, dtype=torch.uint8, device="cuda")
        am = torch.zeros(nblocks, dtype=torch.float32, device="cuda")
        av = torch.zeros(nblocks, dtype=torch.float32, device="cuda")
    return theta, grad, qm, qv, am, av


def _sample_blocks(L, rank, n, rng, bucket_filter=None):
    """(tensor, block) pairs whose block lies in `rank` (oracle's view),
    plus the same number of blocks outside it."""
    inside, outside = [], []
    tries = 0
    while (len(inside) < n or len(outside) < n // 4) and tries < 200000:
        tries += 1
        t = int(rng.integers(0, len(L.specs)))
        if bucket_filter is not None and L.specs[t].bucket not in bucket_filter:
            continue
        k = int(rng.integers(0, L.derived[t].nblk))
        r = L.rank_of(L.block_first_position(t, k))
        if rank is None or r == rank:
            if len(inside) < n:
                inside.append((t, k))
        elif len(outside) < n // 4:
            outside.append((t, k))
    return inside, outside


def _gather(L, blocks, theta, grad, qm, qv, am, av):
    out = []
    for t, k in blocks:
        P = torch.from_numpy(L.block_positions(t, k)).cuda()
        b = L.blk0[t] + k
        out.append(dict(theta=theta[P].cpu().numpy(), grad=grad[P].cpu().numpy().view(np.uint16),
                        qm=qm[P].cpu().numpy(), qv=qv[P].cpu().numpy(), am=float(am[b]),
                        av=float(av[b])))
    return out


def _run(L, plan, rank_calls, steps, blocks_in, blocks_out, seed, sigma, warm, with_out=False):
    theta, grad, qm, qv, am, av = _gen_full(L.total, L.n_blocks, seed, sigma, warm)
    out = torch.zeros(L.total, dtype=torch.int16, device="cuda") if with_out else None
    before_in = _gather(L, blocks_in, theta, grad, qm, qv, am, av)
    before_out = _gather(L, blocks_out, theta, grad, qm, qv, am, av)
    grads_in = []
    for si, t in enumerate(steps):
        if si > 0:
            # fresh gradients for the next step (synthetic, device-generated)
            g2 = synth.normal_bf16(L.total, sigma, seed, 60000 + si, device="cuda").view(torch.int16)
            grad.copy_(g2)
            del g2
        grads_in.append([grad[torch.from_numpy(L.block_positions(tt, k)).cuda()].cpu().numpy()
                         .view(np.uint16) for tt, k in blocks_in])
        for (b, r) in rank_calls:
            rs.rs_adam8_step(plan.h, b, r, theta, grad, qm, qv, am, av, step=t, bf16_out=out)
        torch.cuda.synchronize()
        log(f"  step {t} done")
    after_in = _gather(L, blocks_in, theta, grad, qm, qv, am, av)
    after_out = _gather(L, blocks_out, theta, grad, qm, qv, am, av)
    # oracle replay of the sampled blocks
    for j, ((t_i, k), b0, b1) in enumerate(zip(blocks_in, before_in, after_in)):
        th, m8, v8, a_m, a_v = b0["theta"], b0["qm"], b0["qv"], b0["am"], b0["av"]
        o = None
        for si, t in enumerate(steps):
            th, m8, v8, a_m, a_v, o = oracle.adam8_block(th, grads_in[si][j], m8, v8, a_m, a_v,
                                                         oracle.HParams(step=t),
                                                         want_out=with_out)
        got = HostState(b1["theta"], None, b1["qm"], b1["qv"], np.array([b1["am"]], np.float32),
                        np.array([b1["av"]], np.float32))
        exp = HostState(th, None, m8, v8, np.array([a_m], np.float32), np.array([a_v], np.float32))
        assert_step_close(got, exp, what=f"block {t_i}/{k}")
        if with_out:
            P = torch.from_numpy(L.block_positions(t_i, k)).cuda()
            assert np.array_equal(out[P].cpu().numpy().view(np.uint16), oracle.bf16(b1["theta"]))
    # blocks outside the selected ranks are untouched
    for b0, b1 in zip(before_out, after_out):
        assert np.array_equal(b0["theta"], b1["theta"]) and np.array_equal(b0["qm"], b1["qm"])
        assert np.array_equal(b0["qv"], b1["qv"]) and b0["am"] == b1["am"]
    del theta, grad, qm, qv, am, av, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", [rs.RS_SPLIT_TWO_PASS, rs.RS_SPLIT_COOPERATIVE])
def test_llama8b_tiles_ranks_0_and_43(mode):
    """24 tiled layers, 64 ranks: the step of rank 0 (all of it in q) and of
    rank 43 (end of up, padding, start of down) over all 24 layer buckets."""
    w = synth.llama8b_tiles()
    log(f"llama8b tiles mode={mode}")
    L = oracle.Layout(w.specs, w.m, w.g_coll)
    plan = make_plan(w.specs, w.m, w.g_coll, mode=mode)
    check_plan_matches(plan, L)
    rng = np.random.default_rng(0)
    for rank in (0, 43):
        bi, bo = _sample_blocks(L, rank, 24, rng)
        _run(L, plan, [(rs.RS_ALL, rank)], [1, 2], bi, bo, seed=0, sigma=1e-3, warm=False)
    if mode == rs.RS_SPLIT_COOPERATIVE:
        rs.rs_plan_check_device(plan.h)
    plan.free()


@pytest.mark.parametrize("mode", [rs.RS_SPLIT_TWO_PASS, rs.RS_SPLIT_COOPERATIVE,
                                  rs.RS_SPLIT_ORDERED])
def test_moe_bucket_ranks_0_and_46_warm(mode):
    """Fused-expert MoE bucket, 48 ranks, 128-row blocks of 368,640
    elements (23 chunks each), warm states, steps 11 and 12."""
    w = synth.moe_bucket()
    log(f"moe mode={mode}")
    L = oracle.Layout(w.specs, w.m, w.g_coll)
    plan = make_plan(w.specs, w.m, w.g_coll, mode=mode)
    check_plan_matches(plan, L)
    rng = np.random.default_rng(1)
    for rank in (0, 46):
        bi, bo = _sample_blocks(L, rank, 6, rng)
        _run(L, plan, [(0, rank)], [11, 12], bi, bo, seed=0, sigma=1e-3, warm=True)
    if mode != rs.RS_SPLIT_TWO_PASS:
        rs.rs_plan_check_device(plan.h)
    plan.free()


def test_llama8b_full_state_single_rank():
    """Whole 8.03e9-element state on one rank (int64 indexing past 2^32),
    32-row blocks up to 458,752 elements, fused bf16 output."""
    w = synth.llama8b_full()
    log("llama8b full")
    L = oracle.Layout(w.specs, w.m, w.g_coll)
    plan = make_plan(w.specs, w.m, w.g_coll, mode=rs.RS_SPLIT_COOPERATIVE)
    check_plan_matches(plan, L)
    rng = np.random.default_rng(2)
    bi, _ = _sample_blocks(L, None, 12, rng)
    # always include blocks of the last tensor (positions beyond 2^32)
    last = len(w.specs) - 1
    bi += [(last, 0), (last, L.derived[last].nblk - 1)]
    _run(L, plan, [(rs.RS_ALL, rs.RS_ALL)], [1, 2], bi, [], seed=0, sigma=1e-3, warm=False,
         with_out=True)
    rs.rs_plan_check_device(plan.h)
    plan.free()


def test_pack_unpack_full_size_sampled():
    """Pack of one tiled layer bucket and of the MoE bucket, checked at
    sampled positions; unpack of the MoE bucket checked on sampled ranges."""
    for w in (synth.llama8b_tiles(layers=1), synth.moe_bucket()):
        log(f"pack/unpack {w.name}")
        L = oracle.Layout(w.specs, w.m, w.g_coll)
        plan = make_plan(w.specs, w.m, w.g_coll)
        views = [synth.uniform_params(s.numel, 0, i, device="cuda") for i, s in enumerate(w.specs)]
        rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, views)
        buf = torch.full((L.total,), 0x3333, dtype=torch.int16, device="cuda")
        rs.rs_pack_shard(plan.h, rs.RS_ALL, rs.RS_ALL, buf)
        rng = np.random.default_rng(3)
        pos = np.unique(np.concatenate([rng.integers(0, L.total, 200000),
                                        np.array(L.pos), np.array(L.pos) - 1,
                                        np.array([L.total - 1])]))
        pos = pos[(pos >= 0) & (pos < L.total)]
        got = buf[torch.from_numpy(pos).cuda()].cpu().numpy().view(np.uint16)
        exp = np.zeros(pos.size, dtype=np.uint16)
        for i, s in enumerate(w.specs):
            sel = (pos >= L.pos[i]) & (pos < L.pos[i] + s.numel)
            idx = torch.from_numpy(pos[sel] - L.pos[i]).cuda()
            exp[sel] = oracle.bf16(views[i][idx].cpu().numpy())
        assert np.array_equal(got, exp)
        dst = [torch.zeros(s.numel, dtype=torch.int16, device="cuda") for s in w.specs]
        rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, dst)
        rs.rs_unpack_full(plan.h, rs.RS_ALL, buf)
        for i, s in enumerate(w.specs):
            lo = int(rng.integers(0, max(1, s.numel - 4096)))
            a = dst[i][lo:lo + 4096].cpu().numpy().view(np.uint16)
            b = buf[L.pos[i] + lo:L.pos[i] + lo + 4096].cpu().numpy().view(np.uint16)
            assert np.array_equal(a, b)
            assert np.array_equal(dst[i][-8:].cpu().numpy(), buf[L.pos[i] + s.numel - 8:
                                                                  L.pos[i] + s.numel].cpu().numpy())
        plan.free()
        del views, buf, dst
        torch.cuda.empty_cache()
