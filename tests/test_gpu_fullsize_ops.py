"""Full-size GPU parity of the copy-in / copy-out and the group ops against
the oracle, element by element, on the large workloads:
  - the standalone copy-in of the whole 8.03e9-element state at m = 1
    (positions beyond 2^32, every padding gap), tensor by tensor;
  - the whole fused-expert MoE bucket: copy-in against orc_pack and copy-out
    against orc_unpack;
  - l2norm / zero / scale on rank 43 of the 24-bucket tiled model (24
    slices), on the MoE bucket (all ranks, and rank 46) and on the whole
    m = 1 state.
Inputs are generated on the device with torch's seeded generator and copied
to the host before the library runs, so no oracle input comes from the
library.  Host buffers of full-bucket-set size are allocated with
np.zeros (pages that are never written are never backed), and only the
selected slices are filled."""
import math

import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
import synth
from gpu_harness import check_plan_matches, log, make_plan

pytestmark = pytest.mark.gpu

SENT = 0x3C3C  # bf16 1.1767578 -- marks positions outside the selection


def _slices(L, bucket, rank):
    """[lo, hi) buffer ranges of the selection."""
    out = []
    for b in range(L.nb):
        if bucket != rs.RS_ALL and b != bucket:
            continue
        if rank == rs.RS_ALL:
            out.append((L.base[b], L.base[b] + L.m * L.S[b]))
        else:
            lo = L.base[b] + rank * L.S[b]
            out.append((lo, lo + L.S[b]))
    return out


def _fill_random_bf16(dev, lo, hi, seed, stream, chunk=1 << 28):
    for i, a in enumerate(range(lo, hi, chunk)):
        b = min(hi, a + chunk)
        dev[a:b] = synth.normal_bf16(b - a, 1e-3, seed, stream * 4096 + i,
                                     device="cuda").view(torch.int16)


def _d2h_into(host, dev, lo, hi, chunk=1 << 28):
    for a in range(lo, hi, chunk):
        b = min(hi, a + chunk)
        host[a:b] = dev[a:b].cpu().numpy().view(np.uint16)


def _equal_on(host, dev, lo, hi, chunk=1 << 28):
    for a in range(lo, hi, chunk):
        b = min(hi, a + chunk)
        if not np.array_equal(dev[a:b].cpu().numpy().view(np.uint16), host[a:b]):
            return False
    return True


def test_pack_llama8b_full_bitexact_every_tensor_and_gap():
    """Standalone copy-in of the whole m = 1 state (8.03e9 elements, the
    last tensor past 2^32), compared with the oracle's bf16 rule tensor by
    tensor; every padding gap must be zero."""
    w = synth.llama8b_full()
    log("pack llama8b_full")
    L = oracle.Layout(w.specs, w.m, w.g_coll)
    plan = make_plan(w.specs, w.m, w.g_coll)
    check_plan_matches(plan, L)
    assert L.pos[-1] + w.specs[-1].numel > (1 << 32)
    theta = torch.empty(L.total, dtype=torch.float32, device="cuda")
    chunk = 1 << 28
    for i, a in enumerate(range(0, L.total, chunk)):
        b = min(L.total, a + chunk)
        theta[a:b] = synth.uniform_params(b - a, 0, 300 + i, device="cuda")
    views = [theta[L.pos[i]:L.pos[i] + s.numel] for i, s in enumerate(w.specs)]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, views)
    buf = torch.full((L.total,), SENT, dtype=torch.int16, device="cuda")
    rs.rs_pack_shard(plan.h, rs.RS_ALL, rs.RS_ALL, buf)
    torch.cuda.synchronize()
    prev_end = 0
    for i, s in enumerate(w.specs):
        p = L.pos[i]
        if p > prev_end:  # padding gap before tensor i
            assert not buf[prev_end:p].cpu().numpy().any(), f"gap before {s.name}"
        for a in range(0, s.numel, chunk):
            b = min(s.numel, a + chunk)
            exp = oracle.bf16(views[i][a:b].cpu().numpy())
            got = buf[p + a:p + b].cpu().numpy().view(np.uint16)
            assert np.array_equal(got, exp), f"{s.name} [{a}, {b})"
        prev_end = p + s.numel
    if prev_end < L.total:
        assert not buf[prev_end:].cpu().numpy().any(), "trailing padding"
    log(f"  {len(w.specs)} tensors and their gaps match")
    plan.free()
    del theta, views, buf
    torch.cuda.empty_cache()


def test_moe_pack_unpack_whole_bucket_against_oracle():
    """The whole MoE bucket (48 ranks, 814M buffer elements): copy-in
    against orc_pack and copy-out against orc_unpack, every element."""
    w = synth.moe_bucket()
    log("moe pack/unpack whole bucket")
    L = oracle.Layout(w.specs, w.m, w.g_coll)
    plan = make_plan(w.specs, w.m, w.g_coll)
    check_plan_matches(plan, L)
    dviews = [synth.uniform_params(s.numel, 0, 40 + i, device="cuda")
              for i, s in enumerate(w.specs)]
    hviews = [v.cpu().numpy() for v in dviews]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dviews)
    buf = torch.full((L.total,), SENT, dtype=torch.int16, device="cuda")
    rs.rs_pack_shard(plan.h, rs.RS_ALL, rs.RS_ALL, buf)
    hbuf = np.full(L.total, SENT, dtype=np.uint16)
    L.pack(-1, -1, hviews, hbuf)
    assert _equal_on(hbuf, buf, 0, L.total), "pack"
    # per-rank copy-in of the raggedest rank touches only its slice
    buf.fill_(SENT)
    rs.rs_pack_shard(plan.h, 0, 46, buf)
    h46 = np.full(L.total, SENT, dtype=np.uint16)
    L.pack(0, 46, hviews, h46)
    assert _equal_on(h46, buf, 0, L.total), "pack rank 46"
    del h46, dviews
    # copy-out of an independent random bf16 buffer into separate views
    hsrc = np.zeros(L.total, dtype=np.uint16)
    src = torch.empty(L.total, dtype=torch.int16, device="cuda")
    _fill_random_bf16(src, 0, L.total, 0, 7)
    _d2h_into(hsrc, src, 0, L.total)
    outs = [torch.full((s.numel,), 0x7777, dtype=torch.int16, device="cuda") for s in w.specs]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, outs)
    rs.rs_unpack_full(plan.h, rs.RS_ALL, src)
    hout = [np.zeros(s.numel, dtype=np.uint16) for s in w.specs]
    L.unpack(-1, hout, hsrc)
    for i, s in enumerate(w.specs):
        assert _equal_on(hout[i], outs[i], 0, s.numel), f"unpack {s.name}"
    plan.free()
    del buf, src, outs
    torch.cuda.empty_cache()


def _group_ops_case(specs, m, g_coll, selections, seed):
    L = oracle.Layout(specs, m, g_coll)
    plan = make_plan(specs, m, g_coll)
    check_plan_matches(plan, L)
    dev = torch.full((L.total,), SENT, dtype=torch.int16, device="cuda")
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    for si, (bucket, rank) in enumerate(selections):
        log(f"  selection bucket={bucket} rank={rank}")
        sl = _slices(L, bucket, rank)
        host = np.zeros(L.total, dtype=np.uint16)  # lazily backed: only the selection is filled
        for k, (lo, hi) in enumerate(sl):
            _fill_random_bf16(dev, lo, hi, seed, 100 * si + k)
            _d2h_into(host, dev, lo, hi)
        # l2norm: squares and sum in binary64, 1e-5 relative on the norm
        rs.rs_group_l2norm(plan.h, bucket, rank, dev, rs.RS_BF16, sumsq)
        got = float(sumsq.item())
        exp = L.group_sumsq(bucket, rank, host)
        assert exp > 0 and math.isclose(math.sqrt(got), math.sqrt(exp), rel_tol=1e-5), (got, exp)
        # scale: bf16(float(x) * s), bit-exact
        s = 0.6180339887
        rs.rs_group_scale(plan.h, bucket, rank, dev, rs.RS_BF16, s)
        L.group_scale(bucket, rank, host, s)
        for lo, hi in sl:
            assert _equal_on(host, dev, lo, hi), ("scale", lo, hi)
        # zero
        rs.rs_group_zero(plan.h, bucket, rank, dev, rs.RS_BF16)
        for lo, hi in sl:
            assert _equal_on(np.zeros(hi - lo, np.uint16), dev[lo:hi], 0, hi - lo), ("zero", lo)
        # the neighbours of every selected slice kept the marker
        for lo, hi in sl:
            for p in (lo - 1, hi):
                if 0 <= p < L.total and not any(a <= p < b for a, b in sl):
                    assert int(dev[p].item()) & 0xFFFF == SENT, ("outside touched", p)
        for lo, hi in sl:
            dev[lo:hi].fill_(SENT)
        del host
    plan.free()
    del dev
    torch.cuda.empty_cache()


def test_group_ops_llama8b_tiles_rank43():
    """Rank 43 of the 24-bucket, 64-rank tiled model: its 24 slices (the end
    of up, padding, the start of down in every layer)."""
    w = synth.llama8b_tiles()
    log("group ops llama8b_tiles rank 43")
    _group_ops_case(w.specs, w.m, w.g_coll, [(rs.RS_ALL, 43), (5, 43)], seed=11)


def test_group_ops_moe_all_ranks_and_rank46():
    w = synth.moe_bucket()
    log("group ops moe")
    _group_ops_case(w.specs, w.m, w.g_coll, [(rs.RS_ALL, rs.RS_ALL), (0, 46), (0, 47)], seed=12)


def test_group_ops_llama8b_full():
    """The whole m = 1 state: 8.03e9 bf16 gradients (16 GB)."""
    w = synth.llama8b_full()
    log("group ops llama8b_full")
    _group_ops_case(w.specs, w.m, w.g_coll, [(rs.RS_ALL, rs.RS_ALL)], seed=13)


def _special_f32():
    bits = np.array([
        0x7FA00000, 0xFF800001, 0x7FC00000, 0xFFFFFFFF, 0x7F800001, 0xFFC12345,  # NaNs
        0x7F800000, 0xFF800000,                                                  # infinities
        0x00000001, 0x807FFFFF, 0x00400000, 0x00008000, 0x00018000, 0x00008001,  # subnormals
        0x80008000, 0x007FFFFF, 0x00800000, 0x80000000, 0x00000000,
        0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7F8000,                          # overflow to inf
        0x3F808000, 0x3F818000, 0x3F808001, 0xBF808000,                          # ties
    ], dtype=np.uint32)
    return bits.view(np.float32)


def test_pack_nan_payloads_and_subnormals_match_oracle():
    """The copy-in's bf16 rule on NaN payloads (quiet NaN with the sign
    kept), subnormals, ties and overflow, in the 16-byte vector body and in
    the scalar head/tail of a tensor."""
    w = synth.tiny()
    L = oracle.Layout(w.specs, w.m, w.g_coll)
    plan = make_plan(w.specs, w.m, w.g_coll)
    sp = _special_f32()
    hv = [synth.uniform_params(s.numel, 9, i).numpy() for i, s in enumerate(w.specs)]
    for i, v in enumerate(hv):
        n = min(v.size, sp.size)
        v[:n] = sp[:n]                       # head of every tensor
        v[v.size // 2:v.size // 2 + n] = sp[:n]  # middle (vector body)
        v[v.size - n:] = sp[:n]              # tail
    dv = [torch.from_numpy(v.copy()).cuda() for v in hv]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dv)
    buf = torch.full((L.total,), SENT, dtype=torch.int16, device="cuda")
    rs.rs_pack_shard(plan.h, rs.RS_ALL, rs.RS_ALL, buf)
    exp = np.full(L.total, SENT, dtype=np.uint16)
    L.pack(-1, -1, hv, exp)
    got = buf.cpu().numpy().view(np.uint16)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, [(int(p), hex(int(got[p])), hex(int(exp[p]))) for p in bad[:8]]
    plan.free()
