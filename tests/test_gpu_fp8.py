"""GPU parity of the FP8 copy-in (E4M3 codes + one scale per quantisation
block) and its copy-out against the oracle: bit-exact codes, scales and
bf16 views."""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
import synth
from synth import ELEMENT, ROWS, TILE, TensorSpec
from gpu_harness import check_plan_matches, dev_to_u16, log, make_plan

pytestmark = pytest.mark.gpu


def _kinds_specs():
    # every chunk kind of the FP8 table (16384-element chunks): whole tiles,
    # split row blocks (> 16384 elements), runs of small blocks, scalar
    # blocks (odd widths), element runs, ragged edges
    return [
        TensorSpec("tile128", (300, 256), TILE, 128, 128),  # 128x128 tiles + clipped band
        TensorSpec("rows_big", (40, 1040), ROWS, 32),       # 33280-element blocks: split
        TensorSpec("tile32", (96, 64), TILE, 32, 32),
        TensorSpec("odd", (45, 7), ROWS, 4),                # scalar
        TensorSpec("bias", (300,), ELEMENT),
        TensorSpec("norm", (1000,), ROWS, 32),              # runs of 32-element blocks
        TensorSpec("tt", (300, 160), TILE, 128, 64),        # clipped columns
    ]


CASES = {
    "kinds": lambda: (_kinds_specs(), 3, 16),
    "tiny": lambda: (synth.tiny().specs, 4, 16),
    "small_tiled_layer": lambda: (synth._llama_layer(512, 1408, 128, TILE, 128, 128, 0), 8, 16),
}


def _views(specs, seed):
    hv = []
    for i, s in enumerate(specs):
        v = synth.uniform_params(s.numel, seed, i).numpy()
        # a spread of magnitudes inside blocks, and an all-zero stretch
        if s.numel > 64:
            v[: s.numel // 7] *= np.float32(1e-3)
            v[-16:] = 0.0
        hv.append(v)
    return hv


def _check_pack(L, plan, hv, dv, bucket, rank):
    buf = torch.full((L.total,), 0x5A, dtype=torch.uint8, device="cuda")
    sc = torch.full((L.n_blocks,), -1.0, dtype=torch.float32, device="cuda")
    rs.rs_pack_shard_fp8(plan.h, bucket, rank, buf, sc)
    exp = np.full(L.total, 0x5A, dtype=np.uint8)
    esc = np.full(L.n_blocks, -1.0, dtype=np.float32)
    L.pack_fp8(bucket, rank, hv, exp, esc)
    got = buf.cpu().numpy()
    bad = np.nonzero(got != exp)[0]
    if bad.size:
        x = np.zeros(L.total, dtype=np.float32)
        for t, v in enumerate(hv):
            x[L.pos[t]:L.pos[t] + v.size] = v
        detail = [(int(i), float(x[i]), int(got[i]), int(exp[i])) for i in bad[:6]]
        raise AssertionError(f"{bad.size} codes differ; (pos, x, got, expected): {detail}")
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), esc.view(np.uint32))
    return buf, sc, exp, esc


@pytest.mark.parametrize("mode", [rs.RS_SPLIT_TWO_PASS, rs.RS_SPLIT_COOPERATIVE,
                                  rs.RS_SPLIT_ORDERED])
@pytest.mark.parametrize("name", list(CASES))
def test_fp8_pack_unpack_bitexact(name, mode):
    specs, m, g = CASES[name]()
    log(f"fp8 {name} mode={mode}")
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g, mode=mode)
    check_plan_matches(plan, L)
    hv = _views(specs, 7)
    dv = [torch.from_numpy(v).cuda() for v in hv]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dv)
    buf, sc, hbuf, hsc = _check_pack(L, plan, hv, dv, rs.RS_ALL, rs.RS_ALL)
    # per-slice calls touch only their slice and reproduce the whole
    for r in sorted({0, m // 2, m - 1}):
        _check_pack(L, plan, hv, dv, rs.RS_ALL, r)
    # copy-out
    outs = [torch.zeros(s.numel, dtype=torch.int16, device="cuda") for s in specs]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, outs)
    rs.rs_unpack_full_fp8(plan.h, rs.RS_ALL, buf, sc)
    hexp = [np.zeros(s.numel, dtype=np.uint16) for s in specs]
    L.unpack_fp8(-1, hexp, hbuf, hsc)  # the oracle's own pack, equal to the device's
    for s, o, e in zip(specs, outs, hexp):
        assert np.array_equal(dev_to_u16(o), e), s.name
    if mode != rs.RS_SPLIT_TWO_PASS:
        rs.rs_plan_check_device(plan.h)
    plan.free()


def _every_code_and_tie():
    """Magnitudes <= 448 that hit every finite E4M3 value, every midpoint
    between neighbours (ties to even) and the binary32 neighbours of each
    midpoint, with both signs; 1024 values whose absmax is 448 (so s = 1)."""
    pos = np.array([oracle.e4m3_to_f32(c) for c in range(127)], dtype=np.float32)
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)  # exact
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    a = np.concatenate([pos, mids, up, dn])
    v = np.concatenate([a, -a, np.zeros(1024 - 2 * a.size, dtype=np.float32)])
    v[-7:] = -0.0
    assert v.size == 1024 and np.abs(v).max() == 448.0
    return v


@pytest.mark.parametrize("options", [rs.RS_ORDER_BY_BLOCK, rs.RS_ORDER_BY_SIZE,
                                     rs.RS_ALIGN_CUT_UNIT | rs.RS_ORDER_BY_SIZE])
def test_fp8_pack_unpack_bitexact_on_reordered_plans(options):
    """Tensors in buffer order different from the given order: block ids
    (scales) and positions follow the planner's order on both sides."""
    specs, m, g = CASES["kinds"]()
    log(f"fp8 reordered options={options:#x}")
    L = oracle.Layout(specs, m, g, order=options & rs.RS_ORDER_MASK,
                      align_unit=bool(options & rs.RS_ALIGN_CUT_UNIT))
    plan = make_plan(specs, m, g, options=options)
    check_plan_matches(plan, L)
    hv = _views(specs, 13)
    dv = [torch.from_numpy(v).cuda() for v in hv]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dv)
    buf, sc, hbuf, hsc = _check_pack(L, plan, hv, dv, rs.RS_ALL, rs.RS_ALL)
    for r in (0, m - 1):
        _check_pack(L, plan, hv, dv, rs.RS_ALL, r)
    outs = [torch.zeros(s.numel, dtype=torch.int16, device="cuda") for s in specs]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, outs)
    rs.rs_unpack_full_fp8(plan.h, rs.RS_ALL, buf, sc)
    hexp = [np.zeros(s.numel, dtype=np.uint16) for s in specs]
    L.unpack_fp8(-1, hexp, hbuf, hsc)
    for s, o, e in zip(specs, outs, hexp):
        assert np.array_equal(dev_to_u16(o), e), s.name
    rs.rs_plan_check_device(plan.h)
    plan.free()


def test_fp8_every_code_and_tie():
    """The E4M3 rounding of the copy-in on every code and every tie, in the
    three vector paths (whole contiguous blocks, 128 x 128 tiles, runs of
    small blocks), plus a block whose scale is a binary32 subnormal (its
    quotients can pass 448 and saturate) and an all-zero block."""
    specs = [TensorSpec("rows", (5, 1024), ROWS, 1),
             TensorSpec("tiles", (256, 256), TILE, 128, 128),
             TensorSpec("small", (64, 64), ROWS, 1)]
    m, g = 2, 16
    log("fp8 every code and tie")
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    check_plan_matches(plan, L)
    A = _every_code_and_tie()
    rng = np.random.default_rng(11)
    rows = np.stack([A, rng.permutation(A),
                     np.float32(2e-38) * np.linspace(-1, 1, 1024, dtype=np.float32),
                     # absmax / 448 = 1.4 * 2^-149 rounds to s = 2^-149: quotients up to 627
                     np.float32(448 * 1.4 * 2.0 ** -149) * np.linspace(-1, 1, 1024, dtype=np.float32),
                     np.where(np.arange(1024) % 2 == 0, 0.0, -0.0).astype(np.float32)])
    tiles = np.concatenate([rng.permutation(A) for _ in range(64)]).reshape(256, 256)
    small = rng.permutation(A).reshape(16, 64).repeat(4, axis=0)
    small[:, 0] = 448.0  # every 64-element block holds the absmax
    hv = [rows.reshape(-1).astype(np.float32), tiles.reshape(-1).astype(np.float32),
          small.reshape(-1).astype(np.float32)]
    dv = [torch.from_numpy(v).cuda() for v in hv]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dv)
    buf, sc, hbuf, hsc = _check_pack(L, plan, hv, dv, rs.RS_ALL, rs.RS_ALL)
    outs = [torch.zeros(s.numel, dtype=torch.int16, device="cuda") for s in specs]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, outs)
    rs.rs_unpack_full_fp8(plan.h, rs.RS_ALL, buf, sc)
    hexp = [np.zeros(s.numel, dtype=np.uint16) for s in specs]
    L.unpack_fp8(-1, hexp, hbuf, hsc)  # the oracle's own pack, equal to the device's
    for s, o, e in zip(specs, outs, hexp):
        assert np.array_equal(dev_to_u16(o), e), s.name
    plan.free()


@pytest.mark.parametrize("w", ["llama8b_tiles_1layer", "moe"])
def test_fp8_full_size_sampled_blocks(w):
    """Full-size buckets: the whole bucket on the GPU, sampled blocks
    recomputed by the oracle's block rule (blocks are independent)."""
    wl = synth.llama8b_tiles(layers=1) if w != "moe" else synth.moe_bucket()
    log(f"fp8 full {w}")
    L = oracle.Layout(wl.specs, wl.m, wl.g_coll)
    plan = make_plan(wl.specs, wl.m, wl.g_coll)
    check_plan_matches(plan, L)
    dv = [synth.uniform_params(s.numel, 3, i, device="cuda") for i, s in enumerate(wl.specs)]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dv)
    buf = torch.zeros(L.total, dtype=torch.uint8, device="cuda")
    sc = torch.zeros(L.n_blocks, dtype=torch.float32, device="cuda")
    rs.rs_pack_shard_fp8(plan.h, rs.RS_ALL, rs.RS_ALL, buf, sc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for _ in range(12):
        t = int(rng.integers(0, len(wl.specs)))
        k = int(rng.integers(0, L.derived[t].nblk))
        P = L.block_positions(t, k)
        x = dv[t][torch.from_numpy(P - L.pos[t]).cuda()].cpu().numpy()
        s, q = oracle.fp8_block(x)
        got = buf[torch.from_numpy(P).cuda()].cpu().numpy()
        assert np.array_equal(got, q), (t, k)
        assert np.float32(sc[L.blk0[t] + k].item()) == np.float32(s)
    rs.rs_plan_check_device(plan.h)
    plan.free()


@pytest.mark.parametrize("mode", [rs.RS_SPLIT_COOPERATIVE, rs.RS_SPLIT_ORDERED])
def test_fp8_status_word_set_takes_wait_free_path_exactly(mode):
    """With the device status word set before the launch, the one-launch
    FP8 copy-in encodes every split block whole in one workgroup (no wait):
    codes and scales stay bit-exact, and rs_plan_check_device reports and
    clears the word."""
    specs, m, g = CASES["kinds"]()
    log(f"fp8 status word fallback mode={mode}")
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g, mode=mode)
    hv = _views(specs, 11)
    dv = [torch.from_numpy(v).cuda() for v in hv]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, dv)
    off = rs.rs_plan_status_offset(plan.h)
    for rank in (rs.RS_ALL, 0, m - 1):
        torch.cuda.synchronize()
        plan.workspace[off:off + 4].view(torch.int32).fill_(1)
        _check_pack(L, plan, hv, dv, rs.RS_ALL, rank)
        with pytest.raises(rs.RaggedShardError) as ei:
            rs.rs_plan_check_device(plan.h)
        assert ei.value.status == rs.RS_EHIP
    _check_pack(L, plan, hv, dv, rs.RS_ALL, rs.RS_ALL)
    rs.rs_plan_check_device(plan.h)
    plan.free()
