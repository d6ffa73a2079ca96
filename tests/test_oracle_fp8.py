"""Pins of the oracle's FP8 copy-in (OCP E4M3 codes with one fp32 scale per
quantisation block; block-wise FP8 as named on the veScale-FSDP page,
section 'Problem and motivation'; scaling rule of this library).  The E4M3
conversion is checked against torch's float8_e4m3fn, an implementation of
the same OCP format; the block packing against invariants of the rule."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import ELEMENT, ROWS, TILE, TensorSpec


def _torch_code(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def _codes(x: np.ndarray) -> np.ndarray:
    return np.array([oracle.e4m3(float(v)) for v in x], dtype=np.uint8)


def test_decode_table_matches_torch():
    q = torch.arange(256, dtype=torch.uint8)
    ref = q.view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        v = oracle.e4m3_to_f32(c)
        if np.isnan(ref[c]):
            assert np.isnan(v) and (c & 0x7f) == 0x7f
        else:
            assert v == ref[c], c


def test_encode_matches_torch_below_overflow():
    vals = np.array([oracle.e4m3_to_f32(c) for c in range(0x7f)], dtype=np.float64)
    mids = (vals[:-1] + vals[1:]) / 2                   # exact ties (binary64 is exact here)
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-14, np.log2(463.0), size=20000))
    xs = np.concatenate([vals, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                         np.nextafter(mids.astype(np.float32), np.float32(1e9)), mags])
    xs = np.concatenate([xs, -xs, [0.0, -0.0]]).astype(np.float32)
    xs = xs[np.abs(xs) < 464.0]
    np.testing.assert_array_equal(_codes(xs), _torch_code(xs))


def test_encode_saturates_and_nan():
    for x in (464.0, 480.0, 1e6, np.inf):
        assert oracle.e4m3(x) == 0x7e and oracle.e4m3(-x) == 0xfe
    assert oracle.e4m3(np.nan) & 0x7f == 0x7f


def _layout_and_views(specs, m, g, seed=0):
    L = oracle.Layout(specs, m, g)
    views = [synth.uniform_params(s.numel, seed, i).numpy() for i, s in enumerate(specs)]
    return L, views


def _specs():
    return [TensorSpec("tile", (200, 96), TILE, 32, 32), TensorSpec("rows", (70, 48), ROWS, 16),
            TensorSpec("bias", (50,), ELEMENT), TensorSpec("zero", (64, 16), ROWS, 8)]


def test_block_rule_invariants():
    specs = _specs()
    L, views = _layout_and_views(specs, 3, 16)
    views[3][:] = 0.0                                    # an all-zero tensor: scale 0, codes 0
    buf = np.full(L.total, 0x55, dtype=np.uint8)
    sc = np.full(L.n_blocks, -1.0, dtype=np.float32)
    L.pack_fp8(-1, -1, views, buf, sc)
    for t, s in enumerate(specs):
        for k in range(L.derived[t].nblk):
            P = L.block_positions(t, k)
            x = views[t][P - L.pos[t]]
            a = np.abs(x).max()
            scale = sc[L.blk0[t] + k]
            if a == 0:
                assert scale == 0 and (buf[P] == 0).all()
                continue
            # the largest element maps to the largest code, +-448
            i = int(np.argmax(np.abs(x)))
            assert buf[P[i]] & 0x7f == 0x7e
            assert scale > 0 and abs(scale * 448 - a) <= 2 * np.spacing(np.float32(a))
            # dequantised values lie within half an E4M3 step of x / scale
            deq = np.array([oracle.e4m3_to_f32(c) for c in buf[P]], dtype=np.float64) * scale
            r = np.abs(x / scale)
            half_step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(r, 2.0 ** -6))) - 4),
                                   2.0 ** -10)
            assert (np.abs(deq - x) <= scale * half_step * (1 + 1e-6) + 1e-30).all()
    # padding is zero
    mask = np.ones(L.total, bool)
    for t, s in enumerate(specs):
        mask[L.pos[t]:L.pos[t] + s.numel] = False
    assert (buf[mask] == 0).all()


def test_rank_packs_compose_and_element_blocks():
    specs = _specs()
    L, views = _layout_and_views(specs, 4, 16, seed=1)
    full = np.zeros(L.total, np.uint8)
    fs = np.zeros(L.n_blocks, np.float32)
    L.pack_fp8(-1, -1, views, full, fs)
    part = np.full(L.total, 0x77, np.uint8)
    ps = np.zeros(L.n_blocks, np.float32)
    for r in range(4):
        L.pack_fp8(-1, r, views, part, ps)
    assert np.array_equal(full, part) and np.array_equal(fs, ps)
    # element blocks: every element is its own block, so its code is +-448
    t = 2
    P = L.pos[t] + np.arange(specs[t].numel)
    assert np.all(full[P] & 0x7f == 0x7e)
    # and the copy-out gives bf16(x) back to within one bf16 step
    outs = [np.zeros(s.numel, np.uint16) for s in specs]
    L.unpack_fp8(-1, outs, full, fs)
    got = oracle.bf16_to_f32(outs[t]).astype(np.float64)
    ref = oracle.bf16_to_f32(oracle.bf16(views[t])).astype(np.float64)
    assert (np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7).all()


def test_unpack_round_trip_error():
    specs = _specs()
    L, views = _layout_and_views(specs, 2, 16, seed=2)
    buf = np.zeros(L.total, np.uint8)
    sc = np.zeros(L.n_blocks, np.float32)
    L.pack_fp8(-1, -1, views, buf, sc)
    outs = [np.zeros(s.numel, np.uint16) for s in specs]
    L.unpack_fp8(-1, outs, buf, sc)
    for t, s in enumerate(specs):
        x = views[t].astype(np.float64)
        got = oracle.bf16_to_f32(outs[t]).astype(np.float64)
        amax = max(np.abs(x).max(), 1e-30)
        # E4M3 keeps 3 mantissa bits: relative error 2^-4 of the value, or
        # 2^-10 of the block scale near zero; bf16 adds 2^-9
        bound = np.abs(x) * (2.0 ** -4 + 2.0 ** -8) + amax / 448 * 2.0 ** -9
        assert (np.abs(got - x) <= bound).all(), s.name
