"""Host side of distributed Muon through the C-ABI (no GPU): SelectRoot and
the uneven root layout against the oracle, and the argument checks."""
import numpy as np
import pytest

import sharded_state_raggedshard_amd as rs
import synth
from oracle import muon as om
from synth import ELEMENT, ROWS, TILE, TensorSpec


def _check(specs, m, g, mats):
    plan = rs.Plan(specs, m, g)
    mu = rs.Muon(plan, mats)
    shapes = []
    for i in mats:
        s = specs[i]
        C = s.shape[-1] if len(s.shape) >= 2 else 1
        shapes.append((s.numel // C, C))
    roots = om.select_roots(shapes, m)
    off, reg = om.root_layout([R * C for R, C in shapes], roots, m, 64)
    assert mu.roots == roots and mu.offsets == off and mu.regions == reg
    assert mu.root_elems == reg[-1]
    assert rs.rs_muon_device_bytes(mu.h) > 0
    mu.free()
    plan.free()


def test_llama_layer_roots_and_layout():
    w = synth.llama_layer_2048()
    _check(w.specs, w.m, w.g_coll, [i for i, s in enumerate(w.specs) if len(s.shape) == 2])


def test_tiled_layers_roots_and_layout():
    w = synth.llama8b_tiles(layers=2)
    _check(w.specs, w.m, w.g_coll, [i for i, s in enumerate(w.specs) if len(s.shape) == 2])


def test_random_matrices_roots_and_layout():
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        specs = [TensorSpec(f"w{i}", (8 * int(rng.integers(1, 40)), 8 * int(rng.integers(1, 40))),
                            ROWS, int(rng.integers(1, 9))) for i in range(n)]
        m = int(rng.integers(1, 10))
        mats = [int(i) for i in rng.permutation(n)[: int(rng.integers(1, n + 1))]]
        _check(specs, m, 16, mats)


def test_bad_arguments():
    specs = [TensorSpec("a", (64, 32), ROWS, 4), TensorSpec("b", (100,), ELEMENT),
             TensorSpec("c", (20, 12), TILE, 4, 4)]
    plan = rs.Plan(specs, 2, 16)
    for bad in ([], [0, 0], [3], [-1], [1], [2]):
        with pytest.raises(rs.RaggedShardError) as ei:
            rs.rs_muon_plan(plan.h, bad)
        assert ei.value.status == rs.RS_EINVAL
    mu = rs.Muon(plan, [0])
    with pytest.raises(rs.RaggedShardError) as ei:           # not uploaded
        rs.rs_muon_orthogonalize(mu.h, rs.RS_ALL, 1 << 20, stream=0)
    assert ei.value.status == rs.RS_ESTATE
    mu.free()
    plan.free()
