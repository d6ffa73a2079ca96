"""The planning-quality report's closed-form accounting of the naive layouts
(hand-checked cases, and built layouts whose cut blocks the oracle counts
one block at a time) and a quick run of the report (host only)."""
import subprocess
import sys
import os

import numpy as np
import pytest

import oracle
import synth
from synth import ELEMENT, ROWS, TensorSpec
from sharded_state_raggedshard_amd import planner_report as pr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flat_layout_accounting_hand_cases():
    # one [10, 4] tensor in 2-row blocks (cut unit 8 elements), m = 2,
    # g_coll 16: S = roundup(20, 16) = 32, 24 elements of padding; the one
    # boundary, at 32, is a band edge (32 % 8 == 0) -> no block cut
    specs = [TensorSpec("a", (10, 4), ROWS, 2)]
    buf, pad, cut = pr.flat_stats(specs, 2)
    assert (buf, pad, cut) == (64, 24, 0)
    # [12, 4] in 3-row blocks (cut unit 12), m = 3: S = roundup(16, 16) = 16,
    # boundaries 16 and 32: 16 % 12 = 4 and 32 % 12 = 8 -> blocks 1 and 2 cut
    specs = [TensorSpec("a", (12, 4), ROWS, 3)]
    assert pr.flat_stats(specs, 3) == (48, 0, 2)


def test_dim0_split_accounting_hand_cases():
    # [10, 4] over m = 4: ceil(10 / 4) = 3 rows per rank -> 12 rows, 2 rows
    # (8 elements) of padding; 2-row blocks cut at rows 3 and 9 (row 6 is a
    # block edge) -> 2 blocks cut
    specs = [TensorSpec("a", (10, 4), ROWS, 2)]
    assert pr.shard0_stats(specs, 4) == (48, 8, 2)
    # fused [E, R, C] = [4, 3, 2] over m = 2: 2 experts (6 rows) per rank,
    # 3-row blocks cut nowhere (6 % 3 == 0); 4-row blocks cut at row 6
    assert pr.shard0_stats([TensorSpec("e", (4, 3, 2), ROWS, 3)], 2) == (24, 0, 0)
    assert pr.shard0_stats([TensorSpec("e", (4, 3, 2), ROWS, 4)], 2) == (24, 0, 1)
    # element tensors are never cut
    assert pr.shard0_stats([TensorSpec("v", (7,), ELEMENT, 1)], 3)[2] == 0


def _built_flat(specs, m):
    """The flat layout built explicitly: per bucket, tensors back to back from
    0, slices of S = roundup(ceil(total / m), g_coll); cut blocks counted by
    the oracle's block geometry (the count invariant I1 requires to be 0)."""
    buckets = {}
    for s in specs:
        buckets.setdefault(int(s.bucket), []).append(s)
    buf = pad = cut = 0
    for lst in buckets.values():
        offs, o = [], 0
        for s in lst:
            offs.append(o)
            o += s.numel
        S = -(-(-(-o // m)) // pr.G_COLL) * pr.G_COLL
        buf += m * S
        pad += m * S - o
        cut += oracle.count_cut_blocks(lst, S, offs)
    return buf, pad, cut


def _built_dim0(specs, m):
    """The dimension-0 split built explicitly: each tensor alone, rank slices
    of ceil(d0 / m) indices of dimension 0 (S = that many elements)."""
    buf = pad = cut = 0
    for s in specs:
        d0 = int(s.shape[0])
        S = -(-d0 // m) * (s.numel // d0)
        buf += m * S
        pad += m * S - s.numel
        cut += oracle.count_cut_blocks([s], S, [0])
    return buf, pad, cut


def _random_inventory(rng):
    specs = []
    for b in range(int(rng.integers(1, 4))):
        for i in range(int(rng.integers(1, 6))):
            br = int(rng.integers(1, 9))
            if rng.integers(0, 4) == 0:
                specs.append(TensorSpec(f"v{b}{i}", (int(rng.integers(1, 90)),), ELEMENT, bucket=b))
            elif rng.integers(0, 2):
                specs.append(TensorSpec(f"w{b}{i}", (int(rng.integers(1, 60)),
                                                     int(rng.integers(1, 12))), ROWS, br, bucket=b))
            else:  # fused experts [E, R, C]
                specs.append(TensorSpec(f"e{b}{i}", (int(rng.integers(1, 9)), int(rng.integers(1, 12)),
                                                     int(rng.integers(1, 8))), ROWS, br, bucket=b))
    return specs


def test_naive_accounting_matches_built_layouts_random():
    rng = np.random.default_rng(2024)
    for _ in range(300):
        specs = _random_inventory(rng)
        m = int(rng.integers(1, 12))
        assert pr.flat_stats(specs, m) == _built_flat(specs, m)
        assert pr.shard0_stats(specs, m) == _built_dim0(specs, m)


@pytest.mark.parametrize("model,rows,m", [("gpt_oss_120b", 16, 64), ("gpt_oss_120b", 128, 8),
                                          ("gpt_oss_120b", 128, 256), ("deepseek_v3", 128, 8),
                                          ("deepseek_v3", 128, 256)])
def test_naive_accounting_matches_built_layouts_on_models(model, rows, m):
    specs = synth.MODEL_SHAPES[model](rows)
    assert pr.flat_stats(specs, m) == _built_flat(specs, m)
    assert pr.shard0_stats(specs, m) == _built_dim0(specs, m)


def test_report_runs_quick():
    r = subprocess.run([sys.executable, "-m", "sharded_state_raggedshard_amd.planner_report",
                        "--quick"], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "| gpt_oss_120b | 128 |" in r.stdout
