"""The planning-quality report's closed-form accounting of the naive layouts
(hand-checked cases) and a quick run of the report (host only)."""
import subprocess
import sys
import os

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


def test_report_runs_quick():
    r = subprocess.run([sys.executable, "-m", "sharded_state_raggedshard_amd.planner_report",
                        "--quick"], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "| gpt_oss_120b | 128 |" in r.stdout
