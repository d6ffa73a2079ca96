"""Host-side checks of bench.py: the one-GPU contract and the Muon flop
accounting (no GPU needed)."""
import math
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def _tiles_brute(shapes, tile):
    """MFMA work counted tile by tile: every output tile of the update, the
    tiles on and above the diagonal of the two symmetric products."""
    tot = 0
    for R, C in shapes:
        n, k = min(R, C), max(R, C)
        tn, tk = math.ceil(n / tile), math.ceil(k / tile)
        for a in range(tn):
            for b in range(tn):
                if b >= a:
                    tot += 2 * tile * tile * k   # A = X X^T
                    tot += 2 * tile * tile * n   # B = c A A + b A
        tot += tn * tk * 2 * tile * tile * n     # Y' = Y B^T + a Y
    return 5 * tot


def test_muon_flops_count_the_tiles_of_the_kernel_that_runs():
    wide = [(320, 192), (192, 448), (64, 64)]            # multiples of 64: 256 x 256 tiles
    ragged = [(136, 200), (264, 520)]                   # otherwise 128 x 128 tiles
    assert bench.muon_tile_flops(wide) == _tiles_brute(wide, 256)
    assert bench.muon_tile_flops(ragged) == _tiles_brute(ragged, 128)
    assert bench.muon_tile_flops(wide + ragged) == _tiles_brute(wide + ragged, 128)
