"""Planning-quality report of the RaggedShard planner (host only, no GPU).

Figure 11 of the veScale-FSDP page (section "Experiments and results")
reports the padding the planner leaves for DeepSeek-V3- and GPT-OSS-shaped
models at 1-, 16- and 128-row granularity (under 3%, except a spike of up to
about 18% for GPT-OSS's fused experts at 128 rows) and a planning time under
0.3 s.  This script plans the same model shapes (tensor shapes only, from
`synth.MODEL_SHAPES`, one bucket per transformer layer) with this library's
planner and prints markdown tables:

1. padding of the planned buffers and the planning time, per model,
   granularity and FSDP group size m;
2. the three tensor orders of the planning rule and the cut-unit alignment
   reading, side by side;
3. two naive layouts for comparison, by closed-form accounting (no layout
   is built): the flat concatenation of all tensors cut into m equal
   slices, and the per-tensor even split of dimension 0 over m ranks;
   their padding and the number of quantisation blocks they cut in two;
4. the padding of one GPT-OSS layer bucket as m sweeps 8..256 (the step
   spike of fused experts).

    python -m sharded_state_raggedshard_amd.planner_report [--quick]
"""
from __future__ import annotations

import argparse
import ctypes as C
import math
import os
import sys
import time
from typing import Dict, List, Sequence, Tuple

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import sharded_state_raggedshard_amd as rs  # noqa: E402
import synth  # noqa: E402

G_COLL = 16


def plan_stats(specs: Sequence, m: int, options: int = 0) -> Dict[str, float]:
    """Plan the whole model (one rs_plan_layout call) and sum over buckets."""
    arr = rs.make_specs(specs)
    h = C.c_void_p()
    t0 = time.perf_counter()
    st = rs.lib().rs_plan_layout(arr, len(specs), m, G_COLL, options, C.byref(h))
    dt = time.perf_counter() - t0
    if st != 0:
        raise rs.RaggedShardError(st, rs.lib().rs_last_error().decode())
    try:
        nb = rs.rs_plan_info(h.value)[1]
        buf = pad = 0
        worst = 0.0
        for b in range(nb):
            S, _, p, _ = rs.rs_plan_bucket(h.value, b)
            buf += m * S
            pad += p
            worst = max(worst, p / (m * S))
    finally:
        rs.rs_plan_free(h.value)
    return {"pad": pad / buf, "worst": worst, "time": dt}


def _view(spec) -> Tuple[int, int, int]:
    """(R, C, rows per index of dimension 0) of a tensor's 2-D view."""
    n = spec.numel
    C_ = int(spec.shape[-1]) if len(spec.shape) >= 2 else 1
    R = n // C_
    return R, C_, R // int(spec.shape[0])


def flat_stats(specs: Sequence, m: int) -> Tuple[int, int, int]:
    """Flat concatenation per bucket, cut into m equal slices (slice size a
    multiple of g_coll): (buffer elements, padding, blocks cut)."""
    buckets: Dict[int, List] = {}
    for s in specs:
        buckets.setdefault(int(s.bucket), []).append(s)
    buf = pad = cut = 0
    for lst in buckets.values():
        total = sum(s.numel for s in lst)
        S = -(-total // m)
        S = -(-S // G_COLL) * G_COLL
        buf += m * S
        pad += m * S - total
        # boundaries j*S, j = 1..m-1, against the tensors' block edges
        o = 0
        starts = []
        for s in lst:
            starts.append(o)
            o += s.numel
        ti = 0
        seen = set()
        for j in range(1, m):
            B = j * S
            if B >= total:
                break
            while starts[ti] + lst[ti].numel <= B:
                ti += 1
            s = lst[ti]
            R, C_, _ = _view(s)
            u = 1 if s.gran == synth.ELEMENT else s.br * C_  # cut unit
            rel = B - starts[ti]
            if rel % u != 0:
                seen.add((ti, rel // u))
        cut += len(seen)
    return buf, pad, cut


def shard0_stats(specs: Sequence, m: int) -> Tuple[int, int, int]:
    """Every tensor split evenly along dimension 0 over m ranks (each rank
    ceil(d0 / m) indices, the last ones padded): (buffer elements, padding,
    blocks cut)."""
    buf = pad = cut = 0
    for s in specs:
        d0 = int(s.shape[0])
        R, C_, rpi = _view(s)
        per = -(-d0 // m)
        buf += m * per * rpi * C_
        pad += (m * per - d0) * rpi * C_
        step = per * rpi  # rows of one rank's shard in the 2-D view
        if s.gran == synth.ELEMENT:
            continue  # single-element blocks are never cut
        k = s.br
        seen = set()
        for j in range(1, m):
            B = j * step
            if B >= R:
                break
            if B % k != 0:
                seen.add(B // k)
        cut += len(seen)
    return buf, pad, cut


def blocks_of(specs: Sequence) -> int:
    return sum(s.numel if s.gran == synth.ELEMENT else math.ceil(_view(s)[0] / s.br)
               for s in specs)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true", help="fewer group sizes")
    args = ap.parse_args()
    ms = [8, 64, 256] if args.quick else [8, 16, 32, 64, 128, 256]
    grans = [1, 16, 128]
    models = list(synth.MODEL_SHAPES)
    print("## Planned padding and planning time (given order)\n")
    print("Padding = sum over buckets of (m S_b - real elements) / sum of m S_b; "
          "worst = the largest single-bucket share; time = one rs_plan_layout call "
          "for the whole model.\n")
    print("| model | rows per block | " + " | ".join(f"m = {m}" for m in ms) + " |")
    print("|---|---|" + "---|" * len(ms))
    for name in models:
        for k in grans:
            specs = synth.MODEL_SHAPES[name](k)
            cells = []
            for m in ms:
                st = plan_stats(specs, m)
                cells.append(f"{100 * st['pad']:.2f}% (worst {100 * st['worst']:.1f}%, "
                             f"{1e3 * st['time']:.0f} ms)")
            print(f"| {name} | {k} | " + " | ".join(cells) + " |")
    print("\n## Tensor orders and the alignment reading (128-row blocks)\n")
    print("| model | m | given | by block size | by element count | given, cut-unit alignment |")
    print("|---|---|---|---|---|---|")
    for name in models:
        specs = synth.MODEL_SHAPES[name](128)
        for m in ([64, 256] if args.quick else [16, 64, 256]):
            cells = [plan_stats(specs, m, o)["pad"] for o in
                     (rs.RS_ORDER_GIVEN, rs.RS_ORDER_BY_BLOCK, rs.RS_ORDER_BY_SIZE,
                      rs.RS_ALIGN_CUT_UNIT)]
            print(f"| {name} | {m} | " + " | ".join(f"{100 * c:.2f}%" for c in cells) + " |")
    print("\n## Naive layouts against the plan\n")
    print("Blocks cut = quantisation blocks that a rank boundary splits in two (the "
          "planned layout cuts none by construction).\n")
    print("| model | rows | m | blocks | plan padding | flat padding | flat blocks cut | "
          "dim-0 split padding | dim-0 split blocks cut |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name in models:
        for k in (16, 128):
            specs = synth.MODEL_SHAPES[name](k)
            nblk = blocks_of(specs)
            for m in (64, 256):
                p = plan_stats(specs, m)["pad"]
                fb, fp, fc = flat_stats(specs, m)
                sb, sp, sc = shard0_stats(specs, m)
                print(f"| {name} | {k} | {m} | {nblk:,} | {100 * p:.2f}% | {100 * fp / fb:.3f}% | "
                      f"{fc:,} | {100 * sp / sb:.2f}% | {sc:,} |")
    print("\n## One GPT-OSS layer bucket, 128-row blocks, padding against m\n")
    layer = [s for s in synth.MODEL_SHAPES["gpt_oss_120b"](128) if s.bucket == 1]
    layer = [synth.TensorSpec(s.name, s.shape, s.gran, s.br, s.bc, 0) for s in layer]
    row = []
    for m in range(8, 257, 8):
        row.append((m, plan_stats(layer, m)["pad"]))
    print("| m | " + " | ".join(str(m) for m, _ in row[:16]) + " |")
    print("|---|" + "---|" * 16)
    print("| padding | " + " | ".join(f"{100 * p:.1f}%" for _, p in row[:16]) + " |")
    print("\n| m | " + " | ".join(str(m) for m, _ in row[16:]) + " |")
    print("|---|" + "---|" * len(row[16:]))
    print("| padding | " + " | ".join(f"{100 * p:.1f}%" for _, p in row[16:]) + " |")


if __name__ == "__main__":
    main()
