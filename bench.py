"""Benchmark of the one-GPU RaggedShard / DBuffer shard-state path.

One step = one pass of the whole hot path over one batch of synthetic
gradients, in stream order on one GPU:
    group_l2norm(grad, all slices) -> clip_coef -> adam8_step(all slices,
    grad scale = clip coefficient) -> pack_shard(all slices, fp32 master ->
    bf16 gathered buffer) -> unpack_full(bf16 buffer -> per-parameter views)
    -> group_zero(the gradient accumulation buffer of the next step)
All m simulated ranks' slices live in one device buffer (the gathered
buffer stands in for AllGather / ReduceScatter).  Two seeded random
gradient buffers alternate between steps, so every step reads a full
synthetic gradient; the zeroing clears a third buffer of the same size (what
the next backward pass would accumulate into).  Inputs are resident in HBM
before the timed region.  Prints one JSON line.

After the step, the FP8 copy-in (fp32 master -> E4M3 codes with one fp32
scale per quantisation block) and its copy-out (codes -> bf16 views) are
timed on their own over the same selection (`fp8_copy`; --no-fp8 skips it).

With --rank R the l2norm, the step, the pack and the zeroing act on rank R's
slices of every bucket (its ragged local shard: the per-rank work of one
GPU in an m-GPU job), and the copy-out unpacks bucket 0 (one gathered
bucket).  No CPU baseline is run in that mode.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama_layer] [--rank R]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8-AdamW shard step params/s + HBM GB/s (% peak); pack/unpack GB/s"
PEAK_GBS = 8000.0  # MI355X HBM3E


def selection_sizes(plan, specs, rank):
    """(real elements, buffer elements, quantisation blocks) of the selected
    slices: everything, or rank `rank`'s slice of every bucket."""
    import sharded_state_raggedshard_amd as rs

    if rank is None:
        return sum(s.numel for s in specs), plan.total, plan.n_blocks
    real = buf = blocks = 0
    for b in range(plan.nb):
        lo = plan.base[b] + rank * plan.S[b]
        hi = lo + plan.S[b]
        buf += plan.S[b]
        blocks += rs.rs_plan_rank_blocks(plan.h, b, rank)[1]
        for i, s in enumerate(specs):
            if int(getattr(s, "bucket", 0)) == b:
                real += max(0, min(hi, plan.pos[i] + s.numel) - max(lo, plan.pos[i]))
    return real, buf, blocks


def algorithmic_bytes(real, buf, total_blocks, unpack_real):
    """Bytes each op must move (not counting padding the op never touches)."""
    pad = buf - real
    return {
        # theta r/w 8, grad 2, q_m r/w 2, q_v r/w 2 per element; absmax m/v r/w per block
        "adam8_step": 14 * real + 16 * total_blocks,
        # read fp32 4 + write bf16 2 per element; zero padding 2
        "pack_shard": 6 * real + 2 * pad,
        # read bf16 2 + write bf16 2 per element
        "unpack_full": 4 * unpack_real,
        # read bf16 over the whole selection
        "group_l2norm": 2 * buf,
        # write bf16 over the whole selection
        "group_zero": 2 * buf,
    }


def fp8_algorithmic_bytes(real, buf, total_blocks, unpack_real, unpack_blocks):
    """Bytes of the FP8 copy-in and copy-out (E4M3 code + fp32 scale per block)."""
    return {
        # read fp32 4 + write code 1 per element; zero padding 1; write scale 4 per block
        "pack_shard_fp8": 5 * real + (buf - real) + 4 * total_blocks,
        # read code 1 + write bf16 2 per element; read scale 4 per block
        "unpack_full_fp8": 3 * unpack_real + 4 * unpack_blocks,
    }


def recorded_traffic(workload: str):
    """HBM bytes per step-kernel launch from the committed rocprofv3 counter
    summary, only while the kernel source is the one that was profiled on
    this workload (otherwise None)."""
    import hashlib
    rec = os.path.join(ROOT, "profiles", "adam8_step_traffic.json")
    try:
        with open(rec) as f:
            r = json.load(f)
        with open(os.path.join(ROOT, r["source"]), "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    if not h.startswith(r["source_sha256_prefix"]) or r.get("workload_key") != workload:
        return None
    return r["hbm_bytes_per_launch"]


def cpu_baseline(w, budget_s: float):
    """The oracle (single-threaded C) running the same hot path on a host
    copy of the same workload, repeated until budget_s is spent."""
    import numpy as np
    import torch

    import oracle
    import synth

    L = oracle.Layout(w.specs, w.m, w.g_coll)
    theta = np.zeros(L.total, dtype=np.float32)
    grads = [np.zeros(L.total, dtype=np.uint16) for _ in range(2)]
    for i, s in enumerate(w.specs):
        theta[L.pos[i]:L.pos[i] + s.numel] = synth.uniform_params(s.numel, w.seed, 2 * i).numpy()
        for j, g in enumerate(grads):
            g[L.pos[i]:L.pos[i] + s.numel] = synth.normal_bf16(
                s.numel, w.grad_sigma, w.seed + 1000 * j, 2 * i + 1).view(
                    torch.int16).numpy().view(np.uint16)
    next_grad = np.zeros(L.total, dtype=np.uint16)
    qm = np.zeros(L.total, dtype=np.int8)
    qv = np.zeros(L.total, dtype=np.uint8)
    am = np.zeros(L.n_blocks, dtype=np.float32)
    av = np.zeros(L.n_blocks, dtype=np.float32)
    buf = np.zeros(L.total, dtype=np.uint16)
    outs = [np.zeros(s.numel, dtype=np.uint16) for s in w.specs]
    fviews = [theta[L.pos[i]:L.pos[i] + s.numel] for i, s in enumerate(w.specs)]
    t0 = time.perf_counter()
    reps = 0
    while True:
        grad = grads[(reps + 1) % 2]
        ss = L.group_sumsq(-1, -1, grad)
        s = oracle.clip_coef(ss, 1.0)
        L.adam8_step(-1, -1, theta, grad, qm, qv, am, av, oracle.HParams(step=reps + 1), gscale=s)
        L.pack(-1, -1, fviews, buf)
        L.unpack(-1, outs, buf)
        L.group_zero(-1, -1, next_grad)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    real = w.real_elems
    return {"value": real * reps / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full hot-path passes (l2norm, clip, adam8 step, pack, unpack, "
                      f"zero) of the whole {w.name} workload, {el:.1f} s, single thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama_layer")
    ap.add_argument("--rank", type=int, default=None,
                    help="time one rank's ragged local shard instead of all m slices")
    ap.add_argument("--split-mode", default="cooperative", choices=["cooperative", "two_pass"])
    ap.add_argument("--chunk", type=int, default=None, help="elements per workgroup in the step")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the separate timing of the FP8 copy-in / copy-out")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="after the timed steps, copy a 1 GiB tensor once (a plain copy "
                         "kernel of known size for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "path (RCCL all-gather / reduce-scatter of the planned buffers) is not part of "
              "this build", file=sys.stderr)
        sys.exit(2)

    import torch

    import sharded_state_raggedshard_amd as rs
    import synth

    w = synth.WORKLOADS[args.workload]()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mode = rs.RS_SPLIT_COOPERATIVE if args.split_mode == "cooperative" else rs.RS_SPLIT_TWO_PASS
    t0 = time.perf_counter()
    plan = rs.Plan(w.specs, w.m, w.g_coll, chunk=args.chunk, split_mode=mode)
    plan_s = time.perf_counter() - t0
    plan.upload()
    total, nblk = plan.total, plan.n_blocks

    # resident state: fp32 master, bf16 grads, int8/uint8 moments, absmax
    theta = torch.zeros(total, dtype=torch.float32, device=dev)
    grads = [torch.zeros(total, dtype=torch.int16, device=dev) for _ in range(2)]
    for i, s in enumerate(w.specs):
        p = plan.pos[i]
        theta[p:p + s.numel] = synth.uniform_params(s.numel, w.seed, 2 * i, device=dev)
        for j, g in enumerate(grads):
            g[p:p + s.numel] = synth.normal_bf16(s.numel, w.grad_sigma, w.seed + 1000 * j,
                                                 2 * i + 1, device=dev).view(torch.int16)
    next_grad = torch.zeros(total, dtype=torch.int16, device=dev)
    qm = torch.zeros(total, dtype=torch.int8, device=dev)
    qv = torch.zeros(total, dtype=torch.uint8, device=dev)
    am = torch.zeros(nblk, dtype=torch.float32, device=dev)
    av = torch.zeros(nblk, dtype=torch.float32, device=dev)
    gathered = torch.zeros(total, dtype=torch.int16, device=dev)
    # fp32 master views are zero-copy views of the fp32 DBuffer; bf16
    # parameter views are separate per-parameter tensors (copy-out target)
    f32_views = [theta[plan.pos[i]:plan.pos[i] + s.numel] for i, s in enumerate(w.specs)]
    bf16_views = [torch.empty(s.numel, dtype=torch.int16, device=dev) for s in w.specs]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, f32_views)
    rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, bf16_views)
    sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
    scale = torch.ones(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sid = int(stream.cuda_stream)
    ALL = rs.RS_ALL
    R = ALL if args.rank is None else args.rank
    UB = ALL if args.rank is None else 0  # bucket(s) the copy-out unpacks
    if args.rank is not None and not 0 <= args.rank < w.m:
        raise SystemExit(f"--rank must be in 0..{w.m - 1}")

    ops = ["group_l2norm", "clip_coef", "adam8_step", "pack_shard", "unpack_full", "group_zero"]

    def step(t, ev=None):
        grad = grads[t % 2]
        if ev is not None:
            ev[0].record(stream)
        rs.rs_group_l2norm(plan.h, ALL, R, grad, rs.RS_BF16, sumsq, stream=sid)
        if ev is not None:
            ev[1].record(stream)
        rs.rs_clip_coef(sumsq, 1.0, scale, stream=sid)
        if ev is not None:
            ev[2].record(stream)
        rs.rs_adam8_step(plan.h, ALL, R, theta, grad, qm, qv, am, av, step=t, grad_scale=scale,
                         stream=sid)
        if ev is not None:
            ev[3].record(stream)
        rs.rs_pack_shard(plan.h, ALL, R, gathered, stream=sid)
        if ev is not None:
            ev[4].record(stream)
        rs.rs_unpack_full(plan.h, UB, gathered, stream=sid)
        if ev is not None:
            ev[5].record(stream)
        rs.rs_group_zero(plan.h, ALL, R, next_grad, rs.RS_BF16, stream=sid)
        if ev is not None:
            ev[6].record(stream)

    t = 1
    for _ in range(args.warmup):
        step(t)
        t += 1
    torch.cuda.synchronize()

    # timed region: K whole steps between two synchronisations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(t, evs[k])
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    rs.rs_plan_check_device(plan.h, stream=sid)

    per_op = {o: 0.0 for o in ops}
    step_ms = 0.0
    for e in evs:
        for j, o in enumerate(ops):
            per_op[o] += e[j].elapsed_time(e[j + 1])
        step_ms += e[0].elapsed_time(e[6])
    per_op = {o: v / args.steps for o, v in per_op.items()}
    ms_per_step = wall * 1e3 / args.steps
    real, buf, sel_blocks = selection_sizes(plan, w.specs, args.rank)
    unpack_real = real if args.rank is None else sum(
        s.numel for s in w.specs if int(getattr(s, "bucket", 0)) == 0)
    value = real / (ms_per_step * 1e-3)

    # FP8 copy-in (E4M3 codes + one fp32 scale per block) and its bf16 copy-out,
    # timed on their own after the step (not part of the step above)
    fp8 = None
    if not args.no_fp8:
        codes = torch.zeros(total, dtype=torch.uint8, device=dev)
        fscale = torch.zeros(nblk, dtype=torch.float32, device=dev)
        for _ in range(max(1, args.warmup)):
            rs.rs_pack_shard_fp8(plan.h, ALL, R, codes, fscale, stream=sid)
            rs.rs_unpack_full_fp8(plan.h, UB, codes, fscale, stream=sid)
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e in fev:
            e[0].record(stream)
            rs.rs_pack_shard_fp8(plan.h, ALL, R, codes, fscale, stream=sid)
            e[1].record(stream)
            rs.rs_unpack_full_fp8(plan.h, UB, codes, fscale, stream=sid)
            e[2].record(stream)
        torch.cuda.synchronize()
        rs.rs_plan_check_device(plan.h, stream=sid)
        unpack_blocks = nblk if args.rank is None else sum(
            rs.rs_plan_rank_blocks(plan.h, 0, r)[1] for r in range(w.m))
        fab = fp8_algorithmic_bytes(real, buf, sel_blocks, unpack_real, unpack_blocks)
        fp8 = {}
        for j, o in enumerate(["pack_shard_fp8", "unpack_full_fp8"]):
            ms = sum(e[j].elapsed_time(e[j + 1]) for e in fev) / args.steps
            gbs = fab[o] / (ms * 1e-3) / 1e9
            fp8[o] = {"ms": round(ms, 5), "alg_bytes": fab[o], "GB/s": round(gbs, 1),
                      "frac": round(gbs / PEAK_GBS, 4)}
        del codes, fscale

    if args.pmc_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    ab = algorithmic_bytes(real, buf, sel_blocks, unpack_real)
    breakdown = {}
    for o in ops:
        d = {"ms": round(per_op[o], 5)}
        if o in ab:
            gbs = ab[o] / (per_op[o] * 1e-3) / 1e9
            d.update({"alg_bytes": ab[o], "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_GBS, 4)})
        breakdown[o] = d
    step_gbs = ab["adam8_step"] / (per_op["adam8_step"] * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 update, int8/uint8 state, bf16 grads and copies",
        "data": "synthetic (seeded torch generators; shapes of the workload)",
        "config": {
            "workload": w.name,
            "tensors": len(w.specs),
            "real_params": real,
            "selection": "all ranks" if args.rank is None else f"rank {args.rank}, all buckets",
            "m_ranks": w.m,
            "g_coll": w.g_coll,
            "S": plan.S[0],
            "padding": plan.padding[0],
            "quant_blocks": sel_blocks,
            "split_mode": args.split_mode,
            "chunk_elems": rs.rs_plan_chunk_elems(plan.h),
            "planner_s": round(plan_s, 4),
        },
        "step_params_per_s": round(real / (per_op["adam8_step"] * 1e-3), 1),
        "ops": breakdown,
        "roofline": {
            "bound": "hbm",
            "kernel": "adam8_step",
            "achieved": round(step_gbs, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(step_gbs / PEAK_GBS, 4),
            "traffic": recorded_traffic(args.workload) if args.rank is None else None,
        },
        "event_ms_per_step": round(step_ms / args.steps, 5),
    }
    if fp8 is not None:
        result["fp8_copy"] = fp8
    if args.cpu_budget > 0 and args.rank is None:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    plan.free()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
