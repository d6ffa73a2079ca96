"""Benchmark of the one-GPU RaggedShard / DBuffer shard-state path.

Headline workload: the whole Llama-8B-shaped state on one rank (8.03e9
fp32 master parameters, 291 tensors, 32-row quantisation blocks, m = 1),
the largest configuration that fits one GPU.  One step = one pass of the
whole hot path over one batch of synthetic gradients, in stream order:
    group_l2norm_clip(grad: the global sum of squares and the clipping
    coefficient in one launch; with m = 1 the whole norm is on this device) ->
    adam8_step(grad scale = the clip coefficient, fused bf16 copy-in into
    the gathered buffer) ->
    unpack_full(gathered buffer -> per-parameter bf16 views) ->
    group_zero(the gradient buffer the next backward pass accumulates into)
Two seeded random gradient buffers alternate between steps, so every step
reads a full gradient.  Inputs are resident in HBM before the timed region;
a step streams about 200 GB, far beyond the 256 MB last-level cache, so
nothing is served from cache.  After the K timed steps, the L2 norm alone
(the form an m-GPU job uses, before its all-reduce), the step without the
fused output, the standalone copy-in (pack_shard) and the FP8 copy-in /
copy-out are timed on their own (K calls each, HIP events).

`per_config` then times every op of the other workloads on their own
(events around each call, 1 GiB of unrelated memory read before each timed
call so no input is served from cache): the Llama-style layer
(all 8 slices), ranks 0 and 43 of the 24-layer tiled model (each rank's 24
slices; copy-out of bucket 0), ranks 0 and 46 of the fused-expert MoE bucket.

`muon` times one distributed-Muon step (gather, Newton-Schulz on every root,
apply) over the 2-D matrices of the Llama-style layer and of one
Llama-8B-shaped layer; the Newton-Schulz products are MFMA work, reported
against the 2.5 PFLOP/s dense bf16 peak.

`cpu_baseline` runs the oracle (plain C) over a bounded sample of the same
workload on the host: the tensors of one layer plus the final norm, cut
into row-block pieces, once on one thread and once on `min(16, cpus)`
threads (the pieces dealt out by size; the oracle code is unchanged).

Prints one JSON line.  `--muon-only` prints only the Muon figures (a line
with the key "muon"), for profiling the Newton-Schulz kernels on their own.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b_full]
                    [--rank R] [--no-per-config] [--cpu-budget S] [--muon-only]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8-AdamW shard step params/s + HBM GB/s (% peak); pack/unpack GB/s"
PEAK_GBS = 8000.0  # MI355X HBM3E
HEADLINE = "llama8b_full"
PER_CONFIG = [("llama_layer", None), ("llama8b_tiles", 0), ("llama8b_tiles", 43), ("moe", 0),
              ("moe", 46)]
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
# distributed Muon: the 2-D matrices of one Llama-style layer (8 ranks) and of
# one Llama-8B-shaped layer (64 ranks)
MUON_CASES = [("llama_layer", 10), ("llama8b_tiles_1layer", 3)]
GEN_CHUNK = 1 << 28


# ------------------------------------------------------------------ sizes

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


def algorithmic_bytes(real, buf, blocks, unpack_real, unpack_blocks):
    """Bytes each op must move (not counting padding the op never touches)."""
    pad = buf - real
    return {
        # theta r/w 8, grad 2, q_m r/w 2, q_v r/w 2 per element; absmax m/v r/w per block
        "adam8_step": 14 * real + 16 * blocks,
        # the same with the fused bf16 copy-in: + bf16 write 2 per element
        "adam8_step_bf16_out": 16 * real + 16 * blocks,
        # read fp32 4 + write bf16 2 per element; zero padding 2
        "pack_shard": 6 * real + 2 * pad,
        # read bf16 2 + write bf16 2 per element
        "unpack_full": 4 * unpack_real,
        # read / write bf16 over the whole selection
        "group_l2norm": 2 * buf,
        "group_l2norm_clip": 2 * buf,
        "group_zero": 2 * buf,
        # read fp32 4 + write code 1 per element; zero padding 1; write scale 4 per block
        "pack_shard_fp8": 5 * real + pad + 4 * blocks,
        # the step with FP8 output: the step + code write 1 per element, scale 4 per block
        "adam8_step_fp8": 15 * real + 20 * blocks,
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


def op_entry(ms, nbytes):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 5), "alg_bytes": int(nbytes), "GB/s": round(gbs, 1),
            "frac": round(gbs / PEAK_GBS, 4)}


# ------------------------------------------------------------- GPU state

class Bench:
    """Resident state of one workload selection: the plan, fp32 master, two
    alternating bf16 gradient buffers, int8/uint8 moments, absmax arrays, the
    gathered bf16 buffer, the next step's gradient buffer and the bf16
    parameter views (copy-out targets)."""

    def __init__(self, w, rank, dev, chunk=None, split_mode=None):
        import torch

        import sharded_state_raggedshard_amd as rs
        import synth

        self.w, self.rank, self.dev = w, rank, dev
        mode = rs.RS_SPLIT_COOPERATIVE if split_mode is None else split_mode
        t0 = time.perf_counter()
        self.plan = plan = rs.Plan(w.specs, w.m, w.g_coll, chunk=chunk, split_mode=mode)
        self.plan_s = time.perf_counter() - t0
        plan.upload()
        total, nblk = plan.total, plan.n_blocks
        self.R = rs.RS_ALL if rank is None else rank
        # the bucket(s) the copy-out unpacks: all, or bucket 0 for one rank's shard
        self.UB = rs.RS_ALL if rank is None else 0
        self.theta = torch.empty(total, dtype=torch.float32, device=dev)
        self.grads = [torch.empty(total, dtype=torch.int16, device=dev) for _ in range(2)]
        self.qm = torch.zeros(total, dtype=torch.int8, device=dev)
        self.qv = torch.zeros(total, dtype=torch.uint8, device=dev)
        if w.warm_states:
            self.am = synth.random_absmax(nblk, 1e-3, w.seed, 77, device=dev)
            self.av = synth.random_absmax(nblk, 1e-6, w.seed, 78, device=dev)
        else:
            self.am = torch.zeros(nblk, dtype=torch.float32, device=dev)
            self.av = torch.zeros(nblk, dtype=torch.float32, device=dev)
        # inputs of the selected slices (the rest of the arrays is never read)
        if rank is None:
            ranges = [(0, total)]
        else:
            ranges = [(plan.base[b] + rank * plan.S[b], plan.base[b] + (rank + 1) * plan.S[b])
                      for b in range(plan.nb)]
        k = 0
        for lo, hi in ranges:
            for a in range(lo, hi, GEN_CHUNK):
                b = min(hi, a + GEN_CHUNK)
                self.theta[a:b] = synth.uniform_params(b - a, w.seed, 100 + k, device=dev)
                for j, g in enumerate(self.grads):
                    g[a:b] = synth.normal_bf16(b - a, w.grad_sigma, w.seed + 1000 * j, 5000 + k,
                                               device=dev).view(torch.int16)
                if w.warm_states:
                    self.qm[a:b] = synth.random_codes_m(b - a, w.seed, 9000 + k, device=dev)
                    self.qv[a:b] = synth.random_codes_v(b - a, w.seed, 9500 + k, device=dev)
                k += 1
        self.next_grad = torch.empty(total, dtype=torch.int16, device=dev)
        self.gathered = torch.zeros(total, dtype=torch.int16, device=dev)
        # fp32 master views are zero-copy views of the fp32 DBuffer; the bf16
        # views of the unpacked bucket(s) are separate tensors, the others
        # alias the gathered buffer (skipped by the copy-out)
        f32_views = [self.theta[plan.pos[i]:plan.pos[i] + s.numel]
                     for i, s in enumerate(w.specs)]
        self.bf16_views = []
        for i, s in enumerate(w.specs):
            if self.UB == rs.RS_ALL or int(s.bucket) == self.UB:
                self.bf16_views.append(torch.empty(s.numel, dtype=torch.int16, device=dev))
            else:
                self.bf16_views.append(self.gathered[plan.pos[i]:plan.pos[i] + s.numel])
        rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, f32_views)
        rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, self.bf16_views)
        self.sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        self.scale = torch.ones(1, dtype=torch.float32, device=dev)
        self.codes8 = torch.zeros(total, dtype=torch.uint8, device=dev)
        self.scale8 = torch.zeros(nblk, dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream()
        self.sid = int(self.stream.cuda_stream)
        real, buf, blocks = selection_sizes(plan, w.specs, rank)
        if rank is None:
            unpack_real, unpack_blocks = real, blocks
        else:
            unpack_real = sum(s.numel for s in w.specs if int(s.bucket) == 0)
            unpack_blocks = sum(rs.rs_plan_rank_blocks(plan.h, 0, r)[1] for r in range(w.m))
        self.real, self.buf, self.blocks = real, buf, blocks
        self.ab = algorithmic_bytes(real, buf, blocks, unpack_real, unpack_blocks)
        self.t = w.first_step
        torch.cuda.synchronize()

    # the ops, each on torch's current stream
    def op(self, name, t=None):
        import sharded_state_raggedshard_amd as rs

        p, R, sid = self.plan.h, self.R, self.sid
        t = self.t if t is None else t
        grad = self.grads[t % 2]
        if name == "group_l2norm":
            rs.rs_group_l2norm(p, rs.RS_ALL, R, grad, rs.RS_BF16, self.sumsq, stream=sid)
        elif name == "clip_coef":
            rs.rs_clip_coef(self.sumsq, 1.0, self.scale, stream=sid)
        elif name == "group_l2norm_clip":
            rs.rs_group_l2norm_clip(p, rs.RS_ALL, R, grad, rs.RS_BF16, 1.0, self.sumsq, self.scale,
                                    stream=sid)
        elif name == "adam8_step":
            rs.rs_adam8_step(p, rs.RS_ALL, R, self.theta, grad, self.qm, self.qv, self.am, self.av,
                             step=t, grad_scale=self.scale, stream=sid)
        elif name == "adam8_step_bf16_out":
            rs.rs_adam8_step(p, rs.RS_ALL, R, self.theta, grad, self.qm, self.qv, self.am, self.av,
                             step=t, grad_scale=self.scale, bf16_out=self.gathered, stream=sid)
        elif name == "adam8_step_fp8":
            rs.rs_adam8_step_fp8(p, rs.RS_ALL, R, self.theta, grad, self.qm, self.qv, self.am,
                                 self.av, self.codes8, self.scale8, step=t,
                                 grad_scale=self.scale, stream=sid)
        elif name == "pack_shard":
            rs.rs_pack_shard(p, rs.RS_ALL, R, self.gathered, stream=sid)
        elif name == "unpack_full":
            rs.rs_unpack_full(p, self.UB, self.gathered, stream=sid)
        elif name == "group_zero":
            rs.rs_group_zero(p, rs.RS_ALL, R, self.next_grad, rs.RS_BF16, stream=sid)
        elif name == "pack_shard_fp8":
            rs.rs_pack_shard_fp8(p, rs.RS_ALL, R, self.codes8, self.scale8, stream=sid)
        elif name == "unpack_full_fp8":
            rs.rs_unpack_full_fp8(p, self.UB, self.codes8, self.scale8, stream=sid)
        else:
            raise KeyError(name)

    def time_op(self, name, reps, warmup, cold=None):
        """Average event time (ms) of `reps` calls of one op; with `cold`, a
        1 GiB buffer is read (untimed) before every call."""
        import torch

        for _ in range(warmup):
            self.op(name)
            self.t += 1
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for e0, e1 in evs:
            if cold is not None:
                cold.sum()  # evicts the op's inputs from the caches (read only: no dirty lines)
            e0.record(self.stream)
            self.op(name)
            e1.record(self.stream)
            self.t += 1
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / reps

    def check(self):
        import sharded_state_raggedshard_amd as rs
        rs.rs_plan_check_device(self.plan.h, stream=self.sid)

    def free(self):
        import torch
        self.plan.free()
        for k in list(self.__dict__):
            if k not in ("w", "ab", "real", "buf", "blocks", "plan_s", "rank"):
                setattr(self, k, None)
        torch.cuda.empty_cache()


STEP_OPS = ["group_l2norm_clip", "adam8_step_bf16_out", "unpack_full", "group_zero"]
ALONE_OPS = ["group_l2norm", "adam8_step", "pack_shard", "pack_shard_fp8", "unpack_full_fp8",
             "adam8_step_fp8"]
CONFIG_OPS = ["group_l2norm", "adam8_step", "pack_shard", "unpack_full", "group_zero",
              "pack_shard_fp8", "unpack_full_fp8", "adam8_step_fp8"]


def time_steps(bn, steps, warmup):
    """K whole steps between two synchronisations; events around every op."""
    import torch

    for _ in range(warmup):
        for o in STEP_OPS:
            bn.op(o)
        bn.t += 1
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STEP_OPS) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(steps):
        e = evs[k]
        e[0].record(bn.stream)
        for j, o in enumerate(STEP_OPS):
            bn.op(o)
            e[j + 1].record(bn.stream)
        bn.t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    bn.check()
    per_op = {o: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps
              for j, o in enumerate(STEP_OPS)}
    ev_step = sum(e[0].elapsed_time(e[-1]) for e in evs) / steps
    return wall * 1e3 / steps, ev_step, per_op


def per_config(dev, reps, warmup):
    import torch

    import synth

    out = []
    cold = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    cold.zero_()
    for name, rank in PER_CONFIG:
        w = synth.WORKLOADS[name]()
        bn = Bench(w, rank, dev)
        ops = {}
        for o in CONFIG_OPS:
            ms = bn.time_op(o, reps, warmup, cold=cold)
            ops[o] = op_entry(ms, bn.ab[o])
        bn.check()
        out.append({"workload": w.name, "selection": "all ranks" if rank is None else
                    f"rank {rank}, all buckets", "real_params": bn.real, "quant_blocks": bn.blocks,
                    "m_ranks": w.m, "planner_s": round(bn.plan_s, 4),
                    "step_params_per_s": round(bn.real / (ops["adam8_step"]["ms"] * 1e-3), 1),
                    "ops": ops})
        bn.free()
        del bn
    del cold
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------- distributed Muon

def muon_tile_flops(shapes):
    """MFMA work the Newton-Schulz kernels do: output tiles of 256 x 256 when
    every dimension is a multiple of 64 (the 256 x 256 kernel runs), else
    128 x 128; the symmetric products (A = X X^T, B = c A A + b A) on and
    above the diagonal only; five steps."""
    tile = 256 if all(R % 64 == 0 and C % 64 == 0 for R, C in shapes) else 128
    tot = 0
    for R, C in shapes:
        n, k = min(R, C), max(R, C)
        tn, tk = -(-n // tile), -(-k // tile)
        sym = tn * (tn + 1) // 2
        tot += 5 * 2 * tile * tile * (sym * k + sym * n + tk * tn * n)
    return tot


def muon_bench(dev, name, reps):
    """One distributed-Muon step over the 2-D matrices of a workload: gather
    (momentum, redistribution to the roots), orthogonalize (Newton-Schulz on
    every root) and apply, each timed with events over `reps` calls."""
    import torch

    import sharded_state_raggedshard_amd as rs
    import synth

    w = synth.llama8b_tiles(layers=1) if name == "llama8b_tiles_1layer" else \
        synth.WORKLOADS[name]()
    plan = rs.Plan(w.specs, w.m, w.g_coll).upload()
    mats = [i for i, s in enumerate(w.specs) if len(s.shape) == 2]
    mu = rs.Muon(plan, mats).upload()
    shapes = [tuple(w.specs[i].shape) for i in mats]
    real = sum(w.specs[i].numel for i in mats)
    theta = torch.empty(plan.total, dtype=torch.float32, device=dev).uniform_(-0.1, 0.1)
    mom = torch.zeros(plan.total, dtype=torch.float32, device=dev)
    grad = (torch.randn(plan.total, device=dev) * 1e-3).to(torch.bfloat16).view(torch.int16)
    root = torch.zeros(mu.root_elems, dtype=torch.int16, device=dev)
    calls = {
        "gather": lambda: rs.rs_muon_gather(mu.h, rs.RS_ALL, mom, grad, root, momentum=0.95),
        "orthogonalize": lambda: rs.rs_muon_orthogonalize(mu.h, rs.RS_ALL, root),
        "apply": lambda: rs.rs_muon_apply(mu.h, rs.RS_ALL, theta, root, lr=1e-3,
                                          weight_decay=0.01),
    }
    for _ in range(2):
        for f in calls.values():
            f()
    torch.cuda.synchronize()
    ms = {}
    for k, f in calls.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()  # Newton-Schulz runs in place: later calls take the previous result
        e1.record()
        torch.cuda.synchronize()
        ms[k] = e0.elapsed_time(e1) / reps
    # five steps of A = X X^T, B = b A + c A A, X = a X + B X as dense products
    dense = sum(5 * (4 * min(R, C) ** 2 * max(R, C) + 2 * min(R, C) ** 3) for R, C in shapes)
    mfma = muon_tile_flops(shapes)
    roots_used = len(set(mu.roots))
    out = {
        "workload": w.name, "matrices": len(mats), "m_ranks": w.m, "roots_used": roots_used,
        "real_params": real,
        "gather": op_entry(ms["gather"], 12 * real),      # g 2, M r/w 8, U 2 per element
        "apply": op_entry(ms["apply"], 10 * real),        # O 2, theta r/w 8 per element
        "orthogonalize": {
            "ms": round(ms["orthogonalize"], 4),
            "mfma_flops": mfma, "dense_flops": dense,
            "TFLOP/s": round(mfma / (ms["orthogonalize"] * 1e-3) / 1e12, 1),
            "frac": round(mfma / (ms["orthogonalize"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "dense_equivalent_TFLOP/s": round(dense / (ms["orthogonalize"] * 1e-3) / 1e12, 1)},
        "step_ms": round(ms["gather"] + ms["orthogonalize"] + ms["apply"], 4),
    }
    mu.free()
    plan.free()
    del theta, mom, grad, root
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ CPU baseline

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _sample_pieces(w, piece_elems=1 << 23):
    """The bounded sample of a workload as row-block pieces: the tensors of
    one layer plus the final norm (or every tensor of a small workload), each
    ROWS tensor cut into pieces of whole blocks.  A piece is its own tensor
    spec with the same blocks, so the oracle does the same work on it."""
    from synth import ROWS, TensorSpec

    specs = [s for s in w.specs if s.name.startswith("l0.") or s.name == "final_norm"]
    if not specs:
        specs = list(w.specs)
    pieces = []
    for s in specs:
        if s.gran != ROWS or len(s.shape) < 2:
            pieces.append(TensorSpec(s.name, s.shape, s.gran, s.br, s.bc, 0))
            continue
        C = int(s.shape[-1])
        R = s.numel // C
        rows = max(s.br, (piece_elems // C) // s.br * s.br)
        for r0 in range(0, R, rows):
            pieces.append(TensorSpec(f"{s.name}[{r0}]", (min(rows, R - r0), C), ROWS, s.br, 0, 0))
    return pieces


class _OracleShard:
    """One thread's pieces in an m = 1 oracle layout, with host inputs."""

    def __init__(self, pieces, w, seed):
        import numpy as np
        import torch

        import oracle
        import synth

        self.L = L = oracle.Layout(pieces, 1, w.g_coll)
        self.theta = np.zeros(L.total, dtype=np.float32)
        self.grads = [np.zeros(L.total, dtype=np.uint16) for _ in range(2)]
        for i, s in enumerate(pieces):
            p = L.pos[i]
            self.theta[p:p + s.numel] = synth.uniform_params(s.numel, seed, 2 * i).numpy()
            for j, g in enumerate(self.grads):
                g[p:p + s.numel] = synth.normal_bf16(s.numel, w.grad_sigma, seed + 1000 * j,
                                                     2 * i + 1).view(torch.int16).numpy().view(
                                                         np.uint16)
        self.next_grad = np.zeros(L.total, dtype=np.uint16)
        self.qm = np.zeros(L.total, dtype=np.int8)
        self.qv = np.zeros(L.total, dtype=np.uint8)
        self.am = np.zeros(L.n_blocks, dtype=np.float32)
        self.av = np.zeros(L.n_blocks, dtype=np.float32)
        self.buf = np.zeros(L.total, dtype=np.uint16)
        self.outs = [np.zeros(s.numel, dtype=np.uint16) for s in pieces]
        self.fviews = [self.theta[L.pos[i]:L.pos[i] + s.numel] for i, s in enumerate(pieces)]
        self.real = sum(s.numel for s in pieces)

    def sumsq(self, t):
        return self.L.group_sumsq(-1, -1, self.grads[t % 2])

    def rest(self, t, s):
        import oracle
        L = self.L
        L.adam8_step(-1, -1, self.theta, self.grads[t % 2], self.qm, self.qv, self.am, self.av,
                     oracle.HParams(step=t), gscale=s, out=self.buf)
        L.pack(-1, -1, self.fviews, self.buf)
        L.unpack(-1, self.outs, self.buf)
        L.group_zero(-1, -1, self.next_grad)


def _cpu_leg(pieces, w, threads, budget_s):
    import oracle

    order = sorted(range(len(pieces)), key=lambda i: -pieces[i].numel)
    bins = [[] for _ in range(threads)]
    load = [0] * threads
    for i in order:  # largest first onto the least-loaded thread
        k = load.index(min(load))
        bins[k].append(pieces[i])
        load[k] += pieces[i].numel
    bins = [b for b in bins if b]
    shards = [_OracleShard(b, w, 17 + k) for k, b in enumerate(bins)]
    real = sum(s.real for s in shards)

    def one_pass(ex, t):
        ss = sum(ex.map(lambda sh: sh.sumsq(t), shards))  # the all-reduce of the norm
        s = oracle.clip_coef(ss, 1.0)
        list(ex.map(lambda sh: sh.rest(t, s), shards))

    with cf.ThreadPoolExecutor(max_workers=len(shards)) as ex:
        one_pass(ex, 1)  # untimed: first touch of every page
        t0 = time.perf_counter()
        reps = 0
        while True:
            one_pass(ex, reps + 2)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return real * reps / el, reps, el, real, len(shards)


def cpu_baseline(w, budget_s: float):
    """The oracle timed on the host over a bounded sample of the workload:
    min(16, cpus) threads over one layer's tensors, and one thread over its
    attention projections."""
    pieces = _sample_pieces(w)
    nthreads = max(1, min(16, os.cpu_count() or 1))
    vn, repsn, eln, real, used = _cpu_leg(pieces, w, nthreads, budget_s / 2)
    names = sorted({p.name.split("[")[0] for p in pieces})
    what = (f"{len(names)} tensors ({real} real params: "
            f"{'one layer and the final norm' if len(names) < len(w.specs) else 'all tensors'} "
            f"of {w.name}) cut into {len(pieces)} row-block pieces; whole hot-path passes "
            "(l2norm, clip, adam8 step with bf16 output, pack, unpack, zero) after one "
            "untimed pass")
    small = [p for p in pieces if p.name.split(".")[-1].split("[")[0] in ("q", "k", "v", "o")]
    small = small or pieces[: max(1, len(pieces) // 4)]
    v1, reps1, el1, real1, _ = _cpu_leg(small, w, 1, budget_s / 2)
    return {"value": round(vn, 1), "unit": "params/s", "cores": used, "kind": "oracle",
            "sample": f"{what}: {repsn} passes in {eln:.1f} s on {used} threads",
            "cpu_model": _cpu_model(), "cpus": os.cpu_count(),
            "single_thread": {"value": round(v1, 1), "unit": "params/s", "cores": 1,
                              "sample": f"the same passes over {real1} real params (the "
                                        f"attention projections of that layer): {reps1} passes "
                                        f"in {el1:.1f} s on one thread"}}


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--rank", type=int, default=None,
                    help="time one rank's ragged local shard instead of all m slices")
    ap.add_argument("--split-mode", default="cooperative", choices=["cooperative", "two_pass"])
    ap.add_argument("--chunk", type=int, default=None, help="elements per workgroup in the step")
    ap.add_argument("--cpu-budget", type=float, default=16.0,
                    help="seconds of oracle work for the CPU baseline, both legs (0 = skip)")
    ap.add_argument("--muon-only", action="store_true",
                    help="time only the distributed-Muon cases and print their figures")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-op timing of the other workloads")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="after the timed steps, copy a 1 GiB tensor once (a plain copy "
                         "kernel of known size for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has "
              "no multi-GPU path (the RCCL all-gather / reduce-scatter of the planned buffers is "
              "not part of it); every figure is one GPU's", file=sys.stderr)
        sys.exit(2)

    import torch

    import sharded_state_raggedshard_amd as rs
    import synth

    w = synth.WORKLOADS[args.workload]()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.muon_only:
        print(json.dumps({"muon": [muon_bench(dev, n, r) for n, r in MUON_CASES]}), flush=True)
        return
    if args.rank is not None and not 0 <= args.rank < w.m:
        raise SystemExit(f"--rank must be in 0..{w.m - 1}")
    mode = rs.RS_SPLIT_COOPERATIVE if args.split_mode == "cooperative" else rs.RS_SPLIT_TWO_PASS
    bn = Bench(w, args.rank, dev, chunk=args.chunk, split_mode=mode)
    ms_per_step, ev_step, per_op = time_steps(bn, args.steps, args.warmup)
    ops = {}
    for o in STEP_OPS:
        ops[o] = op_entry(per_op[o], bn.ab[o]) if o in bn.ab else {"ms": round(per_op[o], 5)}
    for o in ALONE_OPS:  # timed on their own after the steps
        ops[o] = op_entry(bn.time_op(o, args.steps, 2), bn.ab[o])
    bn.check()
    if args.pmc_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    real = bn.real
    cfg = {
        "workload": w.name,
        "tensors": len(w.specs),
        "real_params": real,
        "selection": "all ranks" if args.rank is None else f"rank {args.rank}, all buckets",
        "m_ranks": w.m,
        "g_coll": w.g_coll,
        "S": bn.plan.S[0],
        "padding": bn.plan.padding[0],
        "quant_blocks": bn.blocks,
        "split_mode": args.split_mode,
        "chunk_elems": rs.rs_plan_chunk_elems(bn.plan.h),
        "planner_s": round(bn.plan_s, 4),
        "step": " -> ".join(STEP_OPS),
    }
    bn.free()
    del bn
    torch.cuda.empty_cache()
    dom = ops["adam8_step_bf16_out"]
    result = {
        "metric": METRIC,
        "value": round(real / (ms_per_step * 1e-3), 1),
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
        "config": cfg,
        "step_params_per_s": round(real / (dom["ms"] * 1e-3), 1),
        "ops": ops,
        "roofline": {
            "bound": "hbm",
            "kernel": "adam8_step (fused bf16 output)",
            "achieved": dom["GB/s"],
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": dom["frac"],
            "traffic": recorded_traffic(args.workload) if args.rank is None else None,
        },
        "event_ms_per_step": round(ev_step, 5),
    }
    if not args.no_per_config:
        result["per_config"] = per_config(dev, max(5, args.steps // 2), 2)
        result["muon"] = [muon_bench(dev, n, r) for n, r in MUON_CASES]
    if args.cpu_budget > 0 and args.rank is None:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
