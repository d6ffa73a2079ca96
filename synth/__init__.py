"""Seeded synthetic workloads: tensor inventories and input generators.

This module is shared by the tests, the benchmark and the smoke check.  It
holds NO arithmetic of the method (no planning, no rounding rule of the
path, no optimizer math): only tensor shapes, granularities, the simulated
rank count and seeded random inputs.  Random values come from torch's
seeded generators (mt19937 on the CPU, Philox on the GPU); bf16 gradients
are made with torch's own float32 -> bfloat16 conversion.

The five workloads mirror the shapes of the structure-aware FSDP
evaluation on the veScale-FSDP page (Llama-style dense layers with 32-row
and 128x128 quantisation blocks, a GPT-OSS-like fused-expert MoE bucket
with 128-row blocks); no dataset or trained weight is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import numpy as np
import torch

ELEMENT, ROWS, TILE = 0, 1, 2


@dataclass(frozen=True)
class TensorSpec:
    """One RaggedShard tensor: row-major shape and quantisation granularity.

    gran: ELEMENT (each element is a block), ROWS (br = k rows per block) or
    TILE (br x bc tiles).  bucket: index of the communication bucket.
    """

    name: str
    shape: Tuple[int, ...]
    gran: int
    br: int = 0
    bc: int = 0
    bucket: int = 0

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= int(s)
        return n


@dataclass
class Workload:
    name: str
    specs: List[TensorSpec]
    m: int
    g_coll: int
    grad_sigma: float
    steps: int
    seed: int = 0
    warm_states: bool = False
    first_step: int = 1
    note: str = ""

    @property
    def n_buckets(self) -> int:
        return 1 + max(s.bucket for s in self.specs)

    @property
    def real_elems(self) -> int:
        return sum(s.numel for s in self.specs)


def _llama_layer(h: int, ffn: int, kv: int, gran: int, br: int, bc: int, bucket: int,
                 prefix: str = "") -> List[TensorSpec]:
    return [
        TensorSpec(prefix + "q", (h, h), gran, br, bc, bucket),
        TensorSpec(prefix + "k", (kv, h), gran, br, bc, bucket),
        TensorSpec(prefix + "v", (kv, h), gran, br, bc, bucket),
        TensorSpec(prefix + "o", (h, h), gran, br, bc, bucket),
        TensorSpec(prefix + "gate", (ffn, h), gran, br, bc, bucket),
        TensorSpec(prefix + "up", (ffn, h), gran, br, bc, bucket),
        TensorSpec(prefix + "down", (h, ffn), gran, br, bc, bucket),
        TensorSpec(prefix + "norm1", (h,), gran, br, bc, bucket),
        TensorSpec(prefix + "norm2", (h,), gran, br, bc, bucket),
    ]


def tiny() -> Workload:
    """Three fp32 matrices with 32x32 tiles plus an element-granular bias;
    4 simulated ranks, g_coll = 16 elements, 3 steps from zero states."""
    specs = [
        TensorSpec("W1", (64, 96), TILE, 32, 32),
        TensorSpec("W2", (96, 64), TILE, 32, 32),
        TensorSpec("W3", (128, 32), TILE, 32, 32),
        TensorSpec("bias", (96,), ELEMENT),
    ]
    return Workload("tiny_tile32_m4", specs, m=4, g_coll=16, grad_sigma=1e-2, steps=3)


def llama_layer_2048() -> Workload:
    """One Llama-style layer (hidden 2048, ffn 5632, MHA) with 32-row
    blocks, all 8 simulated ranks on one GPU."""
    specs = [
        TensorSpec("q", (2048, 2048), ROWS, 32),
        TensorSpec("k", (2048, 2048), ROWS, 32),
        TensorSpec("v", (2048, 2048), ROWS, 32),
        TensorSpec("o", (2048, 2048), ROWS, 32),
        TensorSpec("gate", (5632, 2048), ROWS, 32),
        TensorSpec("up", (5632, 2048), ROWS, 32),
        TensorSpec("down", (2048, 5632), ROWS, 32),
        TensorSpec("norm1", (2048,), ROWS, 32),
        TensorSpec("norm2", (2048,), ROWS, 32),
    ]
    return Workload("llama_layer_h2048_rows32_m8", specs, m=8, g_coll=16, grad_sigma=1e-3,
                    steps=2)


def llama8b_tiles(layers: int = 24) -> Workload:
    """Llama-8B-shaped layers (hidden 4096, ffn 14336, GQA kv 1024) with
    128x128 tiles, one bucket per layer, 64 simulated ranks."""
    specs: List[TensorSpec] = []
    for b in range(layers):
        specs += _llama_layer(4096, 14336, 1024, TILE, 128, 128, b, prefix=f"l{b}.")
    return Workload(f"llama8b_{layers}layers_tile128_m64", specs, m=64, g_coll=16,
                    grad_sigma=1e-3, steps=2)


def moe_bucket() -> Workload:
    """GPT-OSS-like MoE bucket: 32 fused experts gate_up [32,5760,2880] and
    down [32,2880,2880] plus the router [32,2880]; 128-row blocks over the
    flattened leading dims; 48 simulated ranks; nonzero warm states."""
    specs = [
        TensorSpec("gate_up", (32, 5760, 2880), ROWS, 128),
        TensorSpec("down", (32, 2880, 2880), ROWS, 128),
        TensorSpec("router", (32, 2880), ROWS, 128),
    ]
    return Workload("moe32_rows128_m48", specs, m=48, g_coll=16, grad_sigma=1e-3, steps=1,
                    warm_states=True, first_step=11)


def llama8b_full() -> Workload:
    """Whole Llama-8B-shaped state (32 layers, vocab 128256) on one rank
    with 32-row blocks."""
    specs = [TensorSpec("embed", (128256, 4096), ROWS, 32)]
    for i in range(32):
        specs += _llama_layer(4096, 14336, 1024, ROWS, 32, 0, 0, prefix=f"l{i}.")
    specs += [TensorSpec("final_norm", (4096,), ROWS, 32),
              TensorSpec("lm_head", (128256, 4096), ROWS, 32)]
    return Workload("llama8b_full_rows32_m1", specs, m=1, g_coll=16, grad_sigma=1e-3, steps=2)


# ------------------------------------------------ model shape inventories
# Tensor shapes only (architecture hyper-parameters, no weights), for the
# planning-quality report: every matrix and vector of one layer in one
# bucket (FSDP wraps one transformer block per bucket), the embedding in a
# bucket of its own, the final norm and the output head in the last one.  Matrices and 1-D tensors take
# ROWS(k) (1-D tensors as [n, 1]); fused expert tensors [E, R, C] are viewed
# as [E * R, C].

def gpt_oss_120b_shapes(rows: int) -> List[TensorSpec]:
    """GPT-OSS-120B-shaped: 36 layers, hidden 2880, 64 query heads and 8 KV
    heads of 64, 128 experts with fused gate/up [128, 2880, 5760] and down
    [128, 2880, 2880] (plus biases), vocabulary 201088."""
    h, E, ff, hd, nq, nkv, vocab, layers = 2880, 128, 2880, 64, 64, 8, 201088, 36
    out = [TensorSpec("embed", (vocab, h), ROWS, rows, 0, 0)]
    for l in range(layers):
        b = l + 1
        p = f"l{l}."
        out += [
            TensorSpec(p + "norm1", (h,), ROWS, rows, 0, b),
            TensorSpec(p + "q", (nq * hd, h), ROWS, rows, 0, b),
            TensorSpec(p + "q_bias", (nq * hd,), ROWS, rows, 0, b),
            TensorSpec(p + "k", (nkv * hd, h), ROWS, rows, 0, b),
            TensorSpec(p + "k_bias", (nkv * hd,), ROWS, rows, 0, b),
            TensorSpec(p + "v", (nkv * hd, h), ROWS, rows, 0, b),
            TensorSpec(p + "v_bias", (nkv * hd,), ROWS, rows, 0, b),
            TensorSpec(p + "o", (h, nq * hd), ROWS, rows, 0, b),
            TensorSpec(p + "o_bias", (h,), ROWS, rows, 0, b),
            TensorSpec(p + "sinks", (nq,), ROWS, rows, 0, b),
            TensorSpec(p + "norm2", (h,), ROWS, rows, 0, b),
            TensorSpec(p + "router", (E, h), ROWS, rows, 0, b),
            TensorSpec(p + "router_bias", (E,), ROWS, rows, 0, b),
            TensorSpec(p + "gate_up", (E, h, 2 * ff), ROWS, rows, 0, b),
            TensorSpec(p + "gate_up_bias", (E, 2 * ff), ROWS, rows, 0, b),
            TensorSpec(p + "down", (E, ff, h), ROWS, rows, 0, b),
            TensorSpec(p + "down_bias", (E, h), ROWS, rows, 0, b),
        ]
    out += [TensorSpec("final_norm", (h,), ROWS, rows, 0, layers + 1),
            TensorSpec("lm_head", (vocab, h), ROWS, rows, 0, layers + 1)]
    return out


def deepseek_v3_shapes(rows: int) -> List[TensorSpec]:
    """DeepSeek-V3-shaped: 61 layers, hidden 7168, multi-head latent
    attention (128 heads, q rank 1536, kv rank 512, rope 64, nope 128, value
    128), the first 3 layers dense (ffn 18432), the others 256 routed experts
    and 1 shared expert of ffn 2048 stored as separate matrices, vocabulary
    129280."""
    h, layers, dense, E, eff, dff, vocab = 7168, 61, 3, 256, 2048, 18432, 129280
    nh, qr, kvr, rope, nope, vd = 128, 1536, 512, 64, 128, 128
    out = [TensorSpec("embed", (vocab, h), ROWS, rows, 0, 0)]
    for l in range(layers):
        b = l + 1
        p = f"l{l}."
        out += [
            TensorSpec(p + "norm1", (h,), ROWS, rows, 0, b),
            TensorSpec(p + "q_a", (qr, h), ROWS, rows, 0, b),
            TensorSpec(p + "q_a_norm", (qr,), ROWS, rows, 0, b),
            TensorSpec(p + "q_b", (nh * (nope + rope), qr), ROWS, rows, 0, b),
            TensorSpec(p + "kv_a", (kvr + rope, h), ROWS, rows, 0, b),
            TensorSpec(p + "kv_a_norm", (kvr,), ROWS, rows, 0, b),
            TensorSpec(p + "kv_b", (nh * (nope + vd), kvr), ROWS, rows, 0, b),
            TensorSpec(p + "o", (h, nh * vd), ROWS, rows, 0, b),
            TensorSpec(p + "norm2", (h,), ROWS, rows, 0, b),
        ]
        if l < dense:
            out += [TensorSpec(p + "gate", (dff, h), ROWS, rows, 0, b),
                    TensorSpec(p + "up", (dff, h), ROWS, rows, 0, b),
                    TensorSpec(p + "down", (h, dff), ROWS, rows, 0, b)]
        else:
            out += [TensorSpec(p + "router", (E, h), ROWS, rows, 0, b),
                    TensorSpec(p + "router_bias", (E,), ROWS, rows, 0, b)]
            for e in list(range(E)) + ["shared"]:
                out += [TensorSpec(p + f"e{e}.gate", (eff, h), ROWS, rows, 0, b),
                        TensorSpec(p + f"e{e}.up", (eff, h), ROWS, rows, 0, b),
                        TensorSpec(p + f"e{e}.down", (h, eff), ROWS, rows, 0, b)]
    out += [TensorSpec("final_norm", (h,), ROWS, rows, 0, layers + 1),
            TensorSpec("lm_head", (vocab, h), ROWS, rows, 0, layers + 1)]
    return out


MODEL_SHAPES = {
    "gpt_oss_120b": gpt_oss_120b_shapes,
    "deepseek_v3": deepseek_v3_shapes,
}


WORKLOADS = {
    "tiny": tiny,
    "llama_layer": llama_layer_2048,
    "llama8b_tiles": llama8b_tiles,
    "moe": moe_bucket,
    "llama8b_full": llama8b_full,
}


# --------------------------------------------------------------- generators

def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream) * 7919 + 12345) & ((1 << 63) - 1))
    return g


def uniform_params(n: int, seed: int, stream: int, device="cpu", lo=-0.1, hi=0.1):
    """fp32 values ~ U(lo, hi)."""
    g = _gen(seed, stream, device)
    x = torch.empty(n, dtype=torch.float32, device=device)
    x.uniform_(lo, hi, generator=g)
    return x


def normal_bf16(n: int, sigma: float, seed: int, stream: int, device="cpu"):
    """bf16 values ~ N(0, sigma^2) (sigma is the standard deviation),
    returned as a torch.bfloat16 tensor."""
    g = _gen(seed, stream, device)
    x = torch.empty(n, dtype=torch.float32, device=device)
    x.normal_(0.0, sigma, generator=g)
    return x.to(torch.bfloat16)


def random_codes_m(n: int, seed: int, stream: int, device="cpu"):
    """int8 codes uniform in [-127, 127] (warm first moments)."""
    g = _gen(seed, stream, device)
    return torch.randint(-127, 128, (n,), generator=g, dtype=torch.int16,
                         device=device).to(torch.int8)


def random_codes_v(n: int, seed: int, stream: int, device="cpu"):
    """uint8 codes uniform in [0, 255] (warm second moments)."""
    g = _gen(seed, stream, device)
    return torch.randint(0, 256, (n,), generator=g, dtype=torch.int16,
                         device=device).to(torch.uint8)


def random_absmax(n: int, scale: float, seed: int, stream: int, device="cpu"):
    """Positive fp32 per-block absmax values in [scale/2, 3*scale/2)."""
    g = _gen(seed, stream, device)
    x = torch.empty(n, dtype=torch.float32, device=device)
    x.uniform_(0.5 * scale, 1.5 * scale, generator=g)
    return x


def random_tiny_specs(rng: np.random.Generator, n_max: int = 4, elems_max: int = 64
                      ) -> List[TensorSpec]:
    """Random small tensors with random granularities (for exhaustive
    planner checks)."""
    n = int(rng.integers(1, n_max + 1))
    out = []
    budget = elems_max
    for i in range(n):
        kind = int(rng.integers(0, 3))
        if kind == ELEMENT or budget < 4:
            d0 = int(rng.integers(1, max(2, min(budget, 16) + 1)))
            out.append(TensorSpec(f"t{i}", (d0,), ELEMENT))
            budget -= d0
        elif kind == ROWS:
            C = int(rng.integers(1, 5))
            R = int(rng.integers(1, max(2, budget // C // 2 + 1)))
            k = int(rng.integers(1, 4))
            out.append(TensorSpec(f"t{i}", (R, C), ROWS, k))
            budget -= R * C
        else:
            C = int(rng.integers(1, 5))
            R = int(rng.integers(2, max(3, budget // C // 2 + 1)))
            br = int(rng.integers(2, 4))
            bc = int(rng.integers(1, 3))
            out.append(TensorSpec(f"t{i}", (R, C), TILE, br, bc))
            budget -= R * C
        if budget <= 0:
            break
    return out
