"""Plain CPU oracle of the distributed Muon path -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline use this
module; the library never imports it.  Slow and literal on purpose: numpy
in binary64 (one library matrix product per step), no blocking or fusion.

What it computes follows the veScale-FSDP page (awesome-system-papers),
section "Structure-aware training case study", distributed Muon
(Algorithm 2): SelectRoot() balances the matrices over the ranks, each
matrix's update is redistributed to RaggedShard(r) -- the whole 2-D matrix
on its root r, every other rank holding none of it (an uneven RaggedShard:
per-rank sizes differ) -- Newton-Schulz runs on the root, and the result is
redistributed back and applied; on the other ranks the matrix update is a
no-op.  The page's "RaggedShard" section gives the uneven per-device
distribution this needs.  The Muon update itself is the one the "Muon
Optimizer at Scale" entry of the AI-history comparison page
(ai-history-trend-future, /history/compare) summarises (matrix
orthogonalisation of 2-D updates, weight decay and a calibration to the
parameter scale); the pages give no formulas, so the published form is
read here as:

  M <- mu * M + G                         (binary32, the momentum)
  U  = bf16(M)                            (what the redistribution carries)
  O  = NS5(U)                             (quintic Newton-Schulz, below)
  theta <- theta * (1 - lr * wd) - (lr * 0.2 * sqrt(max(R, C))) * O

NS5 (the published quintic iteration with coefficients (a, b, c) =
(3.4445, -4.7750, 2.0315), five steps): X = U / (||U||_F + 1e-7), taken as
its transpose when R > C so that X is n x k with n <= k; then five times
  A = X X^T,  B = b A + c A A,  X = a X + B X;
and the transpose back.  With `bf16=True` the values the GPU path stores
between products (X after the normalisation, A, B and every new X) are
rounded to bf16 (round to nearest even from the exact binary64 value), the
rest stays binary64: the precision the published iteration runs in.  With
`bf16=False` every step is binary64.

SelectRoot is read as the longest-processing-time rule: matrices in order
of decreasing Newton-Schulz cost (ties: the earlier matrix first), each to
the rank with the least cost so far (ties: the lowest rank).  The cost of an
R x C matrix is the flop count of NS5 on it, 5 (4 n^2 k + 2 n^3) with
n = min(R, C), k = max(R, C).
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
NS_EPS = 1e-7


def ns_flops(R: int, C: int) -> int:
    """Floating-point operations of NS5 on an R x C matrix (each product
    of an n x l by an l x p matrix counted as 2 n l p)."""
    n, k = min(R, C), max(R, C)
    return NS_STEPS * (4 * n * n * k + 2 * n ** 3)


def select_roots(shapes: Sequence[Tuple[int, int]], m: int) -> List[int]:
    """Root rank of every matrix (longest processing time first)."""
    cost = [ns_flops(R, C) for R, C in shapes]
    order = sorted(range(len(shapes)), key=lambda i: (-cost[i], i))
    load = [0] * m
    root = [0] * len(shapes)
    for i in order:
        r = min(range(m), key=lambda j: (load[j], j))
        root[i] = r
        load[r] += cost[i]
    return root


def root_layout(sizes: Sequence[int], roots: Sequence[int], m: int, align: int):
    """The uneven RaggedShard(r) placement on one device: rank r's region
    holds every matrix rooted at r, whole and back to back in the given
    order, each start a multiple of `align` elements; regions follow each
    other in rank order.  Returns (offset of every matrix, region starts
    [m + 1])."""
    off = [0] * len(sizes)
    starts = [0] * (m + 1)
    p = 0
    for r in range(m):
        starts[r] = p
        for i, (n, rt) in enumerate(zip(sizes, roots)):
            if rt == r:
                p = -(-p // align) * align
                off[i] = p
                p += int(n)
        p = -(-p // align) * align
    starts[m] = p
    return off, starts


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Binary64 values rounded to the nearest bf16 value (8 significant
    bits), ties to even; zero and the sign are kept.  Values stay far from
    the bf16 range limits here."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, |m| in [0.5, 1)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def newton_schulz5(U: np.ndarray, bf16: bool = True) -> np.ndarray:
    """NS5 of one R x C matrix (binary64 out, bf16 values when bf16)."""
    a, b, c = NS_COEFFS
    r = bf16_round if bf16 else (lambda v: v)
    X = np.asarray(U, dtype=np.float64)
    tr = X.shape[0] > X.shape[1]
    if tr:
        X = X.T
    X = r(X / (math.sqrt(float(np.sum(X * X))) + NS_EPS))
    for _ in range(NS_STEPS):
        A = r(X @ X.T)
        B = r(b * A + c * (A @ A))
        X = r(a * X + B @ X)
    return X.T if tr else X


def momentum(M: np.ndarray, g_bf16: np.ndarray, mu: float) -> np.ndarray:
    """M <- mu * M + float(g) in binary32 (two roundings)."""
    g = (np.asarray(g_bf16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return (np.float32(mu) * M.astype(np.float32) + g).astype(np.float32)


def apply_update(theta: np.ndarray, O: np.ndarray, R: int, C: int, lr: float, wd: float):
    """theta * (1 - lr wd) - (lr 0.2 sqrt(max(R, C))) * O in binary32, the
    two scalars computed in binary64 and rounded once."""
    c_decay = np.float32(1.0 - lr * wd)
    scale = np.float32(lr * 0.2 * math.sqrt(max(R, C)))
    return (theta.astype(np.float32) * c_decay - scale * O.astype(np.float32)).astype(np.float32)
