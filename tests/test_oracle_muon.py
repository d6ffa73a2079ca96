"""Pins of the distributed-Muon oracle (oracle/muon.py) against closed
forms, brute force and library routines -- never against itself.

Newton-Schulz: the iteration maps every singular value through the scalar
quintic p(x) = a x + b x^3 + c x^5 and keeps the singular vectors, so on a
matrix built as Q1 diag(s) Q2^T the binary64 result must be
Q1 diag(p^5(s / ||s||)) Q2^T.  SelectRoot: exhaustive search for the best
makespan on small inputs and Graham's bound for the longest-processing-
time rule.  Rounding: the bf16 rule against the C oracle's binary32 rule
(itself pinned against torch) and hand-computed ties."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import muon


def _orth(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


def _p5(x):
    a, b, c = muon.NS_COEFFS
    for _ in range(muon.NS_STEPS):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


@pytest.mark.parametrize("R,C", [(24, 40), (40, 24), (32, 32), (7, 50)])
def test_newton_schulz_acts_on_singular_values_by_the_quintic(R, C):
    rng = np.random.default_rng(R * 100 + C)
    n = min(R, C)
    s = np.sort(rng.uniform(0.01, 3.0, n))[::-1]
    s[-1] = 1e-4                                   # a nearly singular direction too
    Q1, Q2 = _orth(rng, R)[:, :n], _orth(rng, C)[:, :n]
    U = (Q1 * s) @ Q2.T
    got = muon.newton_schulz5(U, bf16=False)
    x = s / (math.sqrt(float(np.sum(s * s))) + muon.NS_EPS)
    exp = (Q1 * _p5(x)) @ Q2.T
    assert np.abs(got - exp).max() < 1e-12


def test_newton_schulz_rank_one_closed_form():
    # u v^T / (|u| |v|) has one singular value 1: the result is p^5(1) u^ v^T
    rng = np.random.default_rng(5)
    u, v = rng.standard_normal(17), rng.standard_normal(29)
    got = muon.newton_schulz5(np.outer(u, v), bf16=False)
    f = _p5(1.0 / (1.0 + muon.NS_EPS / (np.linalg.norm(u) * np.linalg.norm(v))))
    exp = f * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert np.abs(got - exp).max() < 1e-13
    assert 0.68 < _p5(1.0) < 0.72                    # 1 is not a fixed point of the quintic


def test_newton_schulz_transpose_symmetry():
    rng = np.random.default_rng(9)
    U = rng.standard_normal((20, 36))
    for bf in (False, True):
        a = muon.newton_schulz5(U, bf16=bf)
        assert np.array_equal(muon.newton_schulz5(U.T, bf16=bf), a.T)


def test_newton_schulz_bf16_close_to_exact():
    # storing the five steps' values in bf16 moves the result by about a
    # percent of its norm (8 significant bits, 16 roundings, damped by the
    # iteration)
    rng = np.random.default_rng(3)
    U = rng.standard_normal((96, 160)) * 1e-3
    a, b = muon.newton_schulz5(U, True), muon.newton_schulz5(U, False)
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 2e-2
    sv = np.linalg.svd(b, compute_uv=False)
    assert 0.6 < sv.min() and sv.max() < 1.25         # the band the quintic drives towards


def test_bf16_round_matches_the_binary32_rule_and_hand_ties():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-30).astype(np.float32)])
    exp = oracle.bf16_to_f32(oracle.bf16(x)).astype(np.float64)
    assert np.array_equal(muon.bf16_round(x.astype(np.float64)), exp)
    one = 1.0
    assert muon.bf16_round(np.array([one + 2 ** -8]))[0] == 1.0            # tie to even
    assert muon.bf16_round(np.array([one + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    assert muon.bf16_round(np.array([one + 2 ** -8 + 2 ** -40]))[0] == 1.0 + 2 ** -7
    assert muon.bf16_round(np.array([-(one + 3 * 2 ** -8)]))[0] == -(1.0 + 2 ** -6)
    # a binary64 value whose binary32 rounding is a bf16 tie: rounding twice
    # (64 -> 32 -> 16) would go to even, the direct rule goes up
    v = 1.0 + 2 ** -8 + 2 ** -30
    assert np.float32(v) == np.float32(1.0 + 2 ** -8)
    assert muon.bf16_round(np.array([v]))[0] == 1.0 + 2 ** -7


def _best_makespan(costs, m):
    best = None
    for assign in itertools.product(range(m), repeat=len(costs)):
        load = [0] * m
        for c, r in zip(costs, assign):
            load[r] += c
        best = max(load) if best is None else min(best, max(load))
    return best


def test_select_roots_within_graham_bound_of_brute_force():
    rng = np.random.default_rng(11)
    for _ in range(300):
        n = int(rng.integers(1, 8))
        m = int(rng.integers(1, 4))
        shapes = [(int(rng.integers(1, 9)) * 8, int(rng.integers(1, 9)) * 8) for _ in range(n)]
        roots = muon.select_roots(shapes, m)
        costs = [muon.ns_flops(R, C) for R, C in shapes]
        assert len(roots) == n and all(0 <= r < m for r in roots)
        load = [0] * m
        for c, r in zip(costs, roots):
            load[r] += c
        opt = _best_makespan(costs, m)
        assert max(load) <= (4 / 3 - 1 / (3 * m)) * opt + 1e-9, (shapes, m)


def test_select_roots_special_cases():
    # no more matrices than ranks: one each, the costliest on rank 0
    shapes = [(64, 64), (256, 64), (128, 128), (64, 512)]
    roots = muon.select_roots(shapes, 8)
    cost = [muon.ns_flops(*s) for s in shapes]
    assert sorted(roots) == [0, 1, 2, 3]
    assert [roots[i] for i in sorted(range(4), key=lambda i: -cost[i])] == [0, 1, 2, 3]
    # equal costs: dealt out in turn
    assert muon.select_roots([(32, 32)] * 7, 3) == [0, 1, 2, 0, 1, 2, 0]
    assert muon.ns_flops(2048, 5632) == 5 * (4 * 2048 * 2048 * 5632 + 2 * 2048 ** 3)
    assert muon.ns_flops(5632, 2048) == muon.ns_flops(2048, 5632)


def test_root_layout_is_an_uneven_ragged_shard():
    sizes = [100, 7, 64, 33, 500]
    roots = [2, 0, 2, 1, 0]
    off, starts = muon.root_layout(sizes, roots, 4, align=16)
    assert starts[0] == 0 and all(starts[r] <= starts[r + 1] for r in range(4))
    for i, (n, r) in enumerate(zip(sizes, roots)):
        assert off[i] % 16 == 0 and starts[r] <= off[i] and off[i] + n <= starts[r + 1]
    # whole matrices, in the given order inside a region, never overlapping
    ivs = sorted((off[i], off[i] + sizes[i]) for i in range(5))
    assert all(a[1] <= b[0] for a, b in zip(ivs, ivs[1:]))
    assert starts[4] - starts[3] == 0                       # rank 3 roots nothing
    assert off[1] == 0 and off[4] == 16                     # rank 0: 7 elements, then 500 at 16


def test_momentum_and_update_rules_special_cases():
    rng = np.random.default_rng(2)
    g = oracle.bf16(rng.standard_normal(1000).astype(np.float32))
    gf = oracle.bf16_to_f32(g)
    M0 = rng.standard_normal(1000).astype(np.float32)
    assert np.array_equal(muon.momentum(M0, g, 0.0), gf)           # mu = 0: M = g exactly
    assert np.array_equal(muon.momentum(np.zeros(1000, np.float32), g, 0.95), gf)
    M = muon.momentum(M0, g, 0.5)                                  # exact: mu a power of two
    assert np.array_equal(M, (M0.astype(np.float64) * 0.5 + gf).astype(np.float32))
    th = rng.standard_normal(64).astype(np.float32)
    lr, wd = 1e-3, 0.01
    c = np.float32(1.0 - lr * wd)
    assert np.array_equal(muon.apply_update(th, np.zeros(64), 8, 8, lr, wd), th * c)
    # lr 0.2 sqrt(max(R, C)) = 2^-5 exactly for a 16 x 4 matrix and lr = 2^-5 / 0.8
    lr2 = 2 ** -5 / 0.8
    O = np.float32(0.5) * np.ones(64, np.float32)
    got = muon.apply_update(th, O, 16, 4, lr2, 0.0)
    assert np.array_equal(got, th - np.float32(2 ** -6))


def test_torch_bf16_of_float32_agrees_with_the_rounding_used():
    # the redistributed update is bf16(M) of a binary32 M: torch's rule
    x = torch.randn(4096, generator=torch.Generator().manual_seed(0))
    t = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(t, oracle.bf16(x.numpy()))
