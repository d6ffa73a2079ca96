"""Pins of the oracle planner against brute force, closed forms, a hand
derivation and invariants (planning problem of the veScale-FSDP page,
section 'Grouped communication: structure-aware planning (Algorithm 1)')."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth import ELEMENT, ROWS, TILE, TensorSpec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cap(specs, g):
    tot = 0
    for s in specs:
        d = oracle.derive(s, g)
        tot += d.N + d.A
    return (tot + g - 1) // g * g + g


@pytest.mark.parametrize("g_coll", [1, 2, 4, 16])
def test_bruteforce_agrees_on_random_tiny(g_coll):
    rng = np.random.default_rng(1000 + g_coll)
    n_cases = 0
    for _ in range(700):
        specs = synth.random_tiny_specs(rng)
        m = int(rng.integers(1, 5))
        got = oracle.plan_bucket(specs, m, g_coll)
        bf = oracle.plan_bruteforce(specs, m, g_coll, _cap(specs, g_coll))
        assert bf is not None
        assert got == bf, (specs, m, g_coll)
        assert oracle.check_plan(specs, m, g_coll, got[0], got[1]) == 0
        n_cases += 1
    assert n_cases == 700


def test_tiny_workload_hand_derivation():
    gold = json.load(open(os.path.join(GOLDEN, "tiny_plan.json")))
    w = synth.tiny()
    S, off = oracle.plan_bucket(w.specs, w.m, w.g_coll)
    assert S == gold["S"]
    assert off == gold["offsets"]
    assert w.m * S - w.real_elems == gold["padding"]


def test_element_granularity_is_flat_concatenation():
    # Element granularity with g_coll = 1 is the flat (FSDP1/ZeRO) layout:
    # offsets are prefix sums and S = ceil(total / m).
    rng = np.random.default_rng(7)
    for _ in range(50):
        sizes = [int(x) for x in rng.integers(1, 200, size=int(rng.integers(1, 8)))]
        specs = [TensorSpec(f"t{i}", (s,), ELEMENT) for i, s in enumerate(sizes)]
        m = int(rng.integers(1, 9))
        S, off = oracle.plan_bucket(specs, m, 1)
        assert S == math.ceil(sum(sizes) / m)
        assert off == list(np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int))


def test_single_rank_closed_form():
    # m = 1: no rank boundary inside the buffer; each tensor starts at the
    # next multiple of its alignment and S rounds the end up to g_coll.
    rng = np.random.default_rng(3)
    for _ in range(100):
        specs = synth.random_tiny_specs(rng, n_max=6, elems_max=200)
        g = int(rng.choice([1, 2, 4, 16]))
        S, off = oracle.plan_bucket(specs, 1, g)
        e = 0
        exp = []
        for s in specs:
            d = oracle.derive(s, g)
            o = -(-e // d.A) * d.A
            exp.append(o)
            e = o + d.N
        assert off == exp
        assert S == -(-e // g) * g


def test_single_tensor_full_blocks_closed_form():
    # One tensor of n_b full blocks of cut unit u with g_coll | u: a rank
    # holds at most floor(S/u) whole blocks, so S = ceil(n_b / m) * u.
    for (R, C, k, m, g) in [(96, 4, 8, 5, 4), (64, 3, 4, 3, 1), (256, 16, 32, 3, 16),
                            (40, 2, 5, 4, 2), (128, 8, 16, 6, 8)]:
        nb = R // k
        spec = TensorSpec("w", (R, C), ROWS, k)
        S, off = oracle.plan_bucket([spec], m, g)
        u = k * C
        assert u % g == 0
        assert S == math.ceil(nb / m) * u, (R, C, k, m, g)
        assert off == [0]


def test_feasibility_not_monotone_in_S():
    # One [2,4] tensor with 1-row blocks (cut unit 4), 2 ranks, g_coll 1:
    # S = 4 works, S = 5, 6, 7 do not, S = 8 does.  A bisection over S would
    # be unsound, so the planner scans.
    spec = [TensorSpec("w", (2, 4), ROWS, 1)]
    pattern = [oracle.feasible_at(spec, 2, 1, S) is not None for S in range(4, 9)]
    assert pattern == [True, False, False, False, True]
    assert oracle.plan_bucket(spec, 2, 1) == (4, [0])


def test_tile_block_positions_match_numpy_slicing():
    rng = np.random.default_rng(5)
    for _ in range(30):
        R, Cc = int(rng.integers(2, 40)), int(rng.integers(1, 40))
        br, bc = int(rng.integers(2, 9)), int(rng.integers(1, 9))
        spec = TensorSpec("w", (R, Cc), TILE, br, bc)
        d = oracle.derive(spec, 1)
        grid = np.arange(R * Cc).reshape(R, Cc)
        nbc = -(-Cc // bc)
        seen = np.zeros(R * Cc, dtype=int)
        for k in range(d.nblk):
            i, j = divmod(k, nbc)
            exp = grid[i * br:(i + 1) * br, j * bc:(j + 1) * bc].ravel() + 1000
            got = oracle.block_positions(spec, 1000, k)
            assert np.array_equal(got, exp)
            seen[got - 1000] += 1
        assert (seen == 1).all()


def test_rows_block_positions_and_counts():
    spec = TensorSpec("w", (10, 3), ROWS, 4)
    d = oracle.derive(spec, 1)
    assert d.nblk == 3 and d.u == 12 and d.b == 12
    assert list(oracle.block_positions(spec, 0, 2)) == list(range(24, 30))
    spec3 = TensorSpec("e", (2, 5, 3), ROWS, 4)      # leading dims fold into rows
    d3 = oracle.derive(spec3, 16)
    assert (d3.R, d3.C, d3.nblk, d3.u, d3.A) == (10, 3, 3, 12, 48)


@pytest.mark.parametrize("name", ["llama_layer", "llama8b_tiles", "moe"])
def test_invariants_on_workloads(name):
    w = synth.WORKLOADS[name]()
    L = oracle.Layout(w.specs, w.m, w.g_coll)
    for b in range(min(L.nb, 2)):
        idx = [i for i, s in enumerate(w.specs) if s.bucket == b]
        assert oracle.check_plan([w.specs[i] for i in idx], w.m, w.g_coll, L.S[b],
                                 [L.offsets[i] for i in idx]) == 0


def test_workload_layouts_hand_checked():
    # Hand checks: a tensor longer than 2S forces S to a multiple of its cut
    # unit (q: 128*4096 and down: 128*14336 for the tiled layer; 128*2880
    # for the fused experts).
    w = synth.llama8b_tiles(layers=1)
    S, off = oracle.plan_bucket(w.specs, w.m, w.g_coll)
    assert S == 3670016 == 7 * 524288 == 2 * 1835008
    assert off[6] == 159645696 and off[6] % 1835008 == 0
    w = synth.moe_bucket()
    S, off = oracle.plan_bucket(w.specs, w.m, w.g_coll)
    assert S == 46 * 368640
    assert off == [0, 530841600, 796262400]


def test_invariant_checker_catches_planted_mistakes():
    w = synth.tiny()
    S, off = oracle.plan_bucket(w.specs, w.m, w.g_coll)
    assert oracle.check_plan(w.specs, w.m, w.g_coll, S, off) == 0
    bad = list(off)
    bad[3] += 1                                   # bias misaligned
    assert oracle.check_plan(w.specs, w.m, w.g_coll, S, bad) == 4
    bad = list(off)
    bad[1] = off[0] + 1024                        # W2 overlaps W1
    assert oracle.check_plan(w.specs, w.m, w.g_coll, S, bad) == 2
    # a larger S with the same offsets is valid but not minimal
    assert oracle.check_plan(w.specs, w.m, w.g_coll, 2 * S, off) == 5
    # W1 at 0 with S = 5120: rank boundary 5120 cuts a 32-row band of W1
    bad = [0, 8192, 14336, 18432]
    assert oracle.check_plan(w.specs, w.m, w.g_coll, S, bad) == 1
    # slices too small for the content
    assert oracle.check_plan(w.specs, w.m, w.g_coll, 4096, off) == 3


# ----------------------------------------------------- planner variants

def test_cut_unit_alignment_reading_tiny_hand_derivation():
    """Other reading of the alignment rule: offsets aligned to lcm(g_coll,
    cut unit) (golden file: S = 6144, W1 @ 0, W2 @ 6144, W3 @ 12288, bias @
    16384)."""
    gold = json.load(open(os.path.join(GOLDEN, "tiny_plan.json")))
    w = synth.tiny()
    S, off = oracle.plan_bucket(w.specs, w.m, w.g_coll, align_unit=True)
    assert S == gold["S_if_alignment_used_cut_unit"]
    assert off == gold["offsets_if_alignment_used_cut_unit"]
    assert oracle.check_plan(w.specs, w.m, w.g_coll, S, off, align_unit=True) == 0


@pytest.mark.parametrize("g_coll", [1, 4, 16])
def test_bruteforce_agrees_with_cut_unit_alignment(g_coll):
    rng = np.random.default_rng(3000 + g_coll)
    for _ in range(300):
        specs = synth.random_tiny_specs(rng)
        m = int(rng.integers(1, 5))
        got = oracle.plan_bucket(specs, m, g_coll, align_unit=True)
        cap = 0
        for s in specs:
            d = oracle.derive(s, g_coll, align_unit=True)
            cap += d.N + d.A
        bf = oracle.plan_bruteforce(specs, m, g_coll, (cap + g_coll - 1) // g_coll * g_coll + g_coll,
                                    align_unit=True)
        assert got == bf, (specs, m, g_coll)


@pytest.mark.parametrize("order", [oracle.ORDER_BY_BLOCK, oracle.ORDER_BY_SIZE])
def test_orders_plan_the_permuted_list(order):
    """A reordered plan is the brute-force optimum of the permuted list
    (block size, or element count, descending; ties keep the given order)."""
    rng = np.random.default_rng(4000 + order)
    for _ in range(300):
        specs = synth.random_tiny_specs(rng)
        m = int(rng.integers(1, 5))
        g = int(rng.choice([1, 2, 4, 16]))
        d = [oracle.derive(s, g) for s in specs]
        key = (lambda i: (-d[i].b, i)) if order == oracle.ORDER_BY_BLOCK else (lambda i: (-d[i].N, i))
        perm = sorted(range(len(specs)), key=key)
        S, off = oracle.plan_bucket(specs, m, g, order=order)
        bf = oracle.plan_bruteforce([specs[i] for i in perm], m, g, _cap(specs, g))
        assert bf is not None and S == bf[0]
        assert [off[i] for i in perm] == bf[1]
        assert oracle.check_plan([specs[i] for i in perm], m, g, S, [off[i] for i in perm]) == 0


def test_order_changes_S_hand_example():
    """m = 3, g_coll = 4; t0 = 14 elements (element blocks), t1 = [16, 1] in
    3 x 1 tiles (cut unit 3, block 3, alignment lcm(4, 3) = 12).
    Given order: t0 @ 0, so t1 starts at 24 at the earliest.  S = 12 leaves
    36 elements, too few; at S = 16 the boundary 32 cuts t1 8 elements in
    (not a multiple of 3) and t1 @ 36 overflows 48; at S = 20 t1 @ 24 ends
    on the boundary 40.  Hence S = 20.
    By size: t1 @ 0 is cut at 12 (a multiple of 3) when S = 12, the lower
    bound roundup(ceil(30 / 3), 4); t0 follows @ 16.  Hence S = 12."""
    specs = [TensorSpec("t0", (14,), ELEMENT), TensorSpec("t1", (16, 1), TILE, 3, 1)]
    assert oracle.plan_bucket(specs, 3, 4) == (20, [0, 24])
    assert oracle.plan_bucket(specs, 3, 4, order=oracle.ORDER_BY_SIZE) == (12, [16, 0])
    assert oracle.plan_bucket(specs, 3, 4, order=oracle.ORDER_BY_BLOCK) == (12, [16, 0])


@pytest.mark.parametrize("g_coll", [1, 2, 4])
def test_scan_skip_rule_rejects_only_infeasible_S(g_coll):
    """The oracle scan skips an S when a tensor longer than 2S would need S to
    be a multiple of its cut unit.  Every S the rule skips must have no
    placement at all, by exhaustive enumeration at that S."""
    rng = np.random.default_rng(77 + g_coll)
    skipped = 0
    cases = []
    for _ in range(600):
        cases.append((synth.random_tiny_specs(rng, n_max=3, elems_max=48), int(rng.integers(2, 5))))
    # one dominant multi-row tensor over several ranks makes the rule fire
    for R, C, k in ((12, 2, 1), (8, 3, 2), (10, 2, 3), (9, 4, 1)):
        cases.append(([TensorSpec("big", (R, C), ROWS, k), TensorSpec("b", (3,), ELEMENT)], 4))
        cases.append(([TensorSpec("a", (2,), ELEMENT), TensorSpec("big", (R, C), TILE, 2, 1)], 3))
    for specs, m in cases:
        total = sum(s.numel for s in specs)
        S0 = -(-(-(-total // m)) // g_coll) * g_coll
        for S in range(S0, _cap(specs, g_coll) + 1, g_coll):
            if not oracle.wide_tensor_ok(specs, g_coll, S):
                skipped += 1
                assert oracle.bruteforce_feasible_at(specs, m, g_coll, S) is None, (specs, m, S)
    assert skipped > 50
