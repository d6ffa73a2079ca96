"""GPU parity of distributed Muon against the oracle (oracle/muon.py),
through the C-ABI.

- gather (momentum and redistribution to the roots): bit-exact;
- apply (redistribution back and update), on a root buffer the test writes:
  bit-exact;
- orthogonalize (Newton-Schulz on bf16 MFMA products), on a root buffer the
  test writes: against the binary64 oracle and the oracle that rounds to
  bf16 where the kernels store.  Tolerance, derived from the arithmetic:
  bf16 keeps 8 significant bits (unit roundoff 2^-9); the iteration stores
  16 rounded values per matrix, binary32 sums add a little more, and the
  iteration damps errors in the directions it has converged -- about 1% of
  the result's Frobenius norm in all; the tests allow 3% against binary64
  and 2% against the bf16-storing oracle, and 6% of the largest |O| for any
  single element;
- per-root calls compose to the all-root call bit for bit, and touch only
  their root's region;
- a whole step (gather, orthogonalize, apply) against the oracle chain, the
  parameter tolerance following from the one on O.
Inputs are seeded and synthetic; no oracle input comes from the library."""
import math

import numpy as np
import pytest
import torch

import oracle
import sharded_state_raggedshard_amd as rs
import synth
from oracle import muon as om
from synth import ROWS, TensorSpec
from gpu_harness import dev_to_u16, log, make_plan, u16_to_dev

pytestmark = pytest.mark.gpu

LR, WD, MU = 1e-3, 0.01, 0.95


def _ragged_specs():
    # edge tiles of every kernel (sizes multiples of 8, not of 64 or 128), both
    # orientations, a square matrix, a 1-D tensor that is not a Muon matrix
    return [TensorSpec("a", (136, 200), ROWS, 8), TensorSpec("b", (200, 136), ROWS, 8),
            TensorSpec("n", (72,), ROWS, 8), TensorSpec("c", (64, 64), ROWS, 32),
            TensorSpec("d", (264, 520), ROWS, 8), TensorSpec("e", (520, 48), ROWS, 8)]


def _wide64_specs():
    # every dimension a multiple of 64, none of 256: the 256 x 256 product
    # kernel on partial tiles, with odd numbers of 64-column stages (K = 192,
    # 320, 448, 576) and a two-stage one (K = 128)
    return [TensorSpec("p", (320, 192), ROWS, 8), TensorSpec("q", (192, 448), ROWS, 8),
            TensorSpec("r", (576, 128), ROWS, 8), TensorSpec("s", (64, 64), ROWS, 8)]


def _mixed32_specs():
    # a matrix whose dimensions are multiples of 32 but not of 64 sends an
    # all-root call to the 128 x 128 kernel, while per-root calls of the other
    # root take the 256 x 256 kernel: the per-root test then compares the two
    # kernels bit for bit
    return [TensorSpec("u", (96, 160), ROWS, 8), TensorSpec("p", (320, 192), ROWS, 8),
            TensorSpec("q", (192, 448), ROWS, 8)]


CASES = {
    "ragged_m3": lambda: (_ragged_specs(), 3, 16),
    "wide64_m2": lambda: (_wide64_specs(), 2, 16),
    "mixed32_m2": lambda: (_mixed32_specs(), 2, 16),
    "llama_layer": lambda: (synth.llama_layer_2048().specs, 8, 16),
}


def _setup(name):
    specs, m, g = CASES[name]()
    L = oracle.Layout(specs, m, g)
    plan = make_plan(specs, m, g)
    mats = [i for i, s in enumerate(specs) if len(s.shape) == 2]
    mu = rs.Muon(plan, mats).upload()
    shapes = [tuple(specs[i].shape) for i in mats]
    return specs, L, plan, mats, mu, shapes


def _rand_bf16(n, seed, stream, sigma):
    return synth.normal_bf16(n, sigma, seed, stream).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name", list(CASES))
def test_gather_bitexact(name):
    specs, L, plan, mats, mu, shapes = _setup(name)
    log(f"muon gather {name}")
    g = np.zeros(L.total, np.uint16)
    M0 = np.zeros(L.total, np.float32)
    for k, i in enumerate(mats):
        p, n = L.pos[i], specs[i].numel
        g[p:p + n] = _rand_bf16(n, 1, k, 1e-3)
        M0[p:p + n] = synth.uniform_params(n, 2, k, lo=-1e-3, hi=1e-3).numpy()
    d_g, d_M = u16_to_dev(g), torch.from_numpy(M0.copy()).cuda()
    root = torch.full((mu.root_elems + 64,), 0x3C3C, dtype=torch.int16, device="cuda")
    rs.rs_muon_gather(mu.h, rs.RS_ALL, d_M, d_g, root, momentum=MU)
    got_M, got_root = d_M.cpu().numpy(), dev_to_u16(root)
    exp_M = M0.copy()
    exp_root = np.full(mu.root_elems + 64, 0x3C3C, np.uint16)
    for k, i in enumerate(mats):
        p, n = L.pos[i], specs[i].numel
        exp_M[p:p + n] = om.momentum(M0[p:p + n], g[p:p + n], MU)
        exp_root[mu.offsets[k]:mu.offsets[k] + n] = oracle.bf16(exp_M[p:p + n])
    assert np.array_equal(got_M.view(np.uint32), exp_M.view(np.uint32))
    assert np.array_equal(got_root, exp_root)
    mu.free()
    plan.free()


@pytest.mark.parametrize("name", list(CASES))
def test_apply_bitexact(name):
    specs, L, plan, mats, mu, shapes = _setup(name)
    log(f"muon apply {name}")
    theta = np.full(L.total, 7.0, np.float32)
    for i, s in enumerate(specs):
        theta[L.pos[i]:L.pos[i] + s.numel] = synth.uniform_params(s.numel, 3, i).numpy()
    O = _rand_bf16(mu.root_elems, 4, 0, 0.05)
    d_th = torch.from_numpy(theta.copy()).cuda()
    rs.rs_muon_apply(mu.h, rs.RS_ALL, d_th, u16_to_dev(O), lr=LR, weight_decay=WD)
    exp = theta.copy()
    for k, i in enumerate(mats):
        p, n = L.pos[i], specs[i].numel
        R, C = shapes[k]
        o = oracle.bf16_to_f32(O[mu.offsets[k]:mu.offsets[k] + n])
        exp[p:p + n] = om.apply_update(theta[p:p + n], o, R, C, LR, WD)
    assert np.array_equal(d_th.cpu().numpy().view(np.uint32), exp.view(np.uint32))
    mu.free()
    plan.free()


def _fro(x):
    return math.sqrt(float(np.sum(np.asarray(x, np.float64) ** 2)))


def _check_O(got, U, what):
    ref64 = om.newton_schulz5(U, bf16=False)
    ref16 = om.newton_schulz5(U, bf16=True)
    e64 = _fro(got - ref64) / _fro(ref64)
    e16 = _fro(got - ref16) / _fro(ref16)
    emax = np.abs(got - ref64).max() / np.abs(ref64).max()
    log(f"  {what}: rel. Frobenius {e64:.2e} (binary64 oracle), {e16:.2e} (bf16 oracle), "
        f"max {emax:.2e}")
    assert e64 < 3e-2 and e16 < 2e-2 and emax < 6e-2, what


@pytest.mark.parametrize("name", list(CASES))
def test_orthogonalize_against_oracle(name):
    specs, L, plan, mats, mu, shapes = _setup(name)
    log(f"muon orthogonalize {name}")
    U = np.zeros(mu.root_elems, np.uint16)
    for k, (R, C) in enumerate(shapes):
        U[mu.offsets[k]:mu.offsets[k] + R * C] = _rand_bf16(R * C, 5, k, 1e-3)
    root = u16_to_dev(U)
    rs.rs_muon_orthogonalize(mu.h, rs.RS_ALL, root)
    got = dev_to_u16(root)
    for k, (R, C) in enumerate(shapes):
        u = oracle.bf16_to_f32(U[mu.offsets[k]:mu.offsets[k] + R * C]).reshape(R, C)
        o = (got[mu.offsets[k]:mu.offsets[k] + R * C].astype(np.uint32) << 16).view(np.float32).reshape(R, C)
        _check_O(o.astype(np.float64), u.astype(np.float64), f"{specs[mats[k]].name} {R}x{C}")
    mu.free()
    plan.free()


def _ns5_torch_fp32(u: torch.Tensor) -> torch.Tensor:
    """The quintic Newton-Schulz iteration (five steps, coefficients of the
    published iteration) in binary32 torch matrix products on the device,
    with no bf16 rounding: a reference for sizes the binary64 oracle is too
    slow for."""
    a, b, c = om.NS_COEFFS
    x = u / (torch.linalg.matrix_norm(u) + 1e-7)
    tr = x.shape[0] > x.shape[1]
    if tr:
        x = x.t().contiguous()
    for _ in range(5):
        A = x @ x.t()
        B = b * A + c * (A @ A)
        x = a * x + B @ x
    return x.t().contiguous() if tr else x


def test_orthogonalize_full_size_llama8b_layer():
    """The 2-D matrices of one Llama-8B-shaped layer (up to 14336 x 4096, 64
    ranks): the kernels against the binary32 torch iteration on the device,
    within the tolerance of the bf16 storage (3% of ||O||_F), and every
    singular value of O at most 1.25 (the quintic maps (0, 1] below it)."""
    w = synth.llama8b_tiles(layers=1)
    log("muon orthogonalize llama8b layer")
    plan = make_plan(w.specs, w.m, w.g_coll)
    mats = [i for i, s in enumerate(w.specs) if len(s.shape) == 2]
    mu = rs.Muon(plan, mats).upload()
    gen = torch.Generator(device="cuda").manual_seed(12)
    root = torch.zeros(mu.root_elems, dtype=torch.int16, device="cuda")
    shapes = [tuple(w.specs[i].shape) for i in mats]
    for k, (R, C) in enumerate(shapes):
        u = (torch.randn(R * C, device="cuda", generator=gen) * 1e-3).to(torch.bfloat16)
        root[mu.offsets[k]:mu.offsets[k] + R * C] = u.view(torch.int16)
    U = root.clone()
    rs.rs_muon_orthogonalize(mu.h, rs.RS_ALL, root)
    torch.cuda.synchronize()
    for k, (R, C) in enumerate(shapes):
        sl = slice(mu.offsets[k], mu.offsets[k] + R * C)
        u = U[sl].view(torch.bfloat16).float().reshape(R, C)
        o = root[sl].view(torch.bfloat16).float().reshape(R, C)
        ref = _ns5_torch_fp32(u)
        err = (torch.linalg.matrix_norm(o - ref) / torch.linalg.matrix_norm(ref)).item()
        assert err < 0.03, (w.specs[mats[k]].name, err)
        assert torch.linalg.svdvals(o).max().item() <= 1.25, w.specs[mats[k]].name
    mu.free()
    plan.free()


def test_per_root_calls_compose_and_stay_in_their_region():
    specs, L, plan, mats, mu, shapes = _setup("ragged_m3")
    log("muon per-root calls")
    U = np.zeros(mu.root_elems, np.uint16)
    for k, (R, C) in enumerate(shapes):
        U[mu.offsets[k]:mu.offsets[k] + R * C] = _rand_bf16(R * C, 6, k, 1e-3)
    whole = u16_to_dev(U)
    rs.rs_muon_orthogonalize(mu.h, rs.RS_ALL, whole)
    parts = u16_to_dev(U)
    for r in range(plan.m):
        before = dev_to_u16(parts)
        rs.rs_muon_orthogonalize(mu.h, r, parts)
        after = dev_to_u16(parts)
        lo, hi = mu.regions[r], mu.regions[r + 1]
        assert np.array_equal(before[:lo], after[:lo]) and np.array_equal(before[hi:], after[hi:])
    assert np.array_equal(dev_to_u16(parts), dev_to_u16(whole))
    mu.free()
    plan.free()


@pytest.mark.parametrize("name", list(CASES))
def test_per_root_calls_on_streams_match_the_all_root_call(name):
    """Per-root calls on four streams at once (each root's matrices use their
    own workspace buffers) give the all-root call's bits."""
    specs, L, plan, mats, mu, shapes = _setup(name)
    log(f"muon per-root calls on streams {name}")
    U = np.zeros(mu.root_elems, np.uint16)
    for k, (R, C) in enumerate(shapes):
        U[mu.offsets[k]:mu.offsets[k] + R * C] = _rand_bf16(R * C, 8, k, 1e-3)
    whole = u16_to_dev(U)
    rs.rs_muon_orthogonalize(mu.h, rs.RS_ALL, whole)
    parts = u16_to_dev(U)
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in range(4)]
    for st in streams:
        st.wait_stream(main)
    roots = sorted(set(mu.roots))
    for j, r in enumerate(roots):
        rs.rs_muon_orthogonalize(mu.h, r, parts, stream=streams[j % len(streams)])
    for st in streams:
        main.wait_stream(st)
    torch.cuda.synchronize()
    assert len(roots) > 1
    assert np.array_equal(dev_to_u16(parts), dev_to_u16(whole))
    mu.free()
    plan.free()


@pytest.mark.parametrize("name", list(CASES))
def test_whole_step_against_oracle(name):
    """gather -> orthogonalize -> apply over all roots, two free-running steps,
    against the oracle chain (momentum exact, O within the tolerance above)."""
    specs, L, plan, mats, mu, shapes = _setup(name)
    log(f"muon whole step {name}")
    theta = np.zeros(L.total, np.float32)
    for i, s in enumerate(specs):
        theta[L.pos[i]:L.pos[i] + s.numel] = synth.uniform_params(s.numel, 8, i).numpy()
    M = np.zeros(L.total, np.float32)
    d_th, d_M = torch.from_numpy(theta.copy()).cuda(), torch.from_numpy(M.copy()).cuda()
    root = torch.zeros(mu.root_elems, dtype=torch.int16, device="cuda")
    ref_th, ref_M = theta.copy(), M.copy()
    for t in (1, 2):
        g = np.zeros(L.total, np.uint16)
        for k, i in enumerate(mats):
            g[L.pos[i]:L.pos[i] + specs[i].numel] = _rand_bf16(specs[i].numel, 10 + t, k, 1e-3)
        rs.rs_muon_gather(mu.h, rs.RS_ALL, d_M, u16_to_dev(g), root, momentum=MU)
        rs.rs_muon_orthogonalize(mu.h, rs.RS_ALL, root)
        rs.rs_muon_apply(mu.h, rs.RS_ALL, d_th, root, lr=LR, weight_decay=WD)
        got_th = d_th.cpu().numpy()
        for k, i in enumerate(mats):
            p, n = L.pos[i], specs[i].numel
            R, C = shapes[k]
            ref_M[p:p + n] = om.momentum(ref_M[p:p + n], g[p:p + n], MU)
            U = oracle.bf16_to_f32(oracle.bf16(ref_M[p:p + n])).reshape(R, C).astype(np.float64)
            O = om.newton_schulz5(U, bf16=False)
            new = om.apply_update(ref_th[p:p + n], O.reshape(-1), R, C, LR, WD)
            # free-running: errors of earlier steps add up (the decay only shrinks them)
            scale = LR * 0.2 * math.sqrt(max(R, C))
            tol = t * scale * 6e-2 * np.abs(O).max() + 1e-6 * np.abs(new)
            assert (np.abs(got_th[p:p + n] - new) <= tol).all(), (specs[i].name, t)
            ref_th[p:p + n] = new
        assert np.array_equal(d_M.cpu().numpy().view(np.uint32), ref_M.view(np.uint32))
    mu.free()
    plan.free()
