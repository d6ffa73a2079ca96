"""ctypes front end of the plain CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by
the CPU-baseline leg of bench.py, never by the HIP library or its Python
binding.  Every function here is argument marshalling around oracle.c;
the arithmetic lives there.

Tensor specs are duck-typed: any object with .shape, .gran, .br, .bc and
.bucket (see synth.TensorSpec).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE binary32, no FMA
    contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


class _Tensor(C.Structure):
    _fields_ = [("ndim", C.c_int32), ("shape", C.c_int64 * 4), ("gran", C.c_int32),
                ("br", C.c_int32), ("bc", C.c_int32), ("align_unit", C.c_int32)]


class _Derived(C.Structure):
    _fields_ = [("N", C.c_int64), ("R", C.c_int64), ("C", C.c_int64), ("u", C.c_int64),
                ("b", C.c_int64), ("A", C.c_int64), ("nblk", C.c_int64)]


class _Layout(C.Structure):
    _fields_ = [("n", C.c_int), ("nb", C.c_int), ("m", C.c_int),
                ("spec", C.POINTER(_Tensor)), ("bucket_of", C.POINTER(C.c_int32)),
                ("pos", C.POINTER(C.c_int64)), ("blk0", C.POINTER(C.c_int64)),
                ("S", C.POINTER(C.c_int64)), ("base", C.POINTER(C.c_int64)),
                ("g_coll", C.c_int64)]


class _HParams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("step", C.c_int64)]


class _Scalars(C.Structure):
    _fields_ = [(k, C.c_float) for k in
                ("beta1", "beta2", "omega1", "omega2", "eps", "c_decay", "step_size", "kappa")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        P64 = C.POINTER(C.c_int64)
        L.orc_derive.argtypes = [C.POINTER(_Tensor), C.c_int64, C.POINTER(_Derived)]
        L.orc_place_fixed_S.argtypes = [C.POINTER(_Derived), C.c_int, C.c_int, C.c_int64,
                                        C.c_int64, P64]
        L.orc_plan_bucket.argtypes = [C.POINTER(_Tensor), C.c_int, C.c_int, C.c_int64, P64, P64]
        L.orc_plan_bruteforce.argtypes = [C.POINTER(_Tensor), C.c_int, C.c_int, C.c_int64,
                                          C.c_int64, P64, P64]
        L.orc_check_plan.argtypes = [C.POINTER(_Tensor), C.c_int, C.c_int, C.c_int64,
                                     C.c_int64, P64]
        L.orc_bruteforce_feasible_at.argtypes = [C.POINTER(_Tensor), C.c_int, C.c_int,
                                                 C.c_int64, C.c_int64, P64]
        L.orc_wide_tensor_ok.argtypes = [C.POINTER(_Tensor), C.c_int, C.c_int64, C.c_int64]
        L.orc_count_cut_blocks.argtypes = [C.POINTER(_Tensor), C.c_int, C.c_int64, P64]
        L.orc_count_cut_blocks.restype = C.c_int64
        L.orc_bf16.argtypes = [C.c_float]
        L.orc_bf16.restype = C.c_uint16
        L.orc_bf16_to_f32.argtypes = [C.c_uint16]
        L.orc_bf16_to_f32.restype = C.c_float
        L.orc_bf16_array.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        LP = C.POINTER(_Layout)
        L.orc_pack.argtypes = [LP, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
        L.orc_unpack.argtypes = [LP, C.c_int, C.c_void_p, C.c_void_p]
        L.orc_group_zero.argtypes = [LP, C.c_int, C.c_int, C.c_void_p, C.c_int]
        L.orc_group_scale.argtypes = [LP, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_float]
        L.orc_group_sumsq.argtypes = [LP, C.c_int, C.c_int, C.c_void_p, C.c_int]
        L.orc_group_sumsq.restype = C.c_double
        L.orc_clip_coef.argtypes = [C.c_double, C.c_double]
        L.orc_clip_coef.restype = C.c_float
        L.orc_scalars_from.argtypes = [C.POINTER(_HParams), C.POINTER(_Scalars)]
        L.orc_adam8_block.argtypes = [C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.POINTER(C.c_float), C.POINTER(C.c_float),
                                      C.POINTER(_Scalars), C.c_float, C.c_void_p]
        L.orc_adam8_step.argtypes = [LP, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(_HParams),
                                     C.c_float, C.c_void_p]
        L.orc_block_positions.argtypes = [C.POINTER(_Tensor), C.c_int64, C.c_int64, P64,
                                          C.c_int64]
        L.orc_block_positions.restype = C.c_int64
        L.orc_fp8_block.argtypes = [C.c_int64, C.c_void_p, C.c_void_p]
        L.orc_fp8_block.restype = C.c_float
        L.orc_e4m3.argtypes = [C.c_float]
        L.orc_e4m3.restype = C.c_uint8
        L.orc_e4m3_to_f32.argtypes = [C.c_uint8]
        L.orc_e4m3_to_f32.restype = C.c_float
        L.orc_pack_fp8.argtypes = [LP, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
        L.orc_unpack_fp8.argtypes = [LP, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
        _lib = L
    return _lib


def _tensor(spec, align_unit: bool = False) -> _Tensor:
    t = _Tensor()
    t.align_unit = 1 if align_unit else 0
    shp = tuple(int(s) for s in spec.shape)
    t.ndim = len(shp)
    for i, s in enumerate(shp):
        t.shape[i] = s
    t.gran = int(spec.gran)
    t.br = int(spec.br)
    t.bc = int(spec.bc)
    return t


def _tensors(specs, align_unit: bool = False) -> "C.Array":
    arr = (_Tensor * len(specs))()
    for i, s in enumerate(specs):
        arr[i] = _tensor(s, align_unit)
    return arr


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


# ----------------------------------------------------------------- planner

@dataclass
class Derived:
    N: int
    R: int
    C: int
    u: int
    b: int
    A: int
    nblk: int


def derive(spec, g_coll: int, align_unit: bool = False) -> Derived:
    d = _Derived()
    if lib().orc_derive(C.byref(_tensor(spec, align_unit)), g_coll, C.byref(d)) != 0:
        raise ValueError(f"invalid spec {spec}")
    return Derived(d.N, d.R, d.C, d.u, d.b, d.A, d.nblk)


# Tensor orders of the planning rule (veScale-FSDP page, section "Grouped
# communication: structure-aware planning"): the default order, by block
# size, by shape.  Read here as: given order; block size (elements of one
# block) descending; element count descending; ties keep the given order.
ORDER_GIVEN, ORDER_BY_BLOCK, ORDER_BY_SIZE = 0, 1, 2


def placement_order(specs: Sequence, g_coll: int, order: int = ORDER_GIVEN) -> List[int]:
    """Indices of specs in the order the planner places them."""
    idx = list(range(len(specs)))
    if order == ORDER_GIVEN:
        return idx
    d = [derive(s, g_coll) for s in specs]
    if order == ORDER_BY_BLOCK:
        return sorted(idx, key=lambda i: -d[i].b)
    if order == ORDER_BY_SIZE:
        return sorted(idx, key=lambda i: -d[i].N)
    raise ValueError(f"unknown order {order}")


def plan_bucket(specs: Sequence, m: int, g_coll: int, order: int = ORDER_GIVEN,
                align_unit: bool = False):
    """(S, offsets) of one bucket: minimal S, lexicographically smallest
    offsets (in placement order); offsets[i] belongs to specs[i]."""
    n = len(specs)
    po = placement_order(specs, g_coll, order)
    off = (C.c_int64 * n)()
    S = C.c_int64()
    rc = lib().orc_plan_bucket(_tensors([specs[i] for i in po], align_unit), n, m, g_coll,
                               C.byref(S), off)
    if rc != 0:
        raise ValueError("oracle planner: invalid input")
    res = [0] * n
    for j, i in enumerate(po):
        res[i] = int(off[j])
    return int(S.value), res


def plan_bruteforce(specs: Sequence, m: int, g_coll: int, S_cap: int, align_unit: bool = False):
    """Exhaustive search, tensors in the given order."""
    n = len(specs)
    off = (C.c_int64 * n)()
    S = C.c_int64()
    rc = lib().orc_plan_bruteforce(_tensors(specs, align_unit), n, m, g_coll, S_cap, C.byref(S),
                                   off)
    if rc != 0:
        return None
    return int(S.value), [int(x) for x in off]


def feasible_at(specs: Sequence, m: int, g_coll: int, S: int, align_unit: bool = False):
    """Greedy placement at one fixed S, or None if infeasible."""
    n = len(specs)
    d = (_Derived * n)()
    for i, s in enumerate(specs):
        if lib().orc_derive(C.byref(_tensor(s, align_unit)), g_coll, C.byref(d[i])) != 0:
            raise ValueError(f"invalid spec {s}")
    off = (C.c_int64 * n)()
    if lib().orc_place_fixed_S(d, n, m, g_coll, S, off):
        return [int(x) for x in off]
    return None


def bruteforce_feasible_at(specs: Sequence, m: int, g_coll: int, S: int,
                           align_unit: bool = False):
    """Exhaustive search at one fixed S (tiny inputs): the lexicographically
    smallest offsets, or None if no placement exists at S."""
    n = len(specs)
    off = (C.c_int64 * n)()
    rc = lib().orc_bruteforce_feasible_at(_tensors(specs, align_unit), n, m, g_coll, S, off)
    if rc < 0:
        raise ValueError("invalid input")
    return [int(x) for x in off] if rc == 1 else None


def wide_tensor_ok(specs: Sequence, g_coll: int, S: int, align_unit: bool = False) -> bool:
    """The planner scan's skip rule at S (False: S is skipped)."""
    rc = lib().orc_wide_tensor_ok(_tensors(specs, align_unit), len(specs), g_coll, S)
    if rc < 0:
        raise ValueError("invalid input")
    return rc == 1


def check_plan(specs: Sequence, m: int, g_coll: int, S: int, offsets: Sequence[int],
               align_unit: bool = False) -> int:
    """Invariants I1..I5; specs and offsets in placement order."""
    n = len(specs)
    off = (C.c_int64 * n)(*offsets)
    return int(lib().orc_check_plan(_tensors(specs, align_unit), n, m, g_coll, S, off))


def count_cut_blocks(specs: Sequence, S: int, offsets: Sequence[int]) -> int:
    """Blocks with elements in two ranks of size S, tensor i at offsets[i]
    (any offsets; the count invariant I1 requires to be zero)."""
    n = len(specs)
    off = (C.c_int64 * n)(*offsets)
    r = int(lib().orc_count_cut_blocks(_tensors(specs), n, S, off))
    if r < 0:
        raise ValueError("invalid input")
    return r


def block_first_position(spec, p0: int, k: int) -> int:
    out = np.empty(1, dtype=np.int64)
    lib().orc_block_positions(C.byref(_tensor(spec)), p0, k,
                              out.ctypes.data_as(C.POINTER(C.c_int64)), 1)
    return int(out[0])


def block_positions(spec, p0: int, k: int) -> np.ndarray:
    cnt = lib().orc_block_positions(C.byref(_tensor(spec)), p0, k, None, 0)
    out = np.empty(max(cnt, 1), dtype=np.int64)
    lib().orc_block_positions(C.byref(_tensor(spec)), p0, k,
                              out.ctypes.data_as(C.POINTER(C.c_int64)), cnt)
    return out[:cnt]


# --------------------------------------------------------------- fp8

def e4m3(x: float) -> int:
    """OCP E4M3 code of x (nearest, ties to even, saturating at +-448)."""
    return int(lib().orc_e4m3(float(x)))


def fp8_block(x: np.ndarray):
    """(scale, codes) of one quantisation block under the FP8 copy-in rule."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.zeros(x.size, dtype=np.uint8)
    s = lib().orc_fp8_block(x.size, _ptr(x), _ptr(q))
    return float(np.float32(s)), q


def e4m3_to_f32(q: int) -> float:
    return float(lib().orc_e4m3_to_f32(int(q)))


# ------------------------------------------------------------------ layout

class Layout:
    """Multi-bucket layout computed by the oracle planner: each bucket is
    planned on its own and the buckets are concatenated."""

    def __init__(self, specs: Sequence, m: int, g_coll: int, bucket_plans=None,
                 order: int = ORDER_GIVEN, align_unit: bool = False):
        self.specs = list(specs)
        self.m = int(m)
        self.g_coll = int(g_coll)
        self.order = int(order)
        self.align_unit = bool(align_unit)
        nb = 1 + max(int(s.bucket) for s in self.specs)
        self.nb = nb
        self.S: List[int] = []
        self.base: List[int] = []
        self.offsets = [0] * len(self.specs)
        base = 0
        cache = {}
        for b in range(nb):
            idx = [i for i, s in enumerate(self.specs) if int(s.bucket) == b]
            if not idx:
                raise ValueError(f"bucket {b} is empty")
            key = tuple((tuple(self.specs[i].shape), self.specs[i].gran, self.specs[i].br,
                         self.specs[i].bc) for i in idx) + (self.order, self.align_unit)
            if bucket_plans is not None:
                S, off = bucket_plans[b]
            elif key in cache:
                # identical tensor lists give identical plans (pure function)
                S, off = cache[key]
            else:
                S, off = plan_bucket([self.specs[i] for i in idx], self.m, self.g_coll,
                                     self.order, self.align_unit)
                cache[key] = (S, off)
            self.S.append(S)
            self.base.append(base)
            for j, i in enumerate(idx):
                self.offsets[i] = off[j]
            base += self.m * S
        self.total = base
        self.derived = [derive(s, self.g_coll, self.align_unit) for s in self.specs]
        self.pos = [self.base[int(s.bucket)] + self.offsets[i] for i, s in enumerate(self.specs)]
        # global block ids: bucket order, then buffer order of the tensors,
        # then block order
        order = sorted(range(len(self.specs)), key=lambda i: (int(self.specs[i].bucket),
                                                              self.pos[i]))
        self.blk0 = [0] * len(self.specs)
        nblk = 0
        for i in order:
            self.blk0[i] = nblk
            nblk += self.derived[i].nblk
        self.n_blocks = nblk
        self._build_c()

    def _build_c(self):
        n = len(self.specs)
        self._spec = _tensors(self.specs)
        self._bucket = (C.c_int32 * n)(*[int(s.bucket) for s in self.specs])
        self._pos = (C.c_int64 * n)(*self.pos)
        self._blk0 = (C.c_int64 * n)(*self.blk0)
        self._S = (C.c_int64 * self.nb)(*self.S)
        self._base = (C.c_int64 * self.nb)(*self.base)
        L = _Layout()
        L.n, L.nb, L.m = n, self.nb, self.m
        L.spec = C.cast(self._spec, C.POINTER(_Tensor))
        L.bucket_of = C.cast(self._bucket, C.POINTER(C.c_int32))
        L.pos = C.cast(self._pos, C.POINTER(C.c_int64))
        L.blk0 = C.cast(self._blk0, C.POINTER(C.c_int64))
        L.S = C.cast(self._S, C.POINTER(C.c_int64))
        L.base = C.cast(self._base, C.POINTER(C.c_int64))
        L.g_coll = self.g_coll
        self._L = L

    def padding(self, bucket: int) -> int:
        real = sum(self.derived[i].N for i, s in enumerate(self.specs) if int(s.bucket) == bucket)
        return self.m * self.S[bucket] - real

    def rank_of(self, pos: int) -> int:
        for b in range(self.nb):
            if self.base[b] <= pos < self.base[b] + self.m * self.S[b]:
                return (pos - self.base[b]) // self.S[b]
        raise ValueError(pos)

    def block_positions(self, t: int, k: int) -> np.ndarray:
        return block_positions(self.specs[t], self.pos[t], k)

    def block_first_position(self, t: int, k: int) -> int:
        return block_first_position(self.specs[t], self.pos[t], k)

    # -------------------------------------------------------------- ops
    def pack(self, bucket: int, rank: int, views: Sequence[np.ndarray], buf: np.ndarray):
        assert buf.dtype == np.uint16 and buf.size >= self.total
        vs = [np.ascontiguousarray(v, dtype=np.float32) for v in views]
        arr = (C.c_void_p * len(vs))(*[v.ctypes.data for v in vs])
        lib().orc_pack(C.byref(self._L), bucket, rank, arr, _ptr(buf))

    def pack_fp8(self, bucket: int, rank: int, views: Sequence[np.ndarray], buf: np.ndarray,
                 scales: np.ndarray):
        assert buf.dtype == np.uint8 and buf.size >= self.total
        assert scales.dtype == np.float32 and scales.size >= self.n_blocks
        vs = [np.ascontiguousarray(v, dtype=np.float32) for v in views]
        arr = (C.c_void_p * len(vs))(*[v.ctypes.data for v in vs])
        lib().orc_pack_fp8(C.byref(self._L), bucket, rank, arr, _ptr(buf), _ptr(scales))

    def unpack_fp8(self, bucket: int, views: Sequence[np.ndarray], buf: np.ndarray,
                   scales: np.ndarray):
        for v in views:
            assert v.dtype == np.uint16 and v.flags.c_contiguous
        arr = (C.c_void_p * len(views))(*[v.ctypes.data for v in views])
        lib().orc_unpack_fp8(C.byref(self._L), bucket, arr, _ptr(buf), _ptr(scales))

    def unpack(self, bucket: int, views: Sequence[np.ndarray], buf: np.ndarray):
        for v in views:
            assert v.dtype == np.uint16 and v.flags.c_contiguous
        arr = (C.c_void_p * len(views))(*[v.ctypes.data for v in views])
        lib().orc_unpack(C.byref(self._L), bucket, arr, _ptr(buf))

    def group_zero(self, bucket: int, rank: int, buf: np.ndarray):
        lib().orc_group_zero(C.byref(self._L), bucket, rank, _ptr(buf), _dtype_code(buf))

    def group_scale(self, bucket: int, rank: int, buf: np.ndarray, s: float):
        lib().orc_group_scale(C.byref(self._L), bucket, rank, _ptr(buf), _dtype_code(buf),
                              C.c_float(s))

    def group_sumsq(self, bucket: int, rank: int, buf: np.ndarray) -> float:
        return float(lib().orc_group_sumsq(C.byref(self._L), bucket, rank, _ptr(buf),
                                           _dtype_code(buf)))

    def adam8_step(self, bucket: int, rank: int, theta: np.ndarray, grad: np.ndarray,
                   qm: np.ndarray, qv: np.ndarray, amax_m: np.ndarray, amax_v: np.ndarray,
                   hp: "HParams", gscale: float = 1.0, out: Optional[np.ndarray] = None):
        assert theta.dtype == np.float32 and grad.dtype == np.uint16
        assert qm.dtype == np.int8 and qv.dtype == np.uint8
        assert amax_m.dtype == np.float32 and amax_v.dtype == np.float32
        lib().orc_adam8_step(C.byref(self._L), bucket, rank, _ptr(theta), _ptr(grad), _ptr(qm),
                             _ptr(qv), _ptr(amax_m), _ptr(amax_v), C.byref(hp.c()),
                             C.c_float(gscale), _ptr(out) if out is not None else None)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(a.dtype)


# ------------------------------------------------------------------ values

def bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    y = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


def bf16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    return (h.astype(np.uint32) << 16).view(np.float32)


def clip_coef(sumsq: float, max_norm: float) -> float:
    return float(lib().orc_clip_coef(sumsq, max_norm))


@dataclass
class HParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1

    def c(self) -> _HParams:
        return _HParams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                        int(self.step))


def scalars(hp: HParams) -> dict:
    s = _Scalars()
    lib().orc_scalars_from(C.byref(hp.c()), C.byref(s))
    return {k: float(getattr(s, k)) for k, _ in _Scalars._fields_}


def adam8_block(theta: np.ndarray, grad: np.ndarray, qm: np.ndarray, qv: np.ndarray,
                am: float, av: float, hp: HParams, gscale: float = 1.0, want_out=False):
    """One block on gathered arrays; returns (theta, qm, qv, am, av, out)."""
    th = np.ascontiguousarray(theta, dtype=np.float32).copy()
    g = np.ascontiguousarray(grad, dtype=np.uint16)
    m = np.ascontiguousarray(qm, dtype=np.int8).copy()
    v = np.ascontiguousarray(qv, dtype=np.uint8).copy()
    a_m = C.c_float(am)
    a_v = C.c_float(av)
    s = _Scalars()
    lib().orc_scalars_from(C.byref(hp.c()), C.byref(s))
    out = np.empty(th.size, dtype=np.uint16) if want_out else None
    lib().orc_adam8_block(th.size, _ptr(th), _ptr(g), _ptr(m), _ptr(v), C.byref(a_m),
                          C.byref(a_v), C.byref(s), C.c_float(gscale),
                          _ptr(out) if out is not None else None)
    return th, m, v, float(a_m.value), float(a_v.value), out
