"""Python binding of libraggedshard (RaggedShard / DBuffer shard-state path
for MI355X).  Argument marshalling only: every step runs in the HIP
library; torch supplies device memory and streams.

Functions carry the names of the C entry points in include/raggedshard.h.
Device arguments accept a torch tensor (its data_ptr is passed) or an int
address.  A non-OK status raises RaggedShardError with rs_last_error().
The library must be built (python -m sharded_state_raggedshard_amd.build);
importing this module fails loudly otherwise.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libraggedshard.so")

RS_OK, RS_EINVAL, RS_EOVERFLOW, RS_ESTATE, RS_EHIP, RS_ENOMEM = 0, -1, -2, -3, -4, -5
RS_ELEMENT, RS_ROWS, RS_TILE = 0, 1, 2
RS_F32, RS_BF16 = 0, 1
RS_VIEW_F32_SRC, RS_VIEW_BF16_DST = 0, 1
RS_ORDER_GIVEN = 0
RS_ORDER_BY_BLOCK = 1
RS_ORDER_BY_SIZE = 2
RS_ORDER_MASK = 0xff
RS_ALIGN_CUT_UNIT = 0x100
RS_SPLIT_TWO_PASS, RS_SPLIT_COOPERATIVE, RS_SPLIT_ORDERED = 0, 1, 2
RS_ALL = -1

# every entry point declared in include/raggedshard.h
EXPORTS = (
    "rs_plan_layout", "rs_plan_free", "rs_plan_info", "rs_plan_bucket", "rs_plan_offsets",
    "rs_plan_rank_blocks", "rs_plan_set_chunk", "rs_plan_set_split_mode", "rs_plan_chunk_count",
    "rs_plan_device_bytes", "rs_plan_upload", "rs_bind_views", "rs_pack_shard", "rs_unpack_full",
    "rs_pack_shard_fp8", "rs_unpack_full_fp8",
    "rs_group_zero", "rs_group_scale", "rs_group_l2norm", "rs_group_l2norm_static",
    "rs_clip_coef", "rs_group_l2norm_clip", "rs_adam8_step", "rs_adam8_step_fp8",
    "rs_plan_check_device", "rs_plan_status_offset", "rs_last_error", "rs_version",
    "rs_muon_plan", "rs_muon_free", "rs_muon_layout", "rs_muon_device_bytes", "rs_muon_upload",
    "rs_muon_gather", "rs_muon_orthogonalize", "rs_muon_apply",
)


class RaggedShardError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class rs_tensor_spec(C.Structure):
    _fields_ = [("ndim", C.c_int32), ("gran", C.c_int32), ("br", C.c_int32), ("bc", C.c_int32),
                ("bucket", C.c_int32), ("reserved", C.c_int32), ("shape", C.c_int64 * 4)]


class rs_adam_hparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("step", C.c_int64)]


class rs_muon_hparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("momentum", C.c_double), ("weight_decay", C.c_double)]


_lib = None


def lib() -> C.CDLL:
    """Loads libraggedshard.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "'python -m sharded_state_raggedshard_amd.build'")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    P64 = C.POINTER(C.c_int64)
    P32 = C.POINTER(C.c_int32)
    sig = {
        "rs_plan_layout": ([C.POINTER(rs_tensor_spec), i32, i32, i64, i32, C.POINTER(vp)], C.c_int),
        "rs_plan_free": ([vp], None),
        "rs_plan_info": ([vp, P32, P32, P32, P64, P64], C.c_int),
        "rs_plan_bucket": ([vp, i32, P64, P64, P64, P64], C.c_int),
        "rs_plan_offsets": ([vp, P64, P64], C.c_int),
        "rs_plan_rank_blocks": ([vp, i32, i32, P64, P64], C.c_int),
        "rs_plan_set_chunk": ([vp, i64], C.c_int),
        "rs_plan_set_split_mode": ([vp, i32], C.c_int),
        "rs_plan_chunk_count": ([vp, P64, P64], C.c_int),
        "rs_plan_device_bytes": ([vp], C.c_size_t),
        "rs_plan_upload": ([vp, vp, C.c_size_t, vp], C.c_int),
        "rs_bind_views": ([vp, i32, C.POINTER(vp), vp], C.c_int),
        "rs_pack_shard": ([vp, i32, i32, vp, vp], C.c_int),
        "rs_unpack_full": ([vp, i32, vp, vp], C.c_int),
        "rs_pack_shard_fp8": ([vp, i32, i32, vp, vp, vp], C.c_int),
        "rs_unpack_full_fp8": ([vp, i32, vp, vp, vp], C.c_int),
        "rs_group_zero": ([vp, i32, i32, vp, i32, vp], C.c_int),
        "rs_group_scale": ([vp, i32, i32, vp, i32, C.c_float, vp], C.c_int),
        "rs_group_l2norm": ([vp, i32, i32, vp, i32, vp, vp], C.c_int),
        "rs_group_l2norm_static": ([vp, i32, i32, vp, i32, vp, vp], C.c_int),
        "rs_clip_coef": ([vp, C.c_double, vp, vp], C.c_int),
        "rs_group_l2norm_clip": ([vp, i32, i32, vp, i32, C.c_double, vp, vp, vp], C.c_int),
        "rs_adam8_step": ([vp, i32, i32, vp, vp, vp, vp, vp, vp, C.POINTER(rs_adam_hparams), vp,
                           vp, vp], C.c_int),
        "rs_adam8_step_fp8": ([vp, i32, i32, vp, vp, vp, vp, vp, vp, C.POINTER(rs_adam_hparams),
                               vp, vp, vp, vp, vp], C.c_int),
        "rs_plan_check_device": ([vp, vp], C.c_int),
        "rs_plan_status_offset": ([vp, C.POINTER(C.c_size_t)], C.c_int),
        "rs_muon_plan": ([vp, P32, i32, C.POINTER(vp)], C.c_int),
        "rs_muon_free": ([vp], None),
        "rs_muon_layout": ([vp, P32, P64, P64, P64], C.c_int),
        "rs_muon_device_bytes": ([vp], C.c_size_t),
        "rs_muon_upload": ([vp, vp, C.c_size_t, vp], C.c_int),
        "rs_muon_gather": ([vp, i32, vp, vp, C.POINTER(rs_muon_hparams), vp, vp], C.c_int),
        "rs_muon_orthogonalize": ([vp, i32, vp, vp], C.c_int),
        "rs_muon_apply": ([vp, i32, vp, vp, C.POINTER(rs_muon_hparams), vp], C.c_int),
        "rs_last_error": ([], C.c_char_p),
        "rs_version": ([], C.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(st: int):
    if st != RS_OK:
        raise RaggedShardError(st, lib().rs_last_error().decode())


def _ptr(x) -> Optional[int]:
    """Device address of a torch tensor (or an int / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def make_specs(specs) -> "C.Array":
    """Duck-typed specs (.shape, .gran, .br, .bc, .bucket) -> rs_tensor_spec[]."""
    arr = (rs_tensor_spec * len(specs))()
    for i, s in enumerate(specs):
        shp = tuple(int(d) for d in s.shape)
        if not 1 <= len(shp) <= 4:
            raise ValueError(f"tensor {i}: ndim must be 1..4")
        arr[i].ndim = len(shp)
        arr[i].gran = int(s.gran)
        arr[i].br = int(s.br)
        arr[i].bc = int(s.bc)
        arr[i].bucket = int(getattr(s, "bucket", 0))
        arr[i].reserved = 0
        for k, d in enumerate(shp):
            arr[i].shape[k] = d
    return arr


# ------------------------------------------------------- entry points

def rs_plan_layout(specs, m: int, g_coll: int, order: int = RS_ORDER_GIVEN) -> int:
    h = C.c_void_p()
    arr = make_specs(specs)
    _check(lib().rs_plan_layout(arr, len(specs), m, g_coll, order, C.byref(h)))
    return h.value


def rs_plan_free(plan: int) -> None:
    lib().rs_plan_free(plan)


def rs_plan_info(plan: int):
    n, nb, m = C.c_int32(), C.c_int32(), C.c_int32()
    tot, nblk = C.c_int64(), C.c_int64()
    _check(lib().rs_plan_info(plan, C.byref(n), C.byref(nb), C.byref(m), C.byref(tot),
                              C.byref(nblk)))
    return n.value, nb.value, m.value, tot.value, nblk.value


def rs_plan_bucket(plan: int, bucket: int):
    S, base, pad, nblk = C.c_int64(), C.c_int64(), C.c_int64(), C.c_int64()
    _check(lib().rs_plan_bucket(plan, bucket, C.byref(S), C.byref(base), C.byref(pad),
                                C.byref(nblk)))
    return S.value, base.value, pad.value, nblk.value


def rs_plan_offsets(plan: int):
    n = rs_plan_info(plan)[0]
    off = (C.c_int64 * n)()
    blk = (C.c_int64 * n)()
    _check(lib().rs_plan_offsets(plan, off, blk))
    return list(off), list(blk)


def rs_plan_rank_blocks(plan: int, bucket: int, rank: int):
    a, c = C.c_int64(), C.c_int64()
    _check(lib().rs_plan_rank_blocks(plan, bucket, rank, C.byref(a), C.byref(c)))
    return a.value, c.value


def rs_plan_set_chunk(plan: int, chunk_elems: int) -> None:
    _check(lib().rs_plan_set_chunk(plan, chunk_elems))


def rs_plan_set_split_mode(plan: int, mode: int) -> None:
    _check(lib().rs_plan_set_split_mode(plan, mode))


def rs_plan_chunk_count(plan: int) -> int:
    n = C.c_int64()
    _check(lib().rs_plan_chunk_count(plan, C.byref(n), None))
    return n.value


def rs_plan_chunk_elems(plan: int) -> int:
    """Chunk size (elements per step workgroup) in effect for the plan."""
    c = C.c_int64()
    _check(lib().rs_plan_chunk_count(plan, None, C.byref(c)))
    return c.value


def rs_plan_device_bytes(plan: int) -> int:
    n = lib().rs_plan_device_bytes(plan)
    if n == 0:
        raise RaggedShardError(RS_EINVAL, lib().rs_last_error().decode())
    return int(n)


def rs_plan_upload(plan: int, workspace, nbytes: int, stream=None) -> None:
    _check(lib().rs_plan_upload(plan, _ptr(workspace), nbytes, _stream(stream)))


def rs_bind_views(plan: int, which: int, views: Sequence, stream=None) -> None:
    arr = (C.c_void_p * len(views))(*[_ptr(v) for v in views])
    _check(lib().rs_bind_views(plan, which, arr, _stream(stream)))


def rs_pack_shard(plan: int, bucket: int, rank: int, buf, stream=None) -> None:
    _check(lib().rs_pack_shard(plan, bucket, rank, _ptr(buf), _stream(stream)))


def rs_unpack_full(plan: int, bucket: int, buf, stream=None) -> None:
    _check(lib().rs_unpack_full(plan, bucket, _ptr(buf), _stream(stream)))


def rs_pack_shard_fp8(plan: int, bucket: int, rank: int, buf, scale, stream=None) -> None:
    """buf: uint8 codes (one byte per buffer element); scale: fp32 per block."""
    _check(lib().rs_pack_shard_fp8(plan, bucket, rank, _ptr(buf), _ptr(scale), _stream(stream)))


def rs_unpack_full_fp8(plan: int, bucket: int, buf, scale, stream=None) -> None:
    _check(lib().rs_unpack_full_fp8(plan, bucket, _ptr(buf), _ptr(scale), _stream(stream)))


def rs_group_zero(plan: int, bucket: int, rank: int, buf, dtype: int, stream=None) -> None:
    _check(lib().rs_group_zero(plan, bucket, rank, _ptr(buf), dtype, _stream(stream)))


def rs_group_scale(plan: int, bucket: int, rank: int, buf, dtype: int, s: float,
                   stream=None) -> None:
    _check(lib().rs_group_scale(plan, bucket, rank, _ptr(buf), dtype, C.c_float(s),
                                _stream(stream)))


def rs_group_l2norm(plan: int, bucket: int, rank: int, buf, dtype: int, sumsq,
                    stream=None) -> None:
    _check(lib().rs_group_l2norm(plan, bucket, rank, _ptr(buf), dtype, _ptr(sumsq),
                                 _stream(stream)))


def rs_group_l2norm_static(plan: int, bucket: int, rank: int, buf, dtype: int, sumsq,
                           stream=None) -> None:
    _check(lib().rs_group_l2norm_static(plan, bucket, rank, _ptr(buf), dtype, _ptr(sumsq),
                                        _stream(stream)))


def rs_clip_coef(sumsq, max_norm: float, scale, stream=None) -> None:
    _check(lib().rs_clip_coef(_ptr(sumsq), max_norm, _ptr(scale), _stream(stream)))


def rs_group_l2norm_clip(plan: int, bucket: int, rank: int, buf, dtype: int, max_norm: float,
                         sumsq, scale, stream=None) -> None:
    _check(lib().rs_group_l2norm_clip(plan, bucket, rank, _ptr(buf), dtype, max_norm, _ptr(sumsq),
                                      _ptr(scale), _stream(stream)))


def rs_adam8_step(plan: int, bucket: int, rank: int, master, grad, qm, qv, amax_m, amax_v,
                  lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1,
                  grad_scale=None, bf16_out=None, stream=None) -> None:
    hp = rs_adam_hparams(lr, beta1, beta2, eps, weight_decay, int(step))
    _check(lib().rs_adam8_step(plan, bucket, rank, _ptr(master), _ptr(grad), _ptr(qm), _ptr(qv),
                               _ptr(amax_m), _ptr(amax_v), C.byref(hp), _ptr(grad_scale),
                               _ptr(bf16_out), _stream(stream)))


def rs_adam8_step_fp8(plan: int, bucket: int, rank: int, master, grad, qm, qv, amax_m, amax_v,
                      fp8, fp8_scale, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                      weight_decay=0.01, step=1, grad_scale=None, bf16_out=None,
                      stream=None) -> None:
    """rs_adam8_step plus the FP8 codes (uint8, one per buffer element) and
    block scales (fp32 per global block) of the new master."""
    hp = rs_adam_hparams(lr, beta1, beta2, eps, weight_decay, int(step))
    _check(lib().rs_adam8_step_fp8(plan, bucket, rank, _ptr(master), _ptr(grad), _ptr(qm),
                                   _ptr(qv), _ptr(amax_m), _ptr(amax_v), C.byref(hp),
                                   _ptr(grad_scale), _ptr(bf16_out), _ptr(fp8),
                                   _ptr(fp8_scale), _stream(stream)))


def rs_plan_check_device(plan: int, stream=None) -> None:
    _check(lib().rs_plan_check_device(plan, _stream(stream)))


def rs_plan_status_offset(plan: int) -> int:
    off = C.c_size_t()
    _check(lib().rs_plan_status_offset(plan, C.byref(off)))
    return int(off.value)


def rs_muon_plan(plan: int, tensors: Sequence[int]) -> int:
    arr = (C.c_int32 * len(tensors))(*[int(t) for t in tensors])
    h = C.c_void_p()
    _check(lib().rs_muon_plan(plan, arr, len(tensors), C.byref(h)))
    return h.value


def rs_muon_free(muon: int) -> None:
    lib().rs_muon_free(muon)


def rs_muon_layout(muon: int, n: int, m: int):
    """(roots, root-buffer offsets, region starts [m + 1], root-buffer length)."""
    roots = (C.c_int32 * n)()
    offs = (C.c_int64 * n)()
    regs = (C.c_int64 * (m + 1))()
    total = C.c_int64()
    _check(lib().rs_muon_layout(muon, roots, offs, regs, C.byref(total)))
    return list(roots), list(offs), list(regs), int(total.value)


def rs_muon_device_bytes(muon: int) -> int:
    return int(lib().rs_muon_device_bytes(muon))


def rs_muon_upload(muon: int, workspace, nbytes: int, stream=None) -> None:
    _check(lib().rs_muon_upload(muon, _ptr(workspace), nbytes, _stream(stream)))


def _muon_hp(lr, momentum, weight_decay):
    return rs_muon_hparams(float(lr), float(momentum), float(weight_decay))


def rs_muon_gather(muon: int, root: int, mom, grad, root_buf, momentum: float = 0.95,
                   stream=None) -> None:
    hp = _muon_hp(0.0, momentum, 0.0)
    _check(lib().rs_muon_gather(muon, root, _ptr(mom), _ptr(grad), C.byref(hp), _ptr(root_buf),
                                _stream(stream)))


def rs_muon_orthogonalize(muon: int, root: int, root_buf, stream=None) -> None:
    _check(lib().rs_muon_orthogonalize(muon, root, _ptr(root_buf), _stream(stream)))


def rs_muon_apply(muon: int, root: int, master, root_buf, lr: float = 1e-3,
                  weight_decay: float = 0.01, stream=None) -> None:
    hp = _muon_hp(lr, 0.0, weight_decay)
    _check(lib().rs_muon_apply(muon, root, _ptr(master), _ptr(root_buf), C.byref(hp),
                               _stream(stream)))


def rs_last_error() -> str:
    return lib().rs_last_error().decode()


def rs_version() -> str:
    return lib().rs_version().decode()


# ------------------------------------------------------------ plan object

class Plan:
    """Owns one rs_plan handle and (after upload) its device workspace."""

    def __init__(self, specs, m: int, g_coll: int, chunk: Optional[int] = None,
                 split_mode: int = RS_SPLIT_COOPERATIVE, order: int = RS_ORDER_GIVEN):
        self.h = rs_plan_layout(specs, m, g_coll, order)
        self.specs = list(specs)
        if chunk is not None:
            rs_plan_set_chunk(self.h, chunk)
        rs_plan_set_split_mode(self.h, split_mode)
        self.n, self.nb, self.m, self.total, self.n_blocks = rs_plan_info(self.h)
        self.offsets, self.blk0 = rs_plan_offsets(self.h)
        self.S, self.base, self.padding = [], [], []
        for b in range(self.nb):
            S, base, pad, _ = rs_plan_bucket(self.h, b)
            self.S.append(S)
            self.base.append(base)
            self.padding.append(pad)
        self.pos = [self.base[int(getattr(s, "bucket", 0))] + self.offsets[i]
                    for i, s in enumerate(self.specs)]
        self.workspace = None

    def upload(self, device="cuda", stream=None):
        import torch
        nbytes = rs_plan_device_bytes(self.h)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        rs_plan_upload(self.h, self.workspace, nbytes, stream)
        return self

    def free(self):
        if self.h:
            rs_plan_free(self.h)
            self.h = None
        self.workspace = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class Muon:
    """Owns one rs_muon handle (distributed Muon over some tensors of a plan)
    and, after upload, its device workspace."""

    def __init__(self, plan: "Plan", tensors: Sequence[int]):
        self.h = rs_muon_plan(plan.h, tensors)
        self.tensors = list(tensors)
        self.m = plan.m
        self.roots, self.offsets, self.regions, self.root_elems = rs_muon_layout(
            self.h, len(self.tensors), self.m)
        self.workspace = None

    def upload(self, device="cuda", stream=None):
        import torch
        nbytes = rs_muon_device_bytes(self.h)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        rs_muon_upload(self.h, self.workspace, nbytes, stream)
        return self

    def free(self):
        if self.h:
            rs_muon_free(self.h)
            self.h = None
        self.workspace = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
