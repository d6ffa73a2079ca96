"""Helpers shared by the GPU tests: device buffers for a workload, host
copies for the oracle, comparison against the tolerances of the step."""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

import oracle
import sharded_state_raggedshard_amd as rs
import synth

SENT_CODE = 0x5A


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def u16_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev_to_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def padding_mask(L: oracle.Layout) -> np.ndarray:
    mask = np.ones(L.total, dtype=bool)
    for i, s in enumerate(L.specs):
        mask[L.pos[i]:L.pos[i] + s.numel] = False
    return mask


@dataclass
class HostState:
    theta: np.ndarray
    grad: np.ndarray
    qm: np.ndarray
    qv: np.ndarray
    am: np.ndarray
    av: np.ndarray

    def copy(self) -> "HostState":
        return HostState(*(x.copy() for x in (self.theta, self.grad, self.qm, self.qv, self.am,
                                              self.av)))


def host_state(L: oracle.Layout, specs, seed: int, sigma: float, warm: bool,
               sentinel: bool = True) -> HostState:
    """Synthetic state in the planned layout (padding holds sentinels)."""
    theta = np.full(L.total, np.float32(7.0) if sentinel else 0, dtype=np.float32)
    grad = np.zeros(L.total, dtype=np.uint16)
    for i, s in enumerate(specs):
        p = L.pos[i]
        theta[p:p + s.numel] = synth.uniform_params(s.numel, seed, 2 * i).numpy()
        grad[p:p + s.numel] = synth.normal_bf16(s.numel, sigma, seed, 2 * i + 1).view(
            torch.int16).numpy().view(np.uint16)
    qm = np.zeros(L.total, dtype=np.int8)
    qv = np.zeros(L.total, dtype=np.uint8)
    am = np.zeros(L.n_blocks, dtype=np.float32)
    av = np.zeros(L.n_blocks, dtype=np.float32)
    if warm:
        qm[:] = synth.random_codes_m(L.total, seed, 10001).numpy()
        qv[:] = synth.random_codes_v(L.total, seed, 10002).numpy()
        am[:] = synth.random_absmax(L.n_blocks, 1e-3, seed, 10003).numpy()
        av[:] = synth.random_absmax(L.n_blocks, 1e-6, seed, 10004).numpy()
    if sentinel:
        pad = padding_mask(L)
        qm[pad] = SENT_CODE
        qv[pad] = SENT_CODE
    return HostState(theta, grad, qm, qv, am, av)


def fresh_grads(L: oracle.Layout, specs, seed: int, sigma: float, step: int) -> np.ndarray:
    grad = np.zeros(L.total, dtype=np.uint16)
    for i, s in enumerate(specs):
        p = L.pos[i]
        grad[p:p + s.numel] = synth.normal_bf16(s.numel, sigma, seed + 1000 * step,
                                                2 * i + 1).view(torch.int16).numpy().view(np.uint16)
    return grad


class DevState:
    def __init__(self, h: HostState, with_out: bool = False):
        self.theta = torch.from_numpy(h.theta.copy()).cuda()
        self.grad = u16_to_dev(h.grad)
        self.qm = torch.from_numpy(h.qm.copy()).cuda()
        self.qv = torch.from_numpy(h.qv.copy()).cuda()
        self.am = torch.from_numpy(h.am.copy()).cuda()
        self.av = torch.from_numpy(h.av.copy()).cuda()
        self.out = torch.zeros(h.theta.size, dtype=torch.int16, device="cuda") if with_out else None

    def host(self) -> HostState:
        torch.cuda.synchronize()
        return HostState(self.theta.cpu().numpy(), dev_to_u16(self.grad), self.qm.cpu().numpy(),
                         self.qv.cpu().numpy(), self.am.cpu().numpy(), self.av.cpu().numpy())

    def step(self, plan: rs.Plan, bucket: int, rank: int, t: int, gscale=None):
        rs.rs_adam8_step(plan.h, bucket, rank, self.theta, self.grad, self.qm, self.qv, self.am,
                         self.av, step=t, grad_scale=gscale, bf16_out=self.out)


def assert_step_close(got: HostState, exp: HostState, mask: Optional[np.ndarray] = None,
                      what: str = ""):
    """Tolerances of the step: params |d| <= 1e-8 + 1e-6 |ref|; codes differ
    by at most 1 on at most 1e-4 of the entries; absmax relative 1e-6."""
    sel = slice(None) if mask is None else mask
    th_g, th_e = got.theta[sel], exp.theta[sel]
    bad = np.abs(th_g - th_e) > 1e-8 + 1e-6 * np.abs(th_e)
    assert not bad.any(), f"{what}: {bad.sum()} params out of tolerance"
    n = th_e.size
    for name, a, b in (("qm", got.qm[sel], exp.qm[sel]), ("qv", got.qv[sel], exp.qv[sel])):
        d = np.abs(a.astype(np.int32) - b.astype(np.int32))
        assert d.max(initial=0) <= 1, f"{what}: {name} differs by {d.max()}"
        assert (d != 0).sum() <= max(1, int(1e-4 * n)), f"{what}: {name} {(d != 0).sum()} differ"
    for name, a, b in (("amax_m", got.am, exp.am), ("amax_v", got.av, exp.av)):
        assert np.allclose(a, b, rtol=1e-6, atol=0), f"{what}: {name}"


def make_plan(specs, m, g_coll, chunk=None, mode=rs.RS_SPLIT_COOPERATIVE, options=0) -> rs.Plan:
    return rs.Plan(specs, m, g_coll, chunk=chunk, split_mode=mode, order=options).upload()


def check_plan_matches(plan: rs.Plan, L: oracle.Layout):
    assert plan.S == L.S and plan.base == L.base and plan.offsets == L.offsets
    assert plan.blk0 == L.blk0 and plan.total == L.total and plan.n_blocks == L.n_blocks
