"""One rank's training-state update with the library, end to end.

    python -m sharded_state_raggedshard_amd.example

Plans two tensors over m = 4 ranks, each in a bucket of its own (a matrix
in 128 x 128 tiles, a vector in 32-element blocks: neither needs padding),
copies fp32 master parameters in, and runs a few steps of: global L2 norm
with the clipping coefficient, the blockwise-int8 AdamW step of rank `rank`
(grad scale = the coefficient, bf16 copy-in of the new parameters fused),
zeroing of the gradients, copy-out to per-parameter bf16 views.  On m GPUs each rank would run the same calls on its own slices
and an AllGather / ReduceScatter would move the bf16 buffer between them; on
one GPU every rank's slice lives in the same arrays.
"""
from __future__ import annotations

import torch

import sharded_state_raggedshard_amd as rs
from synth import ROWS, TILE, TensorSpec


def main(steps: int = 3, rank: int = rs.RS_ALL) -> dict:
    specs = [TensorSpec("w", (1024, 512), TILE, 128, 128, bucket=0),
             TensorSpec("b", (1024,), ROWS, 32, bucket=1)]
    plan = rs.Plan(specs, 4, 16).upload()  # layout, then its device tables
    dev = "cuda"
    total, nblk = plan.total, plan.n_blocks
    # the DBuffers: one array per state in the planned layout
    theta = torch.zeros(total, device=dev)                      # fp32 master
    grad = torch.zeros(total, dtype=torch.int16, device=dev)    # bf16 bits
    qm = torch.zeros(total, dtype=torch.int8, device=dev)       # int8 m codes
    qv = torch.zeros(total, dtype=torch.uint8, device=dev)      # uint8 v codes
    amax_m = torch.zeros(nblk, device=dev)                      # one absmax per block
    amax_v = torch.zeros(nblk, device=dev)
    gathered = torch.zeros(total, dtype=torch.int16, device=dev)  # bf16 buffer
    sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
    clip = torch.zeros(1, device=dev)
    # per-parameter views: fp32 masters to copy in, bf16 weights to copy out
    masters = [torch.randn(s.numel, device=dev) * 0.02 for s in specs]
    weights = [torch.zeros(s.numel, dtype=torch.int16, device=dev) for s in specs]
    rs.rs_bind_views(plan.h, rs.RS_VIEW_F32_SRC, masters)
    rs.rs_bind_views(plan.h, rs.RS_VIEW_BF16_DST, weights)
    rs.rs_pack_shard(plan.h, rs.RS_ALL, rs.RS_ALL, gathered)  # initial bf16 copy-in
    for i, s in enumerate(specs):  # the master in the planned layout
        theta[plan.pos[i]:plan.pos[i] + s.numel] = masters[i]
    for t in range(1, steps + 1):
        # stands in for the backward pass accumulating into the grad DBuffer
        for i, s in enumerate(specs):
            g = (torch.randn(s.numel, device=dev) * 1e-3).to(torch.bfloat16)
            grad[plan.pos[i]:plan.pos[i] + s.numel] = g.view(torch.int16)
        rs.rs_group_l2norm_clip(plan.h, rs.RS_ALL, rank, grad, rs.RS_BF16, 1.0, sumsq, clip)
        rs.rs_adam8_step(plan.h, rs.RS_ALL, rank, theta, grad, qm, qv, amax_m, amax_v,
                         lr=1e-3, step=t, grad_scale=clip, bf16_out=gathered)
        rs.rs_group_zero(plan.h, rs.RS_ALL, rank, grad, rs.RS_BF16)
        rs.rs_unpack_full(plan.h, rs.RS_ALL, gathered)
    rs.rs_plan_check_device(plan.h)  # no cross-workgroup wait gave up
    torch.cuda.synchronize()
    out = {"S": plan.S, "padding": plan.padding, "grad_norm": sumsq.sqrt().item(),
           "clip": clip.item(), "weights": [w.view(torch.bfloat16).float() for w in weights],
           "theta": theta, "plan": plan}
    return out


if __name__ == "__main__":
    r = main()
    print(f"S per bucket {r['S']}, padding {r['padding']}, last grad norm {r['grad_norm']:.4g}, "
          f"clip {r['clip']:.4g}")
    r["plan"].free()
