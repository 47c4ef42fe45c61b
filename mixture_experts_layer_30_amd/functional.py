"""Buffer allocation around the C ABI, in the shape of the functional API the
MoK project card describes (get_workspace -> build_schedule -> forward ->
backward). torch provides the device memory; every computation happens in
libmok's kernels.
"""
from __future__ import annotations

import dataclasses

import torch

from . import (MOK_BF16, backward, buffer_sizes, build_schedule, forward, forward_fused, make_config,
               make_problem, mxfp8_quantize, mxfp8_quantize_transposed, schedule_layout)


@dataclasses.dataclass
class Workspace:
    problem: object
    config: object
    workspace: torch.Tensor
    schedule: torch.Tensor
    fwd_ctx: torch.Tensor | None


def get_workspace(T, H, I, E, topk, dtype=MOK_BF16, device="cuda", training=True, **cfg):
    """Allocate the workspace, schedule and fwd_ctx buffers for one layer shape."""
    problem = make_problem(T, H, I, E, topk, dtype)
    config = make_config(**cfg)
    ws, sb, cb = buffer_sizes(problem, config)
    mk = lambda n: torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)  # noqa: E731
    return Workspace(problem, config, mk(ws), mk(sb), mk(cb) if (training and cb) else None)


def run_schedule(w: Workspace, topk_ids):
    build_schedule(w.problem, topk_ids, w.schedule, w.config)


def run_forward(w: Workspace, x, topk_w, weights, y=None):
    if y is None:
        y = torch.empty_like(x)
    forward(w.problem, w.schedule, x, topk_w, weights, y, w.workspace, w.fwd_ctx, w.config)
    return y


def run_forward_fused(w: Workspace, topk_ids, x, topk_w, weights, y=None):
    """Schedule + forward in one persistent launch (mok_forward_fused)."""
    if y is None:
        y = torch.empty_like(x)
    forward_fused(w.problem, topk_ids, w.schedule, x, topk_w, weights, y, w.workspace, w.fwd_ctx, w.config)
    return y


def run_backward(w: Workspace, x, topk_w, weights, dy):
    wg, wu, wd = weights[:3]
    dx = torch.empty_like(x)
    dwg, dwu, dwd = torch.empty_like(wg), torch.empty_like(wu), torch.empty_like(wd)
    dtw = torch.empty_like(topk_w)
    backward(w.problem, w.schedule, w.fwd_ctx, x, topk_w, weights, dy, dx, dwg, dwu, dwd, dtw,
             w.workspace, w.config)
    return dx, dwg, dwu, dwd, dtw


def quantize_weights_backward(wg, wu, wd):
    """The MXFP8 weight copies the MXFP8 backward needs, quantized along the
    weights' other axis by the library's transposing quantizer: Wd^T
    [E][I][H] blocked along H, and [Wg; Wu]^T [E][H][2I] blocked along 2I
    (Wg into columns [0, I), Wu into [I, 2I)).
    Returns (w_down_t, w_gu_t, s_down_t, s_gu_t)."""
    E, I, H = wg.shape
    dev = wg.device
    qd = torch.empty((E, I, H), dtype=torch.uint8, device=dev)
    sd = torch.empty((E, I, H // 32), dtype=torch.uint8, device=dev)
    qgu = torch.empty((E, H, 2 * I), dtype=torch.uint8, device=dev)
    sgu = torch.empty((E, H, 2 * I // 32), dtype=torch.uint8, device=dev)
    mxfp8_quantize_transposed(wd, qd, sd)
    mxfp8_quantize_transposed(wg, qgu, sgu, col0=0)
    mxfp8_quantize_transposed(wu, qgu, sgu, col0=I)
    return qd, qgu, sd, sgu


def quantize_weights(wg, wu, wd):
    """MXFP8 copies of the expert weights along their contraction axes."""
    out = []
    for m in (wg, wu, wd):
        q = torch.empty(m.shape, dtype=torch.uint8, device=m.device)
        s = torch.empty(m.shape[:-1] + (m.shape[-1] // 32,), dtype=torch.uint8, device=m.device)
        mxfp8_quantize(m.reshape(-1, m.shape[-1]), q, s)
        out.append((q, s))
    (qg, sg), (qu, su), (qd, sd) = out
    return qg, qu, qd, sg, su, sd


def read_schedule(w: Workspace):
    """Copy the schedule arrays to the host (for inspection and tests)."""
    L = schedule_layout(w.problem, w.config)
    s = w.schedule.cpu()
    E, R = w.problem.E, w.problem.T * w.problem.topk

    def arr(off, n):
        return s[off:off + 4 * n].view(torch.int32).numpy().copy()

    nf = int(arr(L.n_fwd_tiles, 1)[0])
    nb = int(arr(L.n_bwd_tiles, 1)[0])
    return {
        "status": int(arr(L.status, 1)[0]),
        "counts": arr(L.counts, E),
        "offsets": arr(L.offsets, E + 1),
        "perm": arr(L.perm, R),
        "dest": arr(L.dest, R),
        "fwd_tiles": arr(L.fwd_tiles, 4 * nf).reshape(nf, 4),
        "mb_tile_start": arr(L.mb_tile_start, L.n_minibatches + 1),
        "bwd_tiles": arr(L.bwd_tiles, 4 * nb).reshape(nb, 4),
        "expert_order": arr(L.expert_order, E),
        "M": L.minibatch_rows, "n_slots": L.ring_slots, "n_mb": L.n_minibatches,
        "fwd_tile_rows": L.fwd_tile_rows, "bwd_tile_rows": L.bwd_tile_rows,
    }
