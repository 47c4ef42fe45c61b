"""Python binding of libmok, a deterministic MoE layer for AMD MI355X (gfx950).

The binding only marshals arguments: every step of the layer runs in the HIP
kernels of libmok.so (see include/mok.h for the contract of each call). PyTorch
supplies device memory and the current stream. There is no fallback: if the
library is missing or fails to load, importing the calls raises.
"""
from __future__ import annotations

import ctypes
import os

__version__ = "0.1.0"

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmok.so")

MOK_OK = 0
MOK_ERR_INVALID_ARG = -1
MOK_ERR_UNSUPPORTED = -2
MOK_ERR_BUFFER_TOO_SMALL = -3
MOK_ERR_DEVICE = -4
MOK_BF16 = 0
MOK_MXFP8 = 1
STATUS_BAD_EXPERT_ID = 0x1
STATUS_WATCHDOG = 0x2


class MokError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("E", ctypes.c_int32), ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Config(ctypes.Structure):
    _fields_ = [("minibatch_rows", ctypes.c_int32), ("ring_slots", ctypes.c_int32),
                ("capacity_multiplier", ctypes.c_float), ("num_cus", ctypes.c_int32),
                ("driver", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("w_down_t", ctypes.c_void_p), ("w_gu_t", ctypes.c_void_p),
                ("s_down_t", ctypes.c_void_p), ("s_gu_t", ctypes.c_void_p)]


class ScheduleLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "status", "counts", "offsets", "perm", "dest", "n_fwd_tiles", "fwd_tiles",
        "mb_tile_start", "n_bwd_tiles", "bwd_tiles", "total")] + [
        (n, ctypes.c_int32) for n in (
            "minibatch_rows", "ring_slots", "n_minibatches", "max_fwd_tiles", "max_bwd_tiles",
            "fwd_tile_rows", "bwd_tile_rows")] + [("arrays", ctypes.c_size_t), ("expert_order", ctypes.c_size_t)]


_lib = None

EXPORTS = ("mok_version", "mok_status_string", "mok_buffer_sizes", "mok_get_schedule_layout",
           "mok_build_schedule", "mok_forward", "mok_backward", "mok_mxfp8_quantize",
           "mok_router_forward", "mok_router_backward", "mok_trace_enable", "mok_trace_collect",
           "mok_mxfp8_quantize_transposed", "mok_probe_mfma", "mok_build_schedule_noalloc",
           "mok_forward_fused")


class TraceStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 40), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("max_ms", ctypes.c_double)]


def lib():
    """The loaded libmok.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmok.so not found at {LIB_PATH}; build it with "
                              "`python -m mixture_experts_layer_30_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.mok_version.restype = ctypes.c_int32
        L.mok_version.argtypes = []
        L.mok_status_string.restype = ctypes.c_char_p
        L.mok_status_string.argtypes = [ctypes.c_int32]
        L.mok_buffer_sizes.restype = ctypes.c_int
        L.mok_buffer_sizes.argtypes = [P(Problem), P(Config), P(sz), P(sz), P(sz)]
        L.mok_get_schedule_layout.restype = ctypes.c_int
        L.mok_get_schedule_layout.argtypes = [P(Problem), P(Config), P(ScheduleLayout)]
        L.mok_build_schedule.restype = ctypes.c_int
        L.mok_build_schedule.argtypes = [P(Problem), P(Config), vp, vp, sz, vp]
        L.mok_build_schedule_noalloc.restype = ctypes.c_int
        L.mok_build_schedule_noalloc.argtypes = [P(Problem), P(Config), vp, vp, sz, vp]
        L.mok_forward.restype = ctypes.c_int
        L.mok_forward.argtypes = [P(Problem), P(Config), vp, vp, vp, P(Weights), vp, vp, vp, sz, vp]
        L.mok_forward_fused.restype = ctypes.c_int
        L.mok_forward_fused.argtypes = [P(Problem), P(Config), vp, vp, sz, vp, vp, P(Weights), vp, vp,
                                        vp, sz, vp]
        L.mok_backward.restype = ctypes.c_int
        L.mok_backward.argtypes = [P(Problem), P(Config), vp, vp, vp, vp, P(Weights), vp, vp,
                                   vp, vp, vp, vp, vp, sz, vp]
        L.mok_mxfp8_quantize.restype = ctypes.c_int
        L.mok_mxfp8_quantize.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, vp, vp]
        L.mok_mxfp8_quantize_transposed.restype = ctypes.c_int
        L.mok_mxfp8_quantize_transposed.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp, vp,
                                                     ctypes.c_int64, ctypes.c_int64, vp]
        L.mok_probe_mfma.restype = ctypes.c_int
        L.mok_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]
        L.mok_router_forward.restype = ctypes.c_int
        L.mok_router_forward.argtypes = [P(Problem), vp, vp, vp, vp, vp, vp]
        L.mok_router_backward.restype = ctypes.c_int
        L.mok_router_backward.argtypes = [P(Problem), P(Config), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.mok_trace_enable.restype = ctypes.c_int
        L.mok_trace_enable.argtypes = [ctypes.c_int32]
        L.mok_trace_collect.restype = ctypes.c_int
        L.mok_trace_collect.argtypes = [P(TraceStat), ctypes.c_int32, P(ctypes.c_int32)]
        _lib = L
    return _lib


def version() -> int:
    return int(lib().mok_version())


def status_string(status: int) -> str:
    return lib().mok_status_string(int(status)).decode()


def _check(status, what):
    if status != MOK_OK:
        raise MokError(status, what)


def make_problem(T, H, I, E, topk, dtype=MOK_BF16) -> Problem:
    return Problem(int(T), int(H), int(I), int(E), int(topk), int(dtype))


def make_config(minibatch_rows=0, ring_slots=0, capacity_multiplier=0.0, num_cus=0, driver=0):
    return Config(int(minibatch_rows), int(ring_slots), float(capacity_multiplier), int(num_cus),
                  int(driver))


def _cfg(config):
    return ctypes.byref(config) if config is not None else None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def buffer_sizes(problem, config=None):
    """(workspace_bytes, schedule_bytes, fwd_ctx_bytes); host only."""
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().mok_buffer_sizes(ctypes.byref(problem), _cfg(config), ctypes.byref(a),
                                  ctypes.byref(b), ctypes.byref(c)), "mok_buffer_sizes")
    return a.value, b.value, c.value


def schedule_layout(problem, config=None) -> ScheduleLayout:
    out = ScheduleLayout()
    _check(lib().mok_get_schedule_layout(ctypes.byref(problem), _cfg(config), ctypes.byref(out)),
           "mok_get_schedule_layout")
    return out


def build_schedule(problem, topk_ids, schedule, config=None, stream=None):
    _check(lib().mok_build_schedule(ctypes.byref(problem), _cfg(config), _ptr(topk_ids),
                                    _ptr(schedule), schedule.numel() * schedule.element_size(),
                                    _stream(stream)), "mok_build_schedule")


def build_schedule_noalloc(problem, topk_ids, schedule, config=None, stream=None):
    """mok_build_schedule with the build's scratch in the library's static
    device array (schedule needs only schedule_layout(...).arrays bytes)."""
    _check(lib().mok_build_schedule_noalloc(ctypes.byref(problem), _cfg(config), _ptr(topk_ids),
                                            _ptr(schedule), schedule.numel() * schedule.element_size(),
                                            _stream(stream)), "mok_build_schedule_noalloc")


def _weights(w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None, w_down_t=None, w_gu_t=None,
             s_down_t=None, s_gu_t=None):
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    return Weights(w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr(), p(s_gate), p(s_up), p(s_down),
                   p(w_down_t), p(w_gu_t), p(s_down_t), p(s_gu_t))


def forward(problem, schedule, x, topk_w, weights, y, workspace, fwd_ctx=None, config=None,
            stream=None):
    """weights: (w_gate, w_up, w_down[, s_gate, s_up, s_down[, w_down_t, w_gu_t, s_down_t,
    s_gu_t]]) tensors (the last four only matter to the MXFP8 backward)."""
    w = _weights(*weights)
    _check(lib().mok_forward(ctypes.byref(problem), _cfg(config), _ptr(schedule), _ptr(x),
                             _ptr(topk_w), ctypes.byref(w), _ptr(y), _ptr(fwd_ctx),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream)), "mok_forward")


def forward_fused(problem, topk_ids, schedule, x, topk_w, weights, y, workspace, fwd_ctx=None,
                  config=None, stream=None):
    """mok_forward_fused: the schedule from topk_ids and the forward, in one
    persistent launch (weights as for forward)."""
    w = _weights(*weights)
    _check(lib().mok_forward_fused(ctypes.byref(problem), _cfg(config), _ptr(topk_ids), _ptr(schedule),
                                   schedule.numel() * schedule.element_size(), _ptr(x), _ptr(topk_w),
                                   ctypes.byref(w), _ptr(y), _ptr(fwd_ctx), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "mok_forward_fused")


def backward(problem, schedule, fwd_ctx, x, topk_w, weights, dy, dx, dw_gate, dw_up, dw_down,
             d_topk_w, workspace, config=None, stream=None):
    w = _weights(*weights)
    _check(lib().mok_backward(ctypes.byref(problem), _cfg(config), _ptr(schedule), _ptr(fwd_ctx),
                              _ptr(x), _ptr(topk_w), ctypes.byref(w), _ptr(dy), _ptr(dx),
                              _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(d_topk_w),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)), "mok_backward")


def mxfp8_quantize(src, q, scales, stream=None):
    """src [rows][K] bf16 -> q [rows][K] uint8 (E4M3), scales [rows][K/32] uint8 (E8M0)."""
    rows, K = src.shape[0], src.shape[-1]
    _check(lib().mok_mxfp8_quantize(_ptr(src), int(rows) if src.dim() == 2 else int(src.numel() // K),
                                    int(K), _ptr(q), _ptr(scales), _stream(stream)),
           "mok_mxfp8_quantize")


def mxfp8_quantize_transposed(src, q, scales, col0=0, stream=None):
    """src [batch][rows][cols] (or [rows][cols]) bf16 -> q[b][c][col0 + r] (E4M3) and
    scales[b][c][(col0 + r) / 32] (E8M0), blocked by 32 along the source rows; q is
    [batch][cols][ld] uint8 and scales [batch][cols][ld/32] uint8 (ld = q.shape[-1])."""
    rows, cols, ld = src.shape[-2], src.shape[-1], q.shape[-1]
    batch = int(src.numel() // (rows * cols)) if rows * cols else 0
    _check(lib().mok_mxfp8_quantize_transposed(_ptr(src), batch, int(rows), int(cols), _ptr(q), _ptr(scales),
                                               int(ld), int(col0), _stream(stream)),
           "mok_mxfp8_quantize_transposed")


def probe_mfma(kind, workgroups, iters, sink, stream=None):
    """Enqueue the matrix-core peak probe (kind 0 bf16, 1 MXFP8); sink holds
    workgroups * 256 float32. Returns the FLOPs it performs."""
    _check(lib().mok_probe_mfma(int(kind), int(workgroups), int(iters), _ptr(sink), _stream(stream)),
           "mok_probe_mfma")
    return float(workgroups) * 4 * 8 * iters * (32768 if kind == 0 else 131072)


def router_forward(problem, x, w_router, bias, topk_ids, topk_w, stream=None):
    """x [T][H] bf16, w_router [E][H] fp32, bias [E] fp32 or None -> topk_ids [T][k] int32,
    topk_w [T][k] fp32 (overwritten)."""
    _check(lib().mok_router_forward(ctypes.byref(problem), _ptr(x), _ptr(w_router), _ptr(bias),
                                    _ptr(topk_ids), _ptr(topk_w), _stream(stream)), "mok_router_forward")


def router_backward(problem, schedule, x, w_router, topk_ids, topk_w, d_topk_w, d_sel, dx, d_w_router,
                    config=None, stream=None):
    """-> d_sel [T][k] fp32, dx [T][H] bf16, d_w_router [E][H] fp32 (overwritten); schedule built
    by build_schedule for these topk_ids."""
    _check(lib().mok_router_backward(ctypes.byref(problem), _cfg(config), _ptr(schedule), _ptr(x),
                                     _ptr(w_router), _ptr(topk_ids), _ptr(topk_w), _ptr(d_topk_w),
                                     _ptr(d_sel), _ptr(dx), _ptr(d_w_router), _stream(stream)),
           "mok_router_backward")


def trace_enable(on=True):
    _check(lib().mok_trace_enable(1 if on else 0), "mok_trace_enable")


def trace_collect():
    """{kernel name: (launches, total_ms, max_ms)}; waits for the traced work."""
    n = ctypes.c_int32()
    buf = (TraceStat * 64)()
    _check(lib().mok_trace_collect(buf, 64, ctypes.byref(n)), "mok_trace_collect")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms, buf[i].max_ms)
            for i in range(min(n.value, 64))}
