"""Python binding of libmoe_mi355x.so: one GPU's share of a Mixture-of-Experts
layer (top-k router, dispatch, grouped Linear-1 + SwiGLU, grouped Linear-2,
weighted combine) as hand-written HIP kernels for MI355X (gfx950).

The functions here only marshal arguments: torch tensors (device memory) and
torch's current HIP stream go to the C ABI declared in include/moe_mi355x.h,
under the same names without the `moe_` prefix. Every step of the layer runs
in the library's kernels; there is no fallback. If the library is missing the
import fails with an error naming the build command.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

__all__ = [
    "MoEError", "Problem", "WorkspaceLayout", "lib", "make_problem", "workspace_size", "workspace_layout",
    "workspace_views", "route_topk", "dispatch", "dispatch_noalloc", "expert_forward", "combine", "layer_forward",
    "check_workspace", "tile_trace", "schedule_of", "store_burst_probe", "owner_plan", "owner_gather",
    "segment_copy", "expert_forward_signal", "segment_copy_wait", "SCHED", "DTYPE", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE_TOO_SMALL",
          4: "MOE_ERR_HIP", 5: "MOE_ERR_DEADLOCK"}
SCHED = {"expert_wave": 0, "interleaved": 1, "separate": 2, "auto": 3}
DTYPE = {"bf16": 0, "fp8_e4m3": 1, "w4a8_mxfp4": 2}
# MOE_FLAG_* of moe_mi355x.h
FLAG_FP32_Y_DEBUG = 1 << 0
FLAG_BF16_COMBINE_BUF = 1 << 1
TILE_FLAGS = {"auto": 0, "narrow": 1 << 2, "wide": 1 << 3}
FLAG_BAND_MAJOR = 1 << 4
FLAG_TILE_TRACE = 1 << 5
FLAG_KEEP_H_F32 = 1 << 6
FLAG_TEST_WAIT_TIMEOUT = 1 << 7


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)}"
        if status == 4:
            msg += f" (hipError {lib().moe_last_hip_error()})"
        super().__init__(msg)


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "d", "f", "E_global", "k", "e_begin", "e_end", "dtype", "quant_block", "num_segments", "sched",
        "lead_D", "wave_experts", "grid")] + [("flags", ctypes.c_uint32), ("row_capacity", ctypes.c_int32)]

    def __repr__(self):
        return "Problem(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "topk_idx", "topk_w", "counts", "offsets", "row_src", "row_dst", "tok_off", "comb_w", "x_perm",
        "x_perm_scale", "h", "h_scale", "h_f32", "combine_buf", "meta", "tile_trace", "tile_trace_capacity",
        "total")]


class OwnerPlanSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("R", "bands", "remote_bands", "segments", "recv_rows")]


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m expert_grouped_gemm_amd.build` "
                              f"(hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        PP = ctypes.POINTER(Problem)
        L.moe_workspace_size.restype = ctypes.c_size_t
        L.moe_workspace_size.argtypes = [PP]
        L.moe_workspace_get_layout.restype = ctypes.c_int
        L.moe_workspace_get_layout.argtypes = [PP, ctypes.POINTER(WorkspaceLayout)]
        L.moe_route_topk.restype = ctypes.c_int
        L.moe_route_topk.argtypes = [PP, _P, _P, _P, _P, _P]
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [PP] + [_P] * 13 + [ctypes.c_size_t, _P]
        L.moe_dispatch_noalloc.restype = ctypes.c_int
        L.moe_dispatch_noalloc.argtypes = [PP] + [_P] * 13
        L.moe_expert_forward.restype = ctypes.c_int
        L.moe_expert_forward.argtypes = [PP] + [_P] * 10 + [ctypes.c_size_t, _P]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [PP, _P, _P, _P, _P, _P, _P]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward.argtypes = [PP] + [_P] * 10 + [ctypes.c_size_t] + [_P] * 6
        L.moe_check_workspace.restype = ctypes.c_int
        L.moe_check_workspace.argtypes = [PP, _P, ctypes.c_size_t, _P]
        L.moe_store_burst_probe.restype = ctypes.c_int
        L.moe_store_burst_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, _P,
                                            ctypes.c_size_t, _P, ctypes.c_size_t, _P]
        L.moe_owner_plan.restype = ctypes.c_int
        L.moe_owner_plan.argtypes = [PP, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int64, _P, _P,
                                     _P, _P, ctypes.c_int64, _P, ctypes.POINTER(OwnerPlanSizes)]
        L.moe_owner_gather.restype = ctypes.c_int
        L.moe_owner_gather.argtypes = [PP, _P, _P, _P, ctypes.c_int64, _P, _P, _P]
        L.moe_segment_copy.restype = ctypes.c_int
        L.moe_segment_copy.argtypes = [PP, _P, ctypes.c_int64, _P, ctypes.c_int64, _P, ctypes.c_int64, _P]
        L.moe_expert_forward_signal.restype = ctypes.c_int
        L.moe_expert_forward_signal.argtypes = [PP] + [_P] * 10 + [ctypes.c_int64, _P, ctypes.c_size_t, _P]
        L.moe_segment_copy_wait.restype = ctypes.c_int
        L.moe_segment_copy_wait.argtypes = [PP, _P, ctypes.c_int64, _P, ctypes.c_int64, _P, ctypes.c_int64, _P,
                                            ctypes.c_int64, _P, ctypes.c_int, _P]
        L.moe_schedule_of.restype = ctypes.c_int
        L.moe_schedule_of.argtypes = [PP]
        L.moe_tile_clock_hz.restype = ctypes.c_double
        L.moe_tile_clock_hz.argtypes = []
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_last_hip_error.restype = ctypes.c_int
        L.moe_last_hip_error.argtypes = []
        L.moe_version.restype = ctypes.c_char_p
        L.moe_version.argtypes = []
        _lib = L
    return _lib


def make_problem(T: int, d: int, f: int, E_global: int, k: int, e_begin: int = 0, e_end: Optional[int] = None,
                 dtype: str = "bf16", num_segments: int = 1, sched: str = "interleaved", lead_D: int = 0,
                 wave_experts: int = 0, grid: int = 0, quant_block: int = 128, tiles: str = "auto",
                 band_major: bool = False, trace: bool = False, keep_h_f32: bool = False,
                 bf16_combine_buf: bool = False, fp32_y: bool = False, row_capacity: int = 0) -> Problem:
    """tiles: "auto" (chosen from the shape), "narrow" or "wide" expert-GEMM tiles;
    band_major: walk the separate / expert-wave tile lists band by band;
    trace: record one timed span per expert-GEMM tile (read with tile_trace);
    keep_h_f32: fp8, store every fp32 SwiGLU value in the workspace view h_f32;
    bf16_combine_buf: the combine buffer holds bf16 rows (MOE_FLAG_BF16_COMBINE_BUF);
    fp32_y: MOE_FLAG_FP32_Y_DEBUG (layer_forward then requires Y_fp32);
    row_capacity: rows the workspace holds for the expert GEMM (0: T * min(k, E_l))."""
    flags = (TILE_FLAGS[tiles] | (FLAG_BAND_MAJOR if band_major else 0) | (FLAG_TILE_TRACE if trace else 0)
             | (FLAG_KEEP_H_F32 if keep_h_f32 else 0) | (FLAG_BF16_COMBINE_BUF if bf16_combine_buf else 0)
             | (FLAG_FP32_Y_DEBUG if fp32_y else 0))
    return Problem(T=T, d=d, f=f, E_global=E_global, k=k, e_begin=e_begin,
                   e_end=E_global if e_end is None else e_end, dtype=DTYPE[dtype], quant_block=quant_block,
                   num_segments=num_segments, sched=SCHED[sched], lead_D=lead_D, wave_experts=wave_experts,
                   grid=grid, flags=flags, row_capacity=row_capacity)


def row_capacity(p: Problem) -> int:
    """Rows the workspace holds for the expert GEMM (the library's rule)."""
    El = p.e_end - p.e_begin
    return max(p.T * min(p.k, El), p.row_capacity)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, where: str):
    if status != 0:
        raise MoEError(status, where)


def workspace_size(p: Problem) -> int:
    n = lib().moe_workspace_size(ctypes.byref(p))
    if n == 0:
        raise MoEError(2, "moe_workspace_size")
    return n


def workspace_layout(p: Problem) -> WorkspaceLayout:
    out = WorkspaceLayout()
    _check(lib().moe_workspace_get_layout(ctypes.byref(p), ctypes.byref(out)), "moe_workspace_get_layout")
    return out


def alloc_workspace(p: Problem, device="cuda") -> torch.Tensor:
    return torch.empty(workspace_size(p), dtype=torch.uint8, device=device)


def workspace_views(p: Problem, ws: torch.Tensor) -> Dict[str, torch.Tensor]:
    """Typed views of the intermediates a moe_layer_forward call leaves in `ws`."""
    L = workspace_layout(p)
    El = p.e_end - p.e_begin
    cap = row_capacity(p)
    esz = 1 if p.dtype != DTYPE["bf16"] else 2   # e4m3 activations for fp8 and W4A8
    edt = torch.uint8 if esz == 1 else torch.bfloat16
    cb_dt = torch.bfloat16 if p.flags & FLAG_BF16_COMBINE_BUF else torch.float32

    def view(off, n, dt, shape):
        nbytes = n * torch.empty((), dtype=dt).element_size()
        return ws[off:off + nbytes].view(dt).view(shape)

    v = dict(
        topk_idx=view(L.topk_idx, p.T * p.k, torch.int32, (p.T, p.k)),
        topk_w=view(L.topk_w, p.T * p.k, torch.float32, (p.T, p.k)),
        counts=view(L.counts, El, torch.int32, (El,)),
        offsets=view(L.offsets, El + 1, torch.int32, (El + 1,)),
        row_src=view(L.row_src, cap, torch.int32, (cap,)),
        row_dst=view(L.row_dst, cap, torch.int32, (cap,)),
        tok_off=view(L.tok_off, p.T + 1, torch.int32, (p.T + 1,)),
        comb_w=view(L.comb_w, cap, torch.float32, (cap,)),
        x_perm=view(L.x_perm, cap * p.d, edt, (cap, p.d)),
        h=view(L.h, cap * p.f, edt, (cap, p.f)),
        combine_buf=view(L.combine_buf, cap * p.d, cb_dt, (cap, p.d)),
        meta=view(L.meta, 64, torch.int32, (64,)),
    )
    if esz == 1:
        v["x_perm_scale"] = view(L.x_perm_scale, cap * (p.d // 128), torch.float32, (p.d // 128, cap))
        v["h_scale"] = view(L.h_scale, cap * (p.f // 128), torch.float32, (p.f // 128, cap))
        v["h_f32"] = view(L.h_f32, cap * p.f, torch.float32, (cap, p.f))
    if L.tile_trace_capacity:
        v["tile_trace"] = view(L.tile_trace, L.tile_trace_capacity * 5, torch.int64, (L.tile_trace_capacity, 5))
    return v


def tile_trace(p: Problem, ws: torch.Tensor) -> Dict[str, "np.ndarray"]:
    """The expert-GEMM tile records of the last call on `ws` (a problem made with
    trace=True), decoded: clock readings t_start, t_ready, t_main_end, t_end in
    microseconds from the earliest start, and kind (1 = Linear-1, 2 = Linear-2),
    nnb (tile width in 32-row weight blocks per half), wg (workgroup), n (tile
    index in units of its width) and band (row band) per tile."""
    import numpy as np
    v = workspace_views(p, ws)
    if "tile_trace" not in v:
        raise ValueError("tile_trace: the problem was made without trace=True")
    count = int(v["meta"][4])
    cap = v["tile_trace"].shape[0]
    if count > cap:
        raise RuntimeError(f"tile_trace: {count} tile records for a region of {cap}")
    hz = lib().moe_tile_clock_hz()
    if hz <= 0:
        raise RuntimeError("tile_trace: the device does not report its wall-clock rate")
    r = v["tile_trace"][:count].cpu().numpy().view(np.uint64)
    t0 = int(r[:, 0].min()) if count else 0
    us = lambda c: (r[:, c].astype(np.int64) - t0) / hz * 1e6
    info = r[:, 4]
    return dict(t_start=us(0), t_ready=us(1), t_main_end=us(2), t_end=us(3),
                kind=(info & 3).astype(np.int64), nnb=((info >> 2) & 7).astype(np.int64),
                wg=((info >> 8) & 0xFFFF).astype(np.int64), n=((info >> 24) & 0xFFFF).astype(np.int64),
                band=(info >> 40).astype(np.int64))


def store_burst_probe(K: int, B: int, reps: int, gap_us: float, buf: torch.Tensor, rec: torch.Tensor,
                      stream=None):
    """moe_store_burst_probe: K producers, reps bursts of B bytes with gap_us
    between them, into `buf` (device bytes); clock readings into `rec`
    (device int64, at least 2*K*reps + 1 elements)."""
    _check(lib().moe_store_burst_probe(K, B, reps, gap_us, _ptr(buf), buf.numel() * buf.element_size(), _ptr(rec),
                                       rec.numel() * rec.element_size(), _stream(stream)),
           "moe_store_burst_probe")


def schedule_of(p: Problem) -> str:
    """The schedule `p` runs, with "auto" resolved."""
    code = lib().moe_schedule_of(ctypes.byref(p))
    names = {v: k for k, v in SCHED.items()}
    if code not in names:
        raise ValueError(f"schedule_of: invalid schedule {p.sched}")
    return names[code]


def route_topk(p: Problem, logits, topk_idx, topk_w, counts_global=None, stream=None):
    _check(lib().moe_route_topk(ctypes.byref(p), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(counts_global),
                                _stream(stream)), "moe_route_topk")


def dispatch(p: Problem, X, X_scale, topk_idx, topk_w, counts, offsets, row_src, row_dst, tok_off, comb_w,
             X_perm, X_perm_scale, workspace, stream=None):
    _check(lib().moe_dispatch(ctypes.byref(p), _ptr(X), _ptr(X_scale), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                              _ptr(offsets), _ptr(row_src), _ptr(row_dst), _ptr(tok_off), _ptr(comb_w),
                              _ptr(X_perm), _ptr(X_perm_scale), _ptr(workspace), workspace.numel(),
                              _stream(stream)), "moe_dispatch")


def dispatch_noalloc(p: Problem, X, X_scale, topk_idx, topk_w, counts, offsets, row_src, row_dst, tok_off, comb_w,
                     X_perm, X_perm_scale, stream=None):
    """moe_dispatch_noalloc: moe_dispatch with the library's own scratch
    array instead of a workspace (no allocation)."""
    _check(lib().moe_dispatch_noalloc(ctypes.byref(p), _ptr(X), _ptr(X_scale), _ptr(topk_idx), _ptr(topk_w),
                                      _ptr(counts), _ptr(offsets), _ptr(row_src), _ptr(row_dst), _ptr(tok_off),
                                      _ptr(comb_w), _ptr(X_perm), _ptr(X_perm_scale), _stream(stream)),
           "moe_dispatch_noalloc")


def expert_forward(p: Problem, X_perm, X_perm_scale, offsets, row_dst, W1, W1_scale, W2, W2_scale, combine_buf,
                   workspace, stream=None):
    _check(lib().moe_expert_forward(ctypes.byref(p), _ptr(X_perm), _ptr(X_perm_scale), _ptr(offsets),
                                    _ptr(row_dst), _ptr(W1), _ptr(W1_scale), _ptr(W2), _ptr(W2_scale),
                                    _ptr(combine_buf), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_expert_forward")


def combine(p: Problem, combine_buf, tok_off, comb_w, Y, Y_fp32=None, stream=None):
    _check(lib().moe_combine(ctypes.byref(p), _ptr(combine_buf), _ptr(tok_off), _ptr(comb_w), _ptr(Y), _ptr(Y_fp32),
                             _stream(stream)), "moe_combine")


def layer_forward(p: Problem, X, X_scale, logits, W1, W1_scale, W2, W2_scale, Y, Y_fp32, workspace, stream=None,
                  topk_idx=None, topk_w=None, counts=None, offsets=None, row_src=None):
    """moe_layer_forward. The optional outputs (device int32 / fp32 tensors of
    shapes [T, k], [T, k], [E_l], [E_l + 1], [row capacity]) receive the
    routing and dispatch results in place of their workspace regions."""
    El = p.e_end - p.e_begin
    for name, t, n in (("topk_idx", topk_idx, p.T * p.k), ("topk_w", topk_w, p.T * p.k), ("counts", counts, El),
                       ("offsets", offsets, El + 1), ("row_src", row_src, row_capacity(p))):
        if t is not None and t.numel() < n:
            raise ValueError(f"layer_forward: {name} holds {t.numel()} elements, needs {n}")
    _check(lib().moe_layer_forward(ctypes.byref(p), _ptr(X), _ptr(X_scale), _ptr(logits), _ptr(W1), _ptr(W1_scale),
                                   _ptr(W2), _ptr(W2_scale), _ptr(Y), _ptr(Y_fp32), _ptr(workspace),
                                   workspace.numel(), _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                                   _ptr(row_src), _stream(stream)), "moe_layer_forward")


def check_workspace(p: Problem, workspace, stream=None):
    _check(lib().moe_check_workspace(ctypes.byref(p), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_check_workspace")


def owner_plan(p: Problem, topk_idx, local_rank: int, tb_M: int, x_bands: int) -> Dict[str, "np.ndarray"]:
    """moe_owner_plan on host arrays: topk_idx int32 [T, k] (numpy or a CPU
    tensor). Returns row_src, expert_off, bands [n, 5], schedule, segments
    [n, 4], recv_start and the sizes, as numpy arrays / ints."""
    import numpy as np
    idx = np.ascontiguousarray(np.asarray(topk_idx, dtype=np.int32))
    if idx.shape != (p.T, p.k):
        raise ValueError(f"owner_plan: topk_idx shape {idx.shape}, expected {(p.T, p.k)}")
    z = OwnerPlanSizes()
    L = lib()
    _check(L.moe_owner_plan(ctypes.byref(p), idx.ctypes.data, local_rank, tb_M, x_bands, None, 0, None, None, None,
                            None, 0, None, ctypes.byref(z)), "moe_owner_plan")
    El = p.e_end - p.e_begin
    row_src = np.empty(max(1, z.R), np.int32)
    expert_off = np.empty(El + 1, np.int32)
    bands = np.empty((max(1, z.bands), 5), np.int32)
    sched = np.empty(max(1, z.bands), np.int32)
    segs = np.empty((max(1, z.bands), 4), np.int32)
    recv_start = np.empty(p.num_segments + 1, np.int32)
    _check(L.moe_owner_plan(ctypes.byref(p), idx.ctypes.data, local_rank, tb_M, x_bands, row_src.ctypes.data,
                            row_src.shape[0], expert_off.ctypes.data, bands.ctypes.data, sched.ctypes.data,
                            segs.ctypes.data, bands.shape[0], recv_start.ctypes.data, ctypes.byref(z)),
           "moe_owner_plan")
    return {"row_src": row_src[:z.R], "expert_off": expert_off, "bands": bands[:z.bands],
            "schedule": sched[:z.bands], "segments": segs[:z.segments], "recv_start": recv_start,
            "R": z.R, "n_bands": z.bands, "remote_bands": z.remote_bands, "n_segments": z.segments,
            "recv_rows": z.recv_rows}


def owner_gather(p: Problem, X, X_scale, row_src, X_pad, X_pad_scale=None, stream=None):
    """moe_owner_gather: X_pad[r] = X[row_src[r] // k] (zeros for -1); fp8
    also the row scales into X_pad_scale [d/128, row capacity]."""
    _check(lib().moe_owner_gather(ctypes.byref(p), _ptr(X), _ptr(X_scale), _ptr(row_src), row_src.numel(),
                                  _ptr(X_pad), _ptr(X_pad_scale), _stream(stream)), "moe_owner_gather")


def segment_copy(p: Problem, O_pad, segments, recv, stream=None):
    """moe_segment_copy: segments int32 [n, 4] on the device."""
    _check(lib().moe_segment_copy(ctypes.byref(p), _ptr(O_pad), O_pad.shape[0], _ptr(segments), segments.shape[0],
                                  _ptr(recv), recv.shape[0], _stream(stream)), "moe_segment_copy")


def expert_forward_signal(p: Problem, X_perm, X_perm_scale, offsets, row_dst, W1, W1_scale, W2, W2_scale,
                          combine_buf, row_done, workspace, stream=None):
    """moe_expert_forward_signal: also publishes stored Linear-2 elements per
    32-row block in row_done (device int32, zeroed by the caller)."""
    _check(lib().moe_expert_forward_signal(ctypes.byref(p), _ptr(X_perm), _ptr(X_perm_scale), _ptr(offsets),
                                           _ptr(row_dst), _ptr(W1), _ptr(W1_scale), _ptr(W2), _ptr(W2_scale),
                                           _ptr(combine_buf), _ptr(row_done), row_done.numel(), _ptr(workspace),
                                           workspace.numel(), _stream(stream)), "moe_expert_forward_signal")


def segment_copy_wait(p: Problem, O_pad, R: int, segments, recv, row_done, err, grid: int = 0, stream=None):
    """moe_segment_copy_wait: each segment waits for its rows in row_done. R is
    the layout's row count (the plan's expert_off[E_l]), which sets the last
    row block's target; O_pad must hold at least R rows."""
    if O_pad.shape[0] < R:
        raise ValueError(f"segment_copy_wait: O_pad holds {O_pad.shape[0]} rows, the layout has {R}")
    _check(lib().moe_segment_copy_wait(ctypes.byref(p), _ptr(O_pad), R, _ptr(segments),
                                       segments.shape[0], _ptr(recv), recv.shape[0], _ptr(row_done),
                                       row_done.numel(), _ptr(err), grid, _stream(stream)), "moe_segment_copy_wait")
