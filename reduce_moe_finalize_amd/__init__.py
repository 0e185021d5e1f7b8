"""Python binding of the fused post-experts boundary (MI355X / gfx950).

Thin ctypes layer over ``libfused_boundary.so`` (C ABI in
``include/fused_boundary.h``): it checks tensor dtypes, devices and shapes,
passes raw device pointers and torch's current HIP stream, and maps status codes
to exceptions.  Every step of the computation runs in the HIP kernel; there is
no CPU path.  If the library is not built, importing this package raises.

    normed, residual_out = fused_reduce_rmsnorm(partials, residual, gamma, eps=1e-6)
    normed, residual_out = fused_moe_finalize_rmsnorm(
        partials, expert_out, expanded_row_idx, topk_weights, residual, gamma,
        shared_out=shared, shared_gate_logits=None, eps=1e-6, weight_bias=0.0)
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

import torch  # loaded first: the library then binds to torch's HIP runtime

__all__ = [
    "LIB_PATH",
    "FusedBoundaryDeclined",
    "FusedBoundaryError",
    "fused_reduce_rmsnorm",
    "fused_moe_finalize_rmsnorm",
    "fused_moe_finalize_rmsnorm_noalloc",
    "NOALLOC_MAX_ROWS",
    "split_reduce_rmsnorm",
    "split_moe_finalize_rmsnorm",
    "split_sum",
    "split_residual_rmsnorm",
    "workspace_bytes",
    "get_plan",
    "plan_override",
    "wait_limit",
    "WAIT_NO_POLL",
    "force_decline",
    "workspace_status",
    "default_workspace",
    "default_workspace_status",
    "reset_default_workspaces",
    "status_string",
    "bandwidth_probe",
    "residency_probe",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfused_boundary.so")

FB_OK, FB_INVALID_ARGUMENT, FB_DECLINED, FB_HIP_ERROR, FB_TOO_MANY_ROWS = 0, 1, 2, 3, 4
NOALLOC_MAX_ROWS = 1024  # FB_NOALLOC_MAX_ROWS: row capacity of the allocation-free entry point
WAIT_NO_POLL = 0xFFFFFFFF  # wait_limit(): every split row gives up without polling
MAX_PARTIALS = 16
MAX_TOP_K = 16


class FusedBoundaryError(RuntimeError):
    """The library reported a HIP launch error."""


class FusedBoundaryDeclined(RuntimeError):
    """The fused kernel does not take this request (shape/alignment); outputs untouched."""


class Plan(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("vec_per_thread", ctypes.c_int32),
                ("split", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("sources_per_batch", ctypes.c_int32), ("workgroups_per_cu", ctypes.c_int32),
                ("units_per_wave", ctypes.c_int32), ("waves", ctypes.c_int32)]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m reduce_moe_finalize_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.fused_reduce_rmsnorm.argtypes = [ctypes.POINTER(vp), i32, vp, vp, f32, f32, i64, i64, vp, vp,
                                         vp, sz, vp]
    lib.fused_reduce_rmsnorm.restype = ctypes.c_int
    lib.fused_moe_finalize_rmsnorm.argtypes = [ctypes.POINTER(vp), i32, vp, i64, vp, vp, i32, vp, vp,
                                               vp, vp, f32, f32, i64, i64, vp, vp, vp, sz, vp]
    lib.fused_moe_finalize_rmsnorm.restype = ctypes.c_int
    lib.fused_moe_finalize_rmsnorm_noalloc.argtypes = [ctypes.POINTER(vp), i32, vp, i64, vp, vp, i32,
                                                       vp, vp, vp, vp, f32, f32, i64, i64, vp, vp, vp]
    lib.fused_moe_finalize_rmsnorm_noalloc.restype = ctypes.c_int
    lib.fused_boundary_workspace_bytes.argtypes = [i64, i64]
    lib.fused_boundary_workspace_bytes.restype = sz
    lib.fused_boundary_status_string.argtypes = [ctypes.c_int]
    lib.fused_boundary_status_string.restype = ctypes.c_char_p
    lib.fused_boundary_last_hip_error.argtypes = []
    lib.fused_boundary_last_hip_error.restype = ctypes.c_int
    lib.fused_boundary_get_plan.argtypes = [i64, i64, i32, i32, i32, sz, ctypes.POINTER(Plan)]
    lib.fused_boundary_get_plan.restype = ctypes.c_int
    lib.fused_boundary_set_plan_override.argtypes = [ctypes.POINTER(Plan)]
    lib.fused_boundary_set_plan_override.restype = ctypes.c_int
    lib.fused_boundary_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.fused_boundary_set_wait_limit.restype = None
    lib.fused_boundary_set_force_decline.argtypes = [ctypes.c_int]
    lib.fused_boundary_set_force_decline.restype = None
    lib.fused_boundary_split_sum.argtypes = [ctypes.POINTER(vp), i32, vp, i64, vp, vp, i32, vp, vp,
                                             i64, i64, vp, vp]
    lib.fused_boundary_split_sum.restype = ctypes.c_int
    lib.fused_boundary_split_residual_rmsnorm.argtypes = [vp, vp, vp, f32, f32, i64, i64, vp, vp, vp]
    lib.fused_boundary_split_residual_rmsnorm.restype = ctypes.c_int
    lib.fused_boundary_split_last_hip_error.argtypes = []
    lib.fused_boundary_split_last_hip_error.restype = ctypes.c_int
    lib.fused_boundary_bandwidth_probe.argtypes = [ctypes.POINTER(vp), i32, vp, i64, vp, i32,
                                                   ctypes.POINTER(vp), i32, i64, i64, i32, i32, vp]
    lib.fused_boundary_bandwidth_probe.restype = ctypes.c_int
    lib.fused_boundary_probe_last_hip_error.argtypes = []
    lib.fused_boundary_probe_last_hip_error.restype = ctypes.c_int
    lib.fused_boundary_residency_probe.argtypes = [i32, i32, i32, ctypes.c_uint64, vp, vp]
    lib.fused_boundary_residency_probe.restype = ctypes.c_int
    return lib


_lib = _load()


def status_string(code: int) -> str:
    return _lib.fused_boundary_status_string(int(code)).decode()


def _check(code: int, what: str):
    if code == FB_OK:
        return
    msg = f"{what}: {status_string(code)}"
    if code in (FB_INVALID_ARGUMENT, FB_TOO_MANY_ROWS):
        raise ValueError(msg)
    if code == FB_DECLINED:
        raise FusedBoundaryDeclined(msg)
    if code == FB_HIP_ERROR:
        raise FusedBoundaryError(f"{msg} (hipError {_lib.fused_boundary_last_hip_error()})")
    raise RuntimeError(msg)


def workspace_bytes(num_tokens: int, hidden: int) -> int:
    return int(_lib.fused_boundary_workspace_bytes(int(num_tokens), int(hidden)))


def get_plan(num_tokens: int, hidden: int, num_partials: int = 8, top_k: int = 0,
             has_shared: bool = False, workspace_bytes_: int = 0) -> dict:
    """Launch plan a call with these sizes would use (top_k=0: the reduce entry point)."""
    p = Plan()
    _check(_lib.fused_boundary_get_plan(int(num_tokens), int(hidden), int(num_partials),
                                        int(top_k), int(bool(has_shared)), int(workspace_bytes_),
                                        ctypes.byref(p)), "get_plan")
    return p.as_dict()


@contextlib.contextmanager
def plan_override(block: int, vec_per_thread: int = 1, sources_per_batch: int = 0,
                  workgroups_per_cu: int = 0, units_per_wave: int = 0):
    """Force the launch shape of calls made inside the block (this thread only).

    ``sources_per_batch=0`` selects the latency kernel (``vec_per_thread`` 1, rows
    split over ``ceil(H/8/block)`` workgroups); 1/2/4/8 the whole-row stream kernel,
    held to ``workgroups_per_cu`` resident workgroups per CU (0: no limit).
    ``units_per_wave`` > 0 selects the balanced kernel (512-element units dealt
    evenly over ``workgroups_per_cu`` (0 = 1) workgroups per CU, at most that many
    per wave); with ``sources_per_batch=2`` and ``units_per_wave=1``, its streamed
    form (one unit per wave, sources fetched two at a time).
    """
    p = Plan(int(block), int(vec_per_thread), 0, 0, int(sources_per_batch),
             int(workgroups_per_cu), int(units_per_wave), 0)
    _check(_lib.fused_boundary_set_plan_override(ctypes.byref(p)), "plan_override")
    try:
        yield
    finally:
        _lib.fused_boundary_set_plan_override(None)


@contextlib.contextmanager
def wait_limit(polls: int):
    """Test hook: split rows give up after ``polls`` polls inside the block (this
    thread); ``WAIT_NO_POLL`` makes every split row give up at once.  A row that
    gives up takes or recomputes its siblings' sums (same outputs) and sets
    status bit 0, which stays set until the workspace is zeroed again."""
    _lib.fused_boundary_set_wait_limit(int(polls))
    try:
        yield
    finally:
        _lib.fused_boundary_set_wait_limit(0)


@contextlib.contextmanager
def force_decline():
    """Test hook: the fused entry points decline every valid call inside the
    block (this thread), as a runtime decline would; ``on_decline`` then applies."""
    _lib.fused_boundary_set_force_decline(1)
    try:
        yield
    finally:
        _lib.fused_boundary_set_force_decline(0)


# Per (device, stream) zero-filled workspaces, grown on demand.  Calls on one
# stream are ordered, so one workspace per stream is race-free.  A workspace is
# 256 bytes plus 512 per token row (4 MiB at T = 8192).  A workspace that a
# larger one replaces is kept too, never freed: a HIP graph captured earlier
# still writes to it on every replay, and freed memory could by then belong to
# another tensor.  Growth at least doubles the size, so few are ever retired.
# Calls made while the stream is being captured into a graph never use this
# cache (see _resolve_workspace).
_workspaces: dict = {}
_retired_workspaces: list = []


def default_workspace(num_tokens: int, hidden: int, device=None) -> torch.Tensor:
    """The cached zero-filled workspace of the current stream, grown to fit.

    Must not be called while that stream is being captured: creating or growing
    the buffer queues a zero fill, which a capture would record and every replay
    would repeat.  To give a captured call split rows, create a workspace before
    capturing (``torch.zeros(workspace_bytes(T, H), dtype=torch.uint8)``) and
    pass it; one workspace per graph that may replay concurrently with others."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        capturing = torch.cuda.is_current_stream_capturing()
    if capturing:
        raise RuntimeError("default_workspace() while the stream is being captured; create the "
                           "workspace before capture and pass it explicitly")
    key = (dev.index, stream.cuda_stream)
    need = workspace_bytes(num_tokens, hidden)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        size = max(need, 4096) if ws is None else max(need, 2 * ws.numel())
        if ws is not None:
            _retired_workspaces.append((key, ws))
        ws = torch.zeros(size, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _resolve_workspace(workspace, T: int, H: int, dev):
    """workspace="auto": the cached per-stream buffer, except during graph
    capture, where the call runs whole rows (no workspace).  A captured graph
    then holds exactly one kernel node per call, carries no zero fill into its
    replays and shares no state with other graphs or streams."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 tensor")
        with torch.cuda.device(dev):
            if torch.cuda.is_current_stream_capturing():
                return None
            return default_workspace(T, H, dev)
    return workspace


def _all_default_workspaces():
    return list(_workspaces.items()) + _retired_workspaces


def reset_default_workspaces() -> None:
    """Zero-fill every "auto" workspace, the retired ones included (each on
    the stream it serves).

    Clears the status words after a split row's bounded wait timed out (bit 0
    of :func:`workspace_status`; the outputs were correct all the same, and
    later calls exchange normally whether or not this is called).  A workspace
    the caller passes is the caller's to zero."""
    for (dev_index, handle), ws in _all_default_workspaces():
        dev = torch.device("cuda", dev_index)
        with torch.cuda.device(dev), torch.cuda.stream(torch.cuda.ExternalStream(handle, device=dev)):
            ws.zero_()  # ordered after the calls already queued on that stream


def workspace_status(ws: torch.Tensor) -> int:
    """Status word of a workspace (bit 0: a split row's wait timed out).  Waits
    for all work on the workspace's device first, whichever stream it was
    queued on."""
    torch.cuda.synchronize(ws.device)
    return int(ws[:4].view(torch.int32).item())


def default_workspace_status() -> int:
    """OR of the status words of every "auto" workspace, the retired ones
    included. Synchronises."""
    st = 0
    for _, ws in _all_default_workspaces():
        st |= workspace_status(ws)
    return st


def _bf16_2d(t: torch.Tensor, name: str, T: int, H: int, dev):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if tuple(t.shape) != (T, H):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(T, H)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _prepare(partials, residual, gamma, out, residual_out, workspace):
    if not isinstance(residual, torch.Tensor):
        raise ValueError("a residual tensor is required")
    if residual.dim() != 2:
        raise ValueError("residual must be [num_tokens, hidden]")
    dev = residual.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP (cuda) device; there is no CPU path")
    T, H = residual.shape
    _bf16_2d(residual, "residual", T, H, dev)
    for i, p in enumerate(partials):
        _bf16_2d(p, f"partials[{i}]", T, H, dev)
    if not isinstance(gamma, torch.Tensor) or gamma.dtype != torch.bfloat16 \
            or tuple(gamma.shape) != (H,) or gamma.device != dev or not gamma.is_contiguous():
        raise ValueError(f"gamma must be a contiguous bfloat16 [{H}] tensor on {dev}")
    if out is None:
        out = torch.empty_like(residual)
    _bf16_2d(out, "out", T, H, dev)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _bf16_2d(residual_out, "residual_out", T, H, dev)
    workspace = _resolve_workspace(workspace, T, H, dev)
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the same device")
    arr = (ctypes.c_void_p * max(1, len(partials)))(*[p.data_ptr() for p in partials])
    ws_ptr = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    return T, H, out, residual_out, arr, ws_ptr, ws_bytes, stream


def fused_reduce_rmsnorm(partials: Sequence[torch.Tensor], residual: torch.Tensor,
                         gamma: torch.Tensor, eps: float = 1e-6, weight_bias: float = 0.0, *,
                         out: Optional[torch.Tensor] = None,
                         residual_out: Optional[torch.Tensor] = None,
                         workspace="auto", on_decline: str = "raise"):
    """Sum of R partial buffers + residual, then RMSNorm scaled by (gamma + weight_bias).

    Returns ``(normed, residual_out)``.  ``residual_out`` may be ``residual``
    itself (in place).  ``workspace``: "auto" (a cached per-stream buffer that
    lets small-T calls split rows; whole rows while the stream is being captured
    into a graph), None (one workgroup per row), or a zero-initialised uint8
    tensor of at least ``workspace_bytes(T, H)``.
    ``on_decline``: "raise" (FusedBoundaryDeclined) or "split" (run the two-launch
    split flow instead, which takes any H and 2-byte alignment).
    """
    partials = list(partials)
    if not 1 <= len(partials) <= MAX_PARTIALS:
        raise ValueError(f"need 1..{MAX_PARTIALS} partial buffers, got {len(partials)}")
    T, H, out, residual_out, arr, ws, wsb, stream = _prepare(partials, residual, gamma, out,
                                                             residual_out, workspace)
    with torch.cuda.device(residual.device):  # launch on the tensors' device
        code = _lib.fused_reduce_rmsnorm(arr, len(partials), _ptr(residual), _ptr(gamma),
                                         float(weight_bias), float(eps), T, H, _ptr(out),
                                         _ptr(residual_out), ws, wsb, stream)
    if code == FB_DECLINED and on_decline == "split":
        return split_reduce_rmsnorm(partials, residual, gamma, eps=eps, weight_bias=weight_bias,
                                    out=out, residual_out=residual_out)
    _check(code, "fused_reduce_rmsnorm")
    return out, residual_out


def fused_moe_finalize_rmsnorm(partials: Sequence[torch.Tensor], expert_out: Optional[torch.Tensor],
                               expanded_row_idx: torch.Tensor, topk_weights: torch.Tensor,
                               residual: torch.Tensor, gamma: torch.Tensor, *,
                               shared_out: Optional[torch.Tensor] = None,
                               shared_gate_logits: Optional[torch.Tensor] = None,
                               eps: float = 1e-6, weight_bias: float = 0.0,
                               out: Optional[torch.Tensor] = None,
                               residual_out: Optional[torch.Tensor] = None,
                               workspace="auto", on_decline: str = "raise"):
    """Partials + MoE finalize (+ shared expert, optionally sigmoid-gated) + residual + RMSNorm.

    ``expert_out`` bf16 [N, H]; ``expanded_row_idx`` int32 [T, K] (row of
    expert_out per token slot; out of range = skipped); ``topk_weights`` fp32
    [T, K]; ``shared_out`` bf16 [T, H] or None; ``shared_gate_logits`` fp32 [T]
    or None.  Returns ``(normed, residual_out)``.  ``on_decline`` as in
    :func:`fused_reduce_rmsnorm`.
    """
    partials = list(partials)
    if len(partials) > MAX_PARTIALS:
        raise ValueError(f"at most {MAX_PARTIALS} partial buffers")
    T, H, out, residual_out, arr, ws, wsb, stream = _prepare(partials, residual, gamma, out,
                                                             residual_out, workspace)
    dev = residual.device
    K, N = _check_routing(expanded_row_idx, topk_weights, expert_out, shared_out,
                          shared_gate_logits, T, H, dev)
    with torch.cuda.device(dev):  # launch on the tensors' device
        code = _lib.fused_moe_finalize_rmsnorm(
            arr, len(partials), _ptr(expert_out), N, _ptr(expanded_row_idx), _ptr(topk_weights),
            K, _ptr(shared_out), _ptr(shared_gate_logits), _ptr(residual), _ptr(gamma),
            float(weight_bias), float(eps), T, H, _ptr(out), _ptr(residual_out), ws, wsb, stream)
    if code == FB_DECLINED and on_decline == "split":
        return split_moe_finalize_rmsnorm(
            partials, expert_out, expanded_row_idx, topk_weights, residual, gamma,
            shared_out=shared_out, shared_gate_logits=shared_gate_logits, eps=eps,
            weight_bias=weight_bias, out=out, residual_out=residual_out)
    _check(code, "fused_moe_finalize_rmsnorm")
    return out, residual_out


def fused_moe_finalize_rmsnorm_noalloc(partials: Sequence[torch.Tensor],
                                       expert_out: Optional[torch.Tensor],
                                       expanded_row_idx: Optional[torch.Tensor],
                                       topk_weights: Optional[torch.Tensor],
                                       residual: torch.Tensor, gamma: torch.Tensor, *,
                                       shared_out: Optional[torch.Tensor] = None,
                                       shared_gate_logits: Optional[torch.Tensor] = None,
                                       eps: float = 1e-6, weight_bias: float = 0.0,
                                       out: torch.Tensor, residual_out: torch.Tensor):
    """The allocation-free entry point: no workspace, split rows exchange through
    the library's static per-GPU scratch (T <= NOALLOC_MAX_ROWS).  Outputs are
    required (nothing is allocated here either).  ``expanded_row_idx=None`` is a
    call without the MoE finalize (top_k 0: the reduce entry point's call).
    Calls that may overlap on one GPU must not be made (they share the scratch).
    Returns ``(out, residual_out)``."""
    partials = list(partials)
    if len(partials) > MAX_PARTIALS:
        raise ValueError(f"at most {MAX_PARTIALS} partial buffers")
    if out is None or residual_out is None:
        raise ValueError("out and residual_out are required (this entry point allocates nothing)")
    T, H, out, residual_out, arr, _, _, stream = _prepare(partials, residual, gamma, out,
                                                          residual_out, None)
    dev = residual.device
    K, N = 0, 0
    if expanded_row_idx is not None:
        K, N = _check_routing(expanded_row_idx, topk_weights, expert_out, shared_out,
                              shared_gate_logits, T, H, dev)
    elif not partials:
        raise ValueError("a call without the MoE finalize needs at least one partial buffer")
    elif shared_out is not None or shared_gate_logits is not None:
        raise ValueError("shared_out needs the MoE finalize (expanded_row_idx, topk_weights)")
    with torch.cuda.device(dev):
        code = _lib.fused_moe_finalize_rmsnorm_noalloc(
            arr, len(partials), _ptr(expert_out) if K else None, N,
            _ptr(expanded_row_idx) if K else None, _ptr(topk_weights) if K else None, K,
            _ptr(shared_out) if K else None, _ptr(shared_gate_logits) if K else None,
            _ptr(residual), _ptr(gamma), float(weight_bias), float(eps), T, H, _ptr(out),
            _ptr(residual_out), stream)
    _check(code, "fused_moe_finalize_rmsnorm_noalloc")
    return out, residual_out


def _check_routing(expanded_row_idx, topk_weights, expert_out, shared_out, shared_gate_logits,
                   T, H, dev):
    if expanded_row_idx.dtype != torch.int32 or expanded_row_idx.dim() != 2 \
            or expanded_row_idx.shape[0] != T or not expanded_row_idx.is_contiguous() \
            or expanded_row_idx.device != dev:
        raise ValueError("expanded_row_idx must be a contiguous int32 [T, K] tensor on the device")
    K = int(expanded_row_idx.shape[1])
    if not 1 <= K <= MAX_TOP_K:
        raise ValueError(f"top_k must be in 1..{MAX_TOP_K}")
    if topk_weights.dtype != torch.float32 or tuple(topk_weights.shape) != (T, K) \
            or not topk_weights.is_contiguous() or topk_weights.device != dev:
        raise ValueError("topk_weights must be a contiguous float32 [T, K] tensor on the device")
    N = 0
    if expert_out is not None:
        if expert_out.dtype != torch.bfloat16 or expert_out.dim() != 2 or expert_out.shape[1] != H \
                or not expert_out.is_contiguous() or expert_out.device != dev:
            raise ValueError("expert_out must be a contiguous bfloat16 [N, H] tensor on the device")
        N = int(expert_out.shape[0])
    if shared_out is not None:
        _bf16_2d(shared_out, "shared_out", T, H, dev)
    _check_gate(shared_gate_logits, T, dev)
    return K, N


def _check_gate(shared_gate_logits, T, dev):
    if shared_gate_logits is None:
        return
    if not isinstance(shared_gate_logits, torch.Tensor) or shared_gate_logits.dtype != torch.float32 \
            or tuple(shared_gate_logits.shape) != (T,) or not shared_gate_logits.is_contiguous() \
            or shared_gate_logits.device != dev:
        raise ValueError("shared_gate_logits must be a contiguous float32 [T] tensor on the device")


# ------------------------------------------------------------------ split flow
def split_sum(partials: Sequence[torch.Tensor], residual_like: torch.Tensor, *,
              expert_out=None, expanded_row_idx=None, topk_weights=None, shared_out=None,
              shared_gate_logits=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Stage 1 of the split flow: bf16(sum of partials + routed experts + shared), [T, H]."""
    partials = list(partials)
    dev = residual_like.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP (cuda) device; there is no CPU path")
    T, H = residual_like.shape
    for i, p in enumerate(partials):
        _bf16_2d(p, f"partials[{i}]", T, H, dev)
    K, N = 0, 0
    if expanded_row_idx is not None:
        K, N = _check_routing(expanded_row_idx, topk_weights, expert_out, shared_out,
                              shared_gate_logits, T, H, dev)
    elif shared_out is not None:
        _bf16_2d(shared_out, "shared_out", T, H, dev)
        _check_gate(shared_gate_logits, T, dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _bf16_2d(out, "out", T, H, dev)
    arr = (ctypes.c_void_p * max(1, len(partials)))(*[p.data_ptr() for p in partials])
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    with torch.cuda.device(dev):
        code = _lib.fused_boundary_split_sum(
            arr, len(partials), _ptr(expert_out), N, _ptr(expanded_row_idx), _ptr(topk_weights),
            K, _ptr(shared_out), _ptr(shared_gate_logits), T, H, _ptr(out), stream)
    if code == FB_HIP_ERROR:
        raise FusedBoundaryError(f"split_sum: hipError {_lib.fused_boundary_split_last_hip_error()}")
    _check(code, "split_sum")
    return out


def split_residual_rmsnorm(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor,
                           eps: float = 1e-6, weight_bias: float = 0.0, *,
                           out: Optional[torch.Tensor] = None,
                           residual_out: Optional[torch.Tensor] = None):
    """Stage 2 of the split flow: residual RMSNorm of a materialised [T, H] tensor."""
    dev = residual.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP (cuda) device; there is no CPU path")
    T, H = residual.shape
    _bf16_2d(x, "x", T, H, dev)
    _bf16_2d(residual, "residual", T, H, dev)
    if gamma.dtype != torch.bfloat16 or tuple(gamma.shape) != (H,) or gamma.device != dev \
            or not gamma.is_contiguous():
        raise ValueError(f"gamma must be a contiguous bfloat16 [{H}] tensor on {dev}")
    out = torch.empty_like(residual) if out is None else out
    residual_out = torch.empty_like(residual) if residual_out is None else residual_out
    _bf16_2d(out, "out", T, H, dev)
    _bf16_2d(residual_out, "residual_out", T, H, dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    with torch.cuda.device(dev):
        code = _lib.fused_boundary_split_residual_rmsnorm(
            _ptr(x), _ptr(residual), _ptr(gamma), float(weight_bias), float(eps), T, H, _ptr(out),
            _ptr(residual_out), stream)
    if code == FB_HIP_ERROR:
        raise FusedBoundaryError(
            f"split_residual_rmsnorm: hipError {_lib.fused_boundary_split_last_hip_error()}")
    _check(code, "split_residual_rmsnorm")
    return out, residual_out


def split_reduce_rmsnorm(partials, residual, gamma, eps=1e-6, weight_bias=0.0, *, out=None,
                         residual_out=None, sum_out=None):
    """The unfused flow: materialise bf16(sum of partials), then residual RMSNorm."""
    y = split_sum(partials, residual, out=sum_out)
    return split_residual_rmsnorm(y, residual, gamma, eps, weight_bias, out=out,
                                  residual_out=residual_out)


def split_moe_finalize_rmsnorm(partials, expert_out, expanded_row_idx, topk_weights, residual,
                               gamma, *, shared_out=None, shared_gate_logits=None, eps=1e-6,
                               weight_bias=0.0, out=None, residual_out=None, sum_out=None):
    """The unfused flow: materialise bf16(partials + MoE finalize + shared), then residual RMSNorm."""
    y = split_sum(partials, residual, expert_out=expert_out, expanded_row_idx=expanded_row_idx,
                  topk_weights=topk_weights, shared_out=shared_out,
                  shared_gate_logits=shared_gate_logits, out=sum_out)
    return split_residual_rmsnorm(y, residual, gamma, eps, weight_bias, out=out,
                                  residual_out=residual_out)


# ------------------------------------------------------------------ diagnostics
def bandwidth_probe(direct: Sequence[torch.Tensor], gathered: Optional[torch.Tensor] = None,
                    gather_idx: Optional[torch.Tensor] = None, outputs: Sequence[torch.Tensor] = (),
                    vec_per_thread: int = 4, workgroups_per_cu: int = 0) -> None:
    """Diagnostic: the boundary's loads (and optionally its two row stores)
    without its arithmetic, one launch on the current stream (see
    fused_boundary_bandwidth_probe).  ``direct``: bf16 [T, H] tensors read at
    each row's offset; ``gathered`` bf16 [N, H] read through ``gather_idx``
    (int32 [T, k]); ``outputs``: up to two bf16 [T, H] tensors it overwrites."""
    direct, outputs = list(direct), list(outputs)
    if not direct and not outputs:
        raise ValueError("bandwidth_probe: nothing to read or write")
    ref = direct[0] if direct else outputs[0]
    if not isinstance(ref, torch.Tensor) or ref.dim() != 2:
        raise ValueError("bandwidth_probe: rows must be [num_tokens, hidden] tensors")
    T, H = ref.shape
    dev = ref.device
    if dev.type != "cuda":
        raise ValueError(f"bandwidth_probe: tensors must be on a GPU, got {dev}")
    for i, t in enumerate(direct):
        _bf16_2d(t, f"direct[{i}]", T, H, dev)
    for i, t in enumerate(outputs):
        _bf16_2d(t, f"outputs[{i}]", T, H, dev)
    if (gathered is None) != (gather_idx is None):
        raise ValueError("bandwidth_probe: gathered and gather_idx go together")
    if gathered is not None:
        if gathered.dim() != 2:
            raise ValueError("gathered must be [num_rows, hidden]")
        _bf16_2d(gathered, "gathered", gathered.shape[0], H, dev)
        if (gather_idx.dtype != torch.int32 or gather_idx.device != dev or gather_idx.dim() != 2
                or gather_idx.shape[0] != T or not gather_idx.is_contiguous()):
            raise ValueError("gather_idx must be a contiguous int32 [num_tokens, k] tensor on "
                             "the rows' device")
    arr = (ctypes.c_void_p * max(1, len(direct)))(*[t.data_ptr() for t in direct])
    outs = (ctypes.c_void_p * max(1, len(outputs)))(*[t.data_ptr() for t in outputs])
    k = 0 if gather_idx is None else int(gather_idx.shape[1])
    n = 0 if gathered is None else int(gathered.shape[0])
    stream = ctypes.c_void_p(torch.cuda.current_stream(ref.device).cuda_stream)
    with torch.cuda.device(ref.device):
        code = _lib.fused_boundary_bandwidth_probe(
            arr, len(direct), _ptr(gathered), n, _ptr(gather_idx), k, outs, len(outputs), T, H,
            int(vec_per_thread), int(workgroups_per_cu), stream)
    if code == FB_HIP_ERROR:
        raise FusedBoundaryError(f"bandwidth_probe: hipError {_lib.fused_boundary_probe_last_hip_error()}")
    _check(code, "bandwidth_probe")


def residency_probe(sgpr_level: int, grid: int, block: int, sleep_ticks: int = 2000,
                    device=None) -> dict:
    """Diagnostic: workgroups a CU really holds at once (see
    fused_boundary_residency_probe).  Launches ``grid`` workgroups of ``block``
    lanes of the probe build ``sgpr_level`` (0, 1, 2: about 20, 88, 104 SGPRs
    per wave), each sleeping ``sleep_ticks`` of the realtime counter, and
    returns {CU id: most workgroups that overlapped on it}."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    out = torch.zeros(3 * int(grid), dtype=torch.int64, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    with torch.cuda.device(dev):
        _check(_lib.fused_boundary_residency_probe(int(sgpr_level), int(grid), int(block),
                                                    int(sleep_ticks), out.data_ptr(), stream),
               "residency_probe")
        torch.cuda.synchronize(dev)
    rows = out.view(-1, 3).cpu().tolist()
    spans = {}
    for hw, t0, t1 in rows:
        cu = ((hw >> 32) & 0xFFFF, (hw & 0xFFFFFFFF) >> 8 & 0xFF)  # XCC, SE/SH/CU fields of HW_ID
        spans.setdefault(cu, []).append((t0, t1))
    most = {}
    for cu, iv in spans.items():
        events = sorted([(a, 1) for a, _ in iv] + [(b, -1) for _, b in iv])
        n = m = 0
        for _, d in events:
            n += d
            m = max(m, n)
        most[cu] = m
    return most
