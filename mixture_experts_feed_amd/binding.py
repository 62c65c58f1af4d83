"""ctypes binding of libinkling_moe.so (argument marshalling only).

Every step of the layer runs in the HIP library; torch supplies device memory
and the current stream.  Names mirror the C ABI in include/inkling_moe.h.
If the library is missing this module raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libinkling_moe.so")

INKLING_OK = 0
INKLING_ERR_INVALID_ARGUMENT = -1
INKLING_ERR_UNSUPPORTED = -2
INKLING_ERR_WORKSPACE = -3
INKLING_ERR_HIP = -4
INKLING_ERR_TOO_LARGE = -5
INKLING_NOALLOC_SCRATCH_BYTES = 64 << 20
INKLING_F32 = 0
INKLING_BF16 = 1

EXPORTED = ("inkling_moe_workspace_size", "inkling_moe_route", "inkling_moe_forward",
            "inkling_moe_strerror", "inkling_moe_last_hip_error", "inkling_moe_set_stage_events",
            "inkling_dense_mlp_workspace_size", "inkling_dense_mlp_forward",
            "inkling_moe_backward_workspace_size", "inkling_moe_backward", "inkling_moe_saved_size",
            "inkling_moe_forward_train", "inkling_moe_forward_noalloc")
INKLING_STAGE_EVENTS = 7
STAGES = ("router_logits", "router_select", "permutation", "gate_up", "down", "shared_down_combine")


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("hidden", ctypes.c_int32), ("n_routed", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class DenseDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class Grads(ctypes.Structure):
    _fields_ = [("d_gate_bank", ctypes.c_void_p), ("d_routed_gate_up", ctypes.c_void_p),
                ("d_routed_down", ctypes.c_void_p), ("d_shared_gate_up", ctypes.c_void_p),
                ("d_shared_down", ctypes.c_void_p), ("weight_grad_dtype", ctypes.c_int32)]


class Gate(ctypes.Structure):
    _fields_ = [("gate_bank", ctypes.c_void_p), ("correction_bias", ctypes.c_void_p),
                ("route_scale", ctypes.c_float), ("global_scale", ctypes.c_float)]


class Experts(ctypes.Structure):
    _fields_ = [("routed_gate_up", ctypes.c_void_p), ("routed_down", ctypes.c_void_p),
                ("shared_gate_up", ctypes.c_void_p), ("shared_down", ctypes.c_void_p)]


class RouteOut(ctypes.Structure):
    _fields_ = [("topk_indices", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
                ("shared_gammas", ctypes.c_void_p), ("expert_counts", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("sorted_slots", ctypes.c_void_p)]


class InklingError(RuntimeError):
    def __init__(self, code: int, where: str):
        lib = load()
        msg = lib.inkling_moe_strerror(code).decode()
        if code == INKLING_ERR_HIP:
            msg += f" (hipError {lib.inkling_moe_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{code}]")
        self.code = code


_LIB: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load the in-tree HIP library (built by mixture_experts_feed_amd.build)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_feed_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.inkling_moe_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_size_t)]
    lib.inkling_moe_workspace_size.restype = ctypes.c_int
    lib.inkling_moe_route.argtypes = [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.POINTER(Gate), ctypes.c_void_p,
                                      ctypes.POINTER(RouteOut), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.inkling_moe_route.restype = ctypes.c_int
    lib.inkling_moe_forward.argtypes = [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.POINTER(Gate),
                                        ctypes.POINTER(Experts), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.POINTER(RouteOut), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.inkling_moe_forward.restype = ctypes.c_int
    lib.inkling_moe_forward_noalloc.argtypes = [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.POINTER(Gate),
                                                ctypes.POINTER(Experts), ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.POINTER(RouteOut), ctypes.c_void_p]
    lib.inkling_moe_forward_noalloc.restype = ctypes.c_int
    lib.inkling_moe_strerror.argtypes = [ctypes.c_int]
    lib.inkling_moe_strerror.restype = ctypes.c_char_p
    lib.inkling_moe_last_hip_error.argtypes = []
    lib.inkling_moe_last_hip_error.restype = ctypes.c_int
    lib.inkling_moe_set_stage_events.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.inkling_moe_set_stage_events.restype = ctypes.c_int
    lib.inkling_dense_mlp_workspace_size.argtypes = [ctypes.POINTER(DenseDims), ctypes.POINTER(ctypes.c_size_t)]
    lib.inkling_dense_mlp_workspace_size.restype = ctypes.c_int
    lib.inkling_dense_mlp_forward.argtypes = [ctypes.POINTER(DenseDims), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.c_void_p]
    lib.inkling_dense_mlp_forward.restype = ctypes.c_int
    lib.inkling_moe_backward_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_size_t)]
    lib.inkling_moe_backward_workspace_size.restype = ctypes.c_int
    lib.inkling_moe_backward.argtypes = [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.POINTER(Gate),
                                         ctypes.POINTER(Experts), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.POINTER(Grads), ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]
    lib.inkling_moe_backward.restype = ctypes.c_int
    lib.inkling_moe_saved_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_size_t)]
    lib.inkling_moe_saved_size.restype = ctypes.c_int
    lib.inkling_moe_forward_train.argtypes = [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.POINTER(Gate),
                                              ctypes.POINTER(Experts), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.inkling_moe_forward_train.restype = ctypes.c_int
    _LIB = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return INKLING_F32
    if dt == torch.bfloat16:
        return INKLING_BF16
    raise ValueError(f"unsupported dtype {dt}")


def make_dims(T, hidden, n_routed, top_k, n_shared, intermediate, dtype, out_dtype=None) -> Dims:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    ocode = code if out_dtype is None else (out_dtype if isinstance(out_dtype, int) else _dtype_code(out_dtype))
    return Dims(int(T), int(hidden), int(n_routed), int(top_k), int(n_shared), int(intermediate), code, ocode)


def workspace_size(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    rc = load().inkling_moe_workspace_size(ctypes.byref(dims), ctypes.byref(n))
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_moe_workspace_size")
    return int(n.value)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def alloc_workspace(dims: Dims, device) -> torch.Tensor:
    return torch.empty(max(1, workspace_size(dims)), dtype=torch.uint8, device=device)


def route(x: torch.Tensor, gate_bank: torch.Tensor, bias: torch.Tensor, top_k: int, route_scale: float,
          global_scale: float, padding_mask: Optional[torch.Tensor] = None, permutation: bool = True,
          workspace: Optional[torch.Tensor] = None, intermediate: int = 64):
    """inkling_moe_route: returns dict(topk_indices, topk_weights, shared_gammas[, expert_counts,
    expert_offsets, sorted_slots])."""
    T, H = x.shape
    E = bias.shape[0]
    S = gate_bank.shape[0] - E
    _need(x, "x")
    _need(gate_bank, "gate_bank", torch.float32)
    _need(bias, "bias", torch.float32)
    dims = make_dims(T, H, E, top_k, S, intermediate, x.dtype)
    dev = x.device
    res = {
        "topk_indices": torch.empty((T, top_k), dtype=torch.int32, device=dev),
        "topk_weights": torch.empty((T, top_k), dtype=torch.float32, device=dev),
        "shared_gammas": torch.empty((T, S), dtype=torch.float32, device=dev),
    }
    if permutation:
        res["expert_counts"] = torch.empty((E,), dtype=torch.int32, device=dev)
        res["expert_offsets"] = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        res["sorted_slots"] = torch.full((max(1, T * top_k),), -1, dtype=torch.int32, device=dev)
    ro = RouteOut(*[_ptr(res.get(n)) for n in ("topk_indices", "topk_weights", "shared_gammas", "expert_counts",
                                               "expert_offsets", "sorted_slots")])
    gate = Gate(gate_bank.data_ptr(), bias.data_ptr(), float(route_scale), float(global_scale))
    if padding_mask is not None:
        _need(padding_mask, "padding_mask", torch.uint8)
    if workspace is None:
        workspace = alloc_workspace(dims, dev)
    rc = load().inkling_moe_route(ctypes.byref(dims), x.data_ptr(), ctypes.byref(gate), _ptr(padding_mask),
                                  ctypes.byref(ro), workspace.data_ptr(), workspace.numel(), _stream(dev))
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_moe_route")
    return res


def _forward_args(x, gate_bank, bias, w_gu, w_d, wsh_gu, wsh_d, top_k, route_scale, global_scale, padding_mask,
                  out, return_routing, out_dtype):
    """Checks and C structs shared by forward() and forward_noalloc()."""
    T, H = x.shape
    E, twoI, _ = w_gu.shape
    S = 0 if wsh_gu is None else wsh_gu.shape[0]
    for t, n in ((x, "x"), (w_gu, "w_gu"), (w_d, "w_d")):
        _need(t, n, x.dtype)
    if S:
        _need(wsh_gu, "wsh_gu", x.dtype)
        _need(wsh_d, "wsh_d", x.dtype)
    _need(gate_bank, "gate_bank", torch.float32)
    _need(bias, "bias", torch.float32)
    if gate_bank.shape[0] != E + S:
        raise ValueError("gate_bank must hold n_routed + n_shared rows")
    if out is not None:
        out_dtype = out.dtype
    out_dtype = x.dtype if out_dtype is None else out_dtype
    dims = make_dims(T, H, E, top_k, S, twoI // 2, x.dtype, out_dtype)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype)
    if padding_mask is not None:
        _need(padding_mask, "padding_mask", torch.uint8)
    routing = None
    ro = None
    if return_routing:
        routing = {
            "topk_indices": torch.empty((T, top_k), dtype=torch.int32, device=dev),
            "topk_weights": torch.empty((T, top_k), dtype=torch.float32, device=dev),
            "shared_gammas": torch.empty((T, S), dtype=torch.float32, device=dev),
            "expert_counts": torch.empty((E,), dtype=torch.int32, device=dev),
            "expert_offsets": torch.empty((E + 1,), dtype=torch.int32, device=dev),
            "sorted_slots": torch.full((max(1, T * top_k),), -1, dtype=torch.int32, device=dev),
        }
        ro = RouteOut(*[_ptr(routing[n]) for n in ("topk_indices", "topk_weights", "shared_gammas",
                                                   "expert_counts", "expert_offsets", "sorted_slots")])
    gate = Gate(gate_bank.data_ptr(), bias.data_ptr(), float(route_scale), float(global_scale))
    ex = Experts(w_gu.data_ptr(), w_d.data_ptr(), _ptr(wsh_gu) if S else None, _ptr(wsh_d) if S else None)
    return dims, gate, ex, out, routing, ro


def forward(x: torch.Tensor, gate_bank: torch.Tensor, bias: torch.Tensor, w_gu: torch.Tensor, w_d: torch.Tensor,
            wsh_gu: Optional[torch.Tensor], wsh_d: Optional[torch.Tensor], top_k: int, route_scale: float,
            global_scale: float, padding_mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, return_routing: bool = False,
            out_dtype: Optional[torch.dtype] = None, saved: Optional[torch.Tensor] = None):
    """inkling_moe_forward: out [T, H] (x's dtype unless out / out_dtype says
    otherwise) and the routing dict if asked.  With `saved` (uint8, saved_size
    bytes) it is inkling_moe_forward_train, which also keeps the gate_up
    projections there for backward()."""
    dims, gate, ex, out, routing, ro = _forward_args(x, gate_bank, bias, w_gu, w_d, wsh_gu, wsh_d, top_k,
                                                     route_scale, global_scale, padding_mask, out, return_routing,
                                                     out_dtype)
    dev = x.device
    if workspace is None:
        workspace = alloc_workspace(dims, dev)
    if saved is not None:
        if return_routing:
            raise ValueError("the training forward does not return the routing")
        if saved.dtype != torch.uint8 or not saved.is_contiguous() or saved.numel() < saved_size(dims):
            raise ValueError("saved must be a contiguous uint8 tensor of saved_size(dims) bytes")
        rc = load().inkling_moe_forward_train(ctypes.byref(dims), x.data_ptr(), ctypes.byref(gate), ctypes.byref(ex),
                                              _ptr(padding_mask), out.data_ptr(), saved.data_ptr(),
                                              workspace.data_ptr(), workspace.numel(), _stream(dev))
        if rc != INKLING_OK:
            raise InklingError(rc, "inkling_moe_forward_train")
        return out
    rc = load().inkling_moe_forward(ctypes.byref(dims), x.data_ptr(), ctypes.byref(gate), ctypes.byref(ex),
                                    _ptr(padding_mask), out.data_ptr(), None if ro is None else ctypes.byref(ro),
                                    workspace.data_ptr(), workspace.numel(), _stream(dev))
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_moe_forward")
    return (out, routing) if return_routing else out


def forward_noalloc(x: torch.Tensor, gate_bank: torch.Tensor, bias: torch.Tensor, w_gu: torch.Tensor,
                    w_d: torch.Tensor, wsh_gu: Optional[torch.Tensor], wsh_d: Optional[torch.Tensor], top_k: int,
                    route_scale: float, global_scale: float, padding_mask: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, return_routing: bool = False,
                    out_dtype: Optional[torch.dtype] = None):
    """inkling_moe_forward_noalloc: forward() without a workspace (the
    library's static scratch of INKLING_NOALLOC_SCRATCH_BYTES per GPU).  With
    `out` given and no routing asked for, this allocates nothing."""
    dims, gate, ex, out, routing, ro = _forward_args(x, gate_bank, bias, w_gu, w_d, wsh_gu, wsh_d, top_k,
                                                     route_scale, global_scale, padding_mask, out, return_routing,
                                                     out_dtype)
    rc = load().inkling_moe_forward_noalloc(ctypes.byref(dims), x.data_ptr(), ctypes.byref(gate), ctypes.byref(ex),
                                            _ptr(padding_mask), out.data_ptr(),
                                            None if ro is None else ctypes.byref(ro), _stream(x.device))
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_moe_forward_noalloc")
    return (out, routing) if return_routing else out


def saved_size(dims: Dims) -> int:
    """inkling_moe_saved_size: bytes of the activations the training forward keeps."""
    n = ctypes.c_size_t(0)
    rc = load().inkling_moe_saved_size(ctypes.byref(dims), ctypes.byref(n))
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_moe_saved_size")
    return n.value


def set_stage_events(events: Optional[ctypes.Array]) -> None:
    """Install (or clear with None) an array of INKLING_STAGE_EVENTS hipEvent_t
    handles recorded by later forward calls on this thread."""
    n = 0 if events is None else len(events)
    rc = load().inkling_moe_set_stage_events(None if events is None else ctypes.cast(events, ctypes.c_void_p), n)
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_moe_set_stage_events")


def make_dense_dims(T, hidden, intermediate, dtype, out_dtype=None) -> DenseDims:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    ocode = code if out_dtype is None else (out_dtype if isinstance(out_dtype, int) else _dtype_code(out_dtype))
    return DenseDims(int(T), int(hidden), int(intermediate), code, ocode)


def dense_workspace_size(dims: DenseDims) -> int:
    n = ctypes.c_size_t(0)
    rc = load().inkling_dense_mlp_workspace_size(ctypes.byref(dims), ctypes.byref(n))
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_dense_mlp_workspace_size")
    return int(n.value)


def dense_mlp_forward(x: torch.Tensor, gate_up: torch.Tensor, down: torch.Tensor, global_scale: float,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """inkling_dense_mlp_forward: InklingDenseMLP on x [T, H] with gate_up
    [2I, H] (interleaved) and down [H, I]."""
    T, H = x.shape
    twoI = gate_up.shape[0]
    for t, n in ((x, "x"), (gate_up, "gate_up"), (down, "down")):
        _need(t, n, x.dtype)
    if gate_up.shape != (twoI, H) or down.shape != (H, twoI // 2):
        raise ValueError("gate_up must be [2I, H] and down [H, I]")
    if out is not None:
        out_dtype = out.dtype
    out_dtype = x.dtype if out_dtype is None else out_dtype
    dims = make_dense_dims(T, H, twoI // 2, x.dtype, out_dtype)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype)
    if workspace is None:
        workspace = torch.empty(max(1, dense_workspace_size(dims)), dtype=torch.uint8, device=dev)
    rc = load().inkling_dense_mlp_forward(ctypes.byref(dims), x.data_ptr(), gate_up.data_ptr(), down.data_ptr(),
                                          float(global_scale), out.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), _stream(dev))
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_dense_mlp_forward")
    return out


def backward_workspace_size(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    rc = load().inkling_moe_backward_workspace_size(ctypes.byref(dims), ctypes.byref(n))
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_moe_backward_workspace_size")
    return int(n.value)


def backward(x: torch.Tensor, gate_bank: torch.Tensor, bias: torch.Tensor, w_gu: torch.Tensor, w_d: torch.Tensor,
             wsh_gu: Optional[torch.Tensor], wsh_d: Optional[torch.Tensor], top_k: int, route_scale: float,
             global_scale: float, dout: torch.Tensor, padding_mask: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, dx_dtype: Optional[torch.dtype] = None,
             grads: Optional[dict] = None, saved: Optional[torch.Tensor] = None,
             weight_grad_dtype: Optional[torch.dtype] = None) -> dict:
    """inkling_moe_backward: dict(dx, d_gate_bank, d_w_gu, d_w_d, d_wsh_gu, d_wsh_d).
    `saved`: the tensor a training forward with the same arguments filled, or
    None to recompute the gate_up projections.  The weight gradients are fp32
    (default) or bf16 (`weight_grad_dtype`, or the dtype of the given
    `grads` tensors)."""
    T, H = x.shape
    E, twoI, _ = w_gu.shape
    S = 0 if wsh_gu is None else wsh_gu.shape[0]
    for t, n in ((x, "x"), (w_gu, "w_gu"), (w_d, "w_d"), (dout, "dout")):
        _need(t, n, x.dtype)
    if S:
        _need(wsh_gu, "wsh_gu", x.dtype)
        _need(wsh_d, "wsh_d", x.dtype)
    _need(gate_bank, "gate_bank", torch.float32)
    _need(bias, "bias", torch.float32)
    dx_dtype = x.dtype if dx_dtype is None else dx_dtype
    dims = make_dims(T, H, E, top_k, S, twoI // 2, x.dtype, dx_dtype)
    dev = x.device
    if grads is None:
        wdt = dict(dtype=torch.float32 if weight_grad_dtype is None else weight_grad_dtype, device=dev)
        grads = {"dx": torch.empty((T, H), dtype=dx_dtype, device=dev),
                 "d_gate_bank": torch.empty(tuple(gate_bank.shape), dtype=torch.float32, device=dev),
                 "d_w_gu": torch.empty(tuple(w_gu.shape), **wdt), "d_w_d": torch.empty(tuple(w_d.shape), **wdt),
                 "d_wsh_gu": torch.empty(tuple(wsh_gu.shape), **wdt) if S else None,
                 "d_wsh_d": torch.empty(tuple(wsh_d.shape), **wdt) if S else None}
    wdtype = grads["d_w_gu"].dtype
    if weight_grad_dtype is not None and weight_grad_dtype != wdtype:
        raise ValueError("weight_grad_dtype differs from the dtype of the given gradient tensors")
    for n in ("d_w_d", "d_wsh_gu", "d_wsh_d"):
        if grads[n] is not None and grads[n].dtype != wdtype:
            raise ValueError("the four weight gradients must share one dtype")
    g = Grads(_ptr(grads["d_gate_bank"]), _ptr(grads["d_w_gu"]), _ptr(grads["d_w_d"]), _ptr(grads["d_wsh_gu"]),
              _ptr(grads["d_wsh_d"]), _dtype_code(wdtype))
    gate = Gate(gate_bank.data_ptr(), bias.data_ptr(), float(route_scale), float(global_scale))
    ex = Experts(w_gu.data_ptr(), w_d.data_ptr(), _ptr(wsh_gu) if S else None, _ptr(wsh_d) if S else None)
    if padding_mask is not None:
        _need(padding_mask, "padding_mask", torch.uint8)
    if workspace is None:
        workspace = torch.empty(max(1, backward_workspace_size(dims)), dtype=torch.uint8, device=dev)
    if saved is not None and (saved.dtype != torch.uint8 or saved.numel() < saved_size(dims)):
        raise ValueError("saved must be the uint8 tensor of saved_size(dims) bytes a training forward filled")
    rc = load().inkling_moe_backward(ctypes.byref(dims), x.data_ptr(), ctypes.byref(gate), ctypes.byref(ex),
                                     _ptr(padding_mask), dout.data_ptr(), _ptr(saved), grads["dx"].data_ptr(),
                                     ctypes.byref(g), workspace.data_ptr(), workspace.numel(), _stream(dev))
    if rc != INKLING_OK:
        raise InklingError(rc, "inkling_moe_backward")
    return grads
