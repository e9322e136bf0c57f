"""ctypes binding of ``libmoe.so`` (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the MoE forward path runs in the
library's HIP kernels.  The functions keep the C names; tensors are torch
tensors on the GPU (PyTorch provides device memory and streams only).

The library is loaded from this package directory.  If it is missing the
first call raises -- there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY may name another build of the same library (the host-sanitized
# libmoe_san.so of build.py); by default the one built in this directory.
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_HERE, "libmoe.so")

MOE_SCORE_SOFTMAX = 0
MOE_SCORE_SIGMOID = 1
MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_TOPK",
          -4: "MOE_ERR_ALIGN", -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_UNSUPPORTED",
          -7: "MOE_ERR_HIP", -8: "MOE_ERR_STATIC_LIMIT"}
MOE_STATIC_WORKSPACE_BYTES = 256 << 20  # include/moe.h

# Every symbol include/moe.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
SIGNATURES = {
    "moe_abi_version": (_I, []),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_workspace_size": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "moe_workspace_size_ex": (_I, [_I, _I, _I, _I, _I, _P, ctypes.POINTER(_SZ)]),
    "moe_plan": (_I, [_I, _I, _I, _I, _I, _P, ctypes.POINTER(_I), ctypes.POINTER(_I),
                      ctypes.POINTER(_I)]),
    "moe_forward": (_I, [_P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "moe_forward_ex": (_I, [_P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "moe_forward_static": (_I, [_P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _P]),
    "moe_router_logits": (_I, [_P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "moe_router_workspace_size": (_I, [_I, _I, _I, ctypes.POINTER(_SZ)]),
    "moe_forward_router": (_I, [_P, _P, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _I, _P, _P, _SZ,
                                _P]),
    "moe_plan_ex": (_I, [_I, _I, _I, _I, _I, _P, _P]),
    "moe_route_workspace_size": (_I, [_I, _I, _I, _P, ctypes.POINTER(_SZ)]),
    "moe_route": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                       _P, ctypes.POINTER(_I), _P, _SZ, _P]),
    "moe_timer_create": (_I, [ctypes.POINTER(_P)]),
    "moe_timer_destroy": (_I, [_P]),
    "moe_timer_record": (_I, [_P, _P]),
    "moe_timer_elapsed_ms": (_I, [_P, _P, ctypes.POINTER(ctypes.c_float)]),
}


class MoeOptions(ctypes.Structure):
    """struct moe_options of include/moe.h."""
    _fields_ = [("block_rows", ctypes.c_int), ("split_k", ctypes.c_int),
                ("tile_variant", ctypes.c_int), ("down_variant", ctypes.c_int),
                ("rotate", ctypes.c_int),
                ("routing_kernels", ctypes.c_int), ("gather_mode", ctypes.c_int),
                ("unfused_swiglu", ctypes.c_int), ("xcd_order", ctypes.c_int),
                ("fold_combine", ctypes.c_int), ("fuse_down", ctypes.c_int),
                ("schedule", ctypes.c_int), ("stage_events", ctypes.c_void_p)]


class MoePlanInfo(ctypes.Structure):
    """struct moe_plan_info of include/moe.h."""
    _fields_ = [(n, ctypes.c_int) for n in (
        "block_rows", "split_k", "fused_down", "routing_launches", "gather_launch",
        "gate_up_variant", "down_variant", "unfused_swiglu", "fold_combine", "xcd_grouped",
        "launches", "split_on_device", "stream_k", "variable_rows")] + [
        ("var_table_offset", ctypes.c_longlong), ("var_count_offset", ctypes.c_longlong)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_string(status)})")


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m expert_dispatch_router_amd.build` (hipcc, gfx950)")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
        return _lib


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def moe_abi_version() -> int:
    return int(lib().moe_abi_version())


def _opts(block_rows=0, split_k=0, stage_events=None, tile_variant=0, rotate=0,
          routing_kernels=0, gather_mode=0, unfused_swiglu=0, xcd_order=0, down_variant=0,
          fold_combine=0, fuse_down=0, schedule=0):
    if not any((block_rows, split_k, tile_variant, rotate, routing_kernels, gather_mode,
                unfused_swiglu, xcd_order, down_variant, fold_combine,
                fuse_down, schedule)) and stage_events is None:
        return None, None
    o = MoeOptions(int(block_rows), int(split_k), int(tile_variant), int(down_variant),
                   int(rotate), int(routing_kernels), int(gather_mode), int(unfused_swiglu),
                   int(xcd_order), int(fold_combine), int(fuse_down), int(schedule), None)
    keep = []
    if stage_events is not None:
        if len(stage_events) != 7:
            raise ValueError("stage_events takes 7 event handles")
        a = (ctypes.c_void_p * 7)(*stage_events)
        keep.append(a)
        o.stage_events = ctypes.cast(a, ctypes.c_void_p)
    return o, keep


def moe_workspace_size(T, d, ffn, E, top_k, block_rows=0, split_k=0, tile_variant=0,
                       rotate=0, routing_kernels=0, gather_mode=0, unfused_swiglu=0,
                       xcd_order=0, down_variant=0, fold_combine=0, fuse_down=0,
                       schedule=0) -> int:
    o, _ = _opts(block_rows, split_k, None, tile_variant, rotate, routing_kernels, gather_mode,
                 unfused_swiglu, xcd_order, down_variant, fold_combine, fuse_down, schedule)
    n = _SZ(0)
    _check("moe_workspace_size_ex", lib().moe_workspace_size_ex(
        T, d, ffn, E, top_k, ctypes.byref(o) if o else None, ctypes.byref(n)))
    return int(n.value)


def moe_plan(T, d, ffn, E, top_k, block_rows=0, split_k=0, tile_variant=0, rotate=0,
             fuse_down=0, with_fusion=False, unfused_swiglu=0):
    """(block_rows, split_k) the library uses for these sizes and options;
    with ``with_fusion`` also whether the down projection is fused into the
    gate/up GEMM."""
    o, _ = _opts(block_rows, split_k, None, tile_variant, rotate, unfused_swiglu=unfused_swiglu,
                 fuse_down=fuse_down)
    bm, sk, fd = _I(0), _I(0), _I(0)
    _check("moe_plan", lib().moe_plan(T, d, ffn, E, top_k, ctypes.byref(o) if o else None,
                                       ctypes.byref(bm), ctypes.byref(sk), ctypes.byref(fd)))
    if with_fusion:
        return int(bm.value), int(sk.value), bool(fd.value)
    return int(bm.value), int(sk.value)


def moe_plan_ex(T, d, ffn, E, top_k, **options) -> dict:
    """The launch plan moe_forward_ex follows for these sizes and options
    (the fields of struct moe_plan_info)."""
    o, _ = _opts(**options)
    info = MoePlanInfo()
    _check("moe_plan_ex", lib().moe_plan_ex(T, d, ffn, E, top_k, ctypes.byref(o) if o else None,
                                             ctypes.byref(info)))
    return {n: int(getattr(info, n)) for n, _ in MoePlanInfo._fields_}


def moe_route_workspace_size(T, E, top_k, block_rows=0, routing_kernels=0) -> int:
    o, _ = _opts(block_rows, routing_kernels=routing_kernels)
    n = _SZ(0)
    _check("moe_route_workspace_size", lib().moe_route_workspace_size(
        T, E, top_k, ctypes.byref(o) if o else None, ctypes.byref(n)))
    return int(n.value)


def _score_code(score) -> int:
    if isinstance(score, str):
        return {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}[score]
    return int(score)


def _dev_ptr(t, dtype, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _same_device(tensors):
    """All given tensors on one GPU (checked before any launch: a kernel
    reading another device's memory faults)."""
    devs = {t.device for _, t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError("tensors on different devices: " +
                         ", ".join(f"{n} on {t.device}" for n, t in tensors if t is not None))


def _check_out(out, shape, name="out"):
    """A caller's output buffer must have exactly the shape the kernels
    write (a smaller one would be written past its end)."""
    if out is not None and tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(out.shape)}")


def _stream_ptr(stream, device):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def moe_forward(x, router_logits, W_gate_up, W_down, top_k, renormalize, out=None,
                score="softmax", workspace=None, stream=None, block_rows=0, split_k=0,
                stage_events=None, tile_variant=0, rotate=0, routing_kernels=0, gather_mode=0,
                unfused_swiglu=0, xcd_order=0, down_variant=0, fold_combine=0, fuse_down=0,
                schedule=0):
    """out[T,d] (bf16) = the MoE forward pass, enqueued on ``stream``.

    x bf16 [T,d]; router_logits fp32 [T,E]; W_gate_up bf16 [E,2F,d];
    W_down bf16 [E,d,F].  ``out`` and ``workspace`` (uint8) are allocated
    with torch when not given.  ``stage_events``: 7 HIP event handles
    recorded between the stages (moe_options; None entries skipped)."""
    T, d = x.shape
    E = router_logits.shape[1]
    F = W_down.shape[2]
    if router_logits.shape[0] != T or tuple(W_gate_up.shape) != (E, 2 * F, d) or \
            tuple(W_down.shape) != (E, d, F):
        raise ValueError("inconsistent shapes")
    _check_out(out, (T, d))
    _same_device([("x", x), ("router_logits", router_logits), ("W_gate_up", W_gate_up),
                  ("W_down", W_down), ("out", out), ("workspace", workspace)])
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16, device=x.device)
    ws_need = moe_workspace_size(T, d, F, E, top_k, block_rows, split_k, tile_variant, rotate,
                                 routing_kernels, gather_mode, unfused_swiglu, xcd_order,
                                 down_variant, fold_combine, fuse_down, schedule)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=x.device)
    o, keep = _opts(block_rows, split_k, stage_events, tile_variant, rotate, routing_kernels,
                    gather_mode, unfused_swiglu, xcd_order, down_variant, fold_combine, fuse_down,
                    schedule)
    rc = lib().moe_forward_ex(
        _dev_ptr(x, torch.bfloat16, "x"), _dev_ptr(router_logits, torch.float32, "router_logits"),
        _dev_ptr(W_gate_up, torch.bfloat16, "W_gate_up"), _dev_ptr(W_down, torch.bfloat16, "W_down"),
        int(top_k), int(bool(renormalize)), _dev_ptr(out, torch.bfloat16, "out"),
        T, d, F, E, _score_code(score), ctypes.byref(o) if o else None,
        _dev_ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream_ptr(stream, x.device))
    del keep
    _check("moe_forward_ex", rc)
    return out


def moe_forward_static(x, router_logits, W_gate_up, W_down, top_k, renormalize, out,
                       score="softmax", stream=None):
    """moe_forward with the library's own fixed device workspace (no device
    memory allocated by the call; the caller passes ``out``, bf16 [T, d]).
    Calls on one GPU must not overlap (they share its workspace array)."""
    T, d = x.shape
    E = router_logits.shape[1]
    F = W_down.shape[2]
    if router_logits.shape[0] != T or tuple(W_gate_up.shape) != (E, 2 * F, d) or \
            tuple(W_down.shape) != (E, d, F):
        raise ValueError("inconsistent shapes")
    if out is None:
        raise ValueError("out is required: this entry point allocates nothing")
    _check_out(out, (T, d))
    _same_device([("x", x), ("router_logits", router_logits), ("W_gate_up", W_gate_up),
                  ("W_down", W_down), ("out", out)])
    rc = lib().moe_forward_static(
        _dev_ptr(x, torch.bfloat16, "x"), _dev_ptr(router_logits, torch.float32, "router_logits"),
        _dev_ptr(W_gate_up, torch.bfloat16, "W_gate_up"), _dev_ptr(W_down, torch.bfloat16, "W_down"),
        int(top_k), int(bool(renormalize)), _dev_ptr(out, torch.bfloat16, "out"),
        T, d, F, E, _score_code(score), _stream_ptr(stream, x.device))
    _check("moe_forward_static", rc)
    return out


def moe_router_workspace_size(T, d, E) -> int:
    n = _SZ(0)
    _check("moe_router_workspace_size", lib().moe_router_workspace_size(T, d, E, ctypes.byref(n)))
    return int(n.value)


def moe_router_logits(x, W_router, out=None, workspace=None, stream=None):
    """logits fp32 [T,E] = x . W_router^T for x bf16 [T,d], W_router bf16
    [E,d], enqueued on ``stream``."""
    T, d = x.shape
    E = W_router.shape[0]
    if tuple(W_router.shape) != (E, d):
        raise ValueError("inconsistent shapes")
    _check_out(out, (T, E))
    _same_device([("x", x), ("W_router", W_router), ("out", out), ("workspace", workspace)])
    if out is None:
        out = torch.empty(T, E, dtype=torch.float32, device=x.device)
    need = moe_router_workspace_size(T, d, E)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    rc = lib().moe_router_logits(_dev_ptr(x, torch.bfloat16, "x"),
                                 _dev_ptr(W_router, torch.bfloat16, "W_router"),
                                 _dev_ptr(out, torch.float32, "logits"), T, d, E,
                                 _dev_ptr(workspace, torch.uint8, "workspace"),
                                 0 if workspace is None else workspace.numel(),
                                 _stream_ptr(stream, x.device))
    _check("moe_router_logits", rc)
    return out


def moe_forward_router(x, W_router, W_gate_up, W_down, top_k, renormalize, out=None,
                       logits_out=None, score="softmax", workspace=None, stream=None,
                       block_rows=0, split_k=0, stage_events=None, tile_variant=0, rotate=0,
                       routing_kernels=0, gather_mode=0, unfused_swiglu=0, xcd_order=0,
                       down_variant=0, fold_combine=0, fuse_down=0, schedule=0):
    """moe_forward from the hidden states: router scores x . W_router^T
    (written to ``logits_out`` when given), then the forward pass."""
    T, d = x.shape
    E = W_router.shape[0]
    F = W_down.shape[2]
    if tuple(W_router.shape) != (E, d) or tuple(W_gate_up.shape) != (E, 2 * F, d) or \
            tuple(W_down.shape) != (E, d, F):
        raise ValueError("inconsistent shapes")
    _check_out(logits_out, (T, E), "logits_out")
    _check_out(out, (T, d))
    _same_device([("x", x), ("W_router", W_router), ("W_gate_up", W_gate_up), ("W_down", W_down),
                  ("out", out), ("logits_out", logits_out), ("workspace", workspace)])
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16, device=x.device)
    ws_need = moe_workspace_size(T, d, F, E, top_k, block_rows, split_k, tile_variant, rotate,
                                 routing_kernels, gather_mode, unfused_swiglu, xcd_order,
                                 down_variant, fold_combine, fuse_down, schedule)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=x.device)
    o, keep = _opts(block_rows, split_k, stage_events, tile_variant, rotate, routing_kernels,
                    gather_mode, unfused_swiglu, xcd_order, down_variant, fold_combine, fuse_down,
                    schedule)
    rc = lib().moe_forward_router(
        _dev_ptr(x, torch.bfloat16, "x"), _dev_ptr(W_router, torch.bfloat16, "W_router"),
        _dev_ptr(W_gate_up, torch.bfloat16, "W_gate_up"), _dev_ptr(W_down, torch.bfloat16, "W_down"),
        int(top_k), int(bool(renormalize)), _dev_ptr(out, torch.bfloat16, "out"),
        None if logits_out is None else _dev_ptr(logits_out, torch.float32, "logits_out"),
        T, d, F, E, _score_code(score), ctypes.byref(o) if o else None,
        _dev_ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream_ptr(stream, x.device))
    del keep
    _check("moe_forward_router", rc)
    return out


def moe_route(router_logits, top_k, renormalize, score="softmax", x=None, block_rows=0,
              workspace=None, stream=None, routing_kernels=0):
    """Runs the routing kernels and returns a dict of GPU tensors: ids, w,
    counts, offsets, perm, inv, blocks [nb_max,2], nb [1], order [nb_max]
    (the blocks longest first), x_perm (if x is given) and the host int bm."""
    T, E = router_logits.shape
    dev = router_logits.device
    A = T * top_k
    if x is not None and x.dim() != 2:
        raise ValueError("x must be [T, d]")
    if x is not None and x.shape[0] != T:
        raise ValueError(f"x must have one row per token: {x.shape[0]} rows for T = {T}")
    _same_device([("router_logits", router_logits), ("x", x), ("workspace", workspace)])
    i32 = dict(dtype=torch.int32, device=dev)
    res = dict(ids=torch.empty(T, top_k, **i32),
               w=torch.empty(T, top_k, dtype=torch.float32, device=dev),
               counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
               perm=torch.empty(A, **i32), inv=torch.empty(A, **i32))
    o, _ = _opts(block_rows, routing_kernels=routing_kernels)
    ws_need = moe_route_workspace_size(T, E, top_k, block_rows, routing_kernels)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=dev)
    bm, _ = moe_plan(T, 64, 64, E, top_k, block_rows)
    nb_max = (A + bm - 1) // bm + min(E, A) if A > 0 else 0
    res["blocks"] = torch.zeros(max(nb_max, 1), 2, **i32)
    res["nb"] = torch.zeros(1, **i32)
    res["order"] = torch.zeros(max(nb_max, 1), **i32)
    d = 0
    if x is not None:
        d = x.shape[1]
        res["x_perm"] = torch.empty(A, d, dtype=torch.bfloat16, device=dev)
    bm_used = _I(0)
    rc = lib().moe_route(
        _dev_ptr(router_logits, torch.float32, "router_logits"), T, E, int(top_k),
        int(bool(renormalize)), _score_code(score), ctypes.byref(o) if o else None,
        res["ids"].data_ptr(), res["w"].data_ptr(), res["counts"].data_ptr(),
        res["offsets"].data_ptr(), res["perm"].data_ptr(), res["inv"].data_ptr(),
        res["blocks"].data_ptr(), res["nb"].data_ptr(), res["order"].data_ptr(),
        _dev_ptr(x, torch.bfloat16, "x") if x is not None else None, d,
        res["x_perm"].data_ptr() if x is not None else None, ctypes.byref(bm_used),
        _dev_ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream_ptr(stream, dev))
    _check("moe_route", rc)
    res["bm"] = int(bm_used.value)
    return res


class Timer:
    """A HIP event created and owned by the library (moe_timer_*)."""

    def __init__(self):
        h = _P(None)
        _check("moe_timer_create", lib().moe_timer_create(ctypes.byref(h)))
        self.handle = h.value

    def record(self, stream=None):
        """Records the event on ``stream`` (torch's current stream if None)."""
        s = torch.cuda.current_stream() if stream is None else stream
        _check("moe_timer_record", lib().moe_timer_record(self.handle, s.cuda_stream))

    def elapsed_ms(self, stop: "Timer") -> float:
        ms = ctypes.c_float(0.0)
        _check("moe_timer_elapsed_ms", lib().moe_timer_elapsed_ms(self.handle, stop.handle,
                                                                  ctypes.byref(ms)))
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle and _lib is not None:
                _lib.moe_timer_destroy(self.handle)
        except Exception:
            pass
