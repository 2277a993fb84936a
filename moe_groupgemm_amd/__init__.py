"""Python binding of the MoE-layer megakernel library (``libmoe_mk.so``, C ABI in include/moe_mk.h).

Argument marshalling only: every step of the layer runs in the HIP library.  PyTorch
supplies device memory and streams.  The functions carry the C names; see the header for
the meaning of each argument.  There is no fallback: if the library is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mk.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe_mk.h")

MOE_MK_SCHED_STATIC = 0
MOE_MK_SCHED_DYNAMIC = 1
MOE_MK_SCHED_STATIC_COOPERATIVE = 2
MOE_MK_OK = 0
MOE_MK_ERR_WATCHDOG = 1
MOE_MK_ERR_NONFINITE = 2
MOE_MK_ERR_QUEUE = 4
MOE_MK_ERR_UNINIT = 8
MOE_MK_DEBUG_DROP_NOTIFY = 1
MOE_MK_DEBUG_TRACE = 2
MOE_MK_DEBUG_NO_PREFETCH = 4
MOE_MK_DEBUG_NARROW_ONLY = 8
MOE_MK_DEBUG_BATCH_RULE = 16
MOE_MK_DEBUG_GROUPED_GATE_UP = 32
TASK_KINDS = ("route", "topk", "scan", "group", "gemm1", "gemm2", "combine")
# control block words (see moe_mk_routing_view)
CTL_WORDS = 512
CTL = {"epoch": 0, "exit": 1, "err": 2, "ev_topk": 5, "ev_scan": 6, "magic": 8, "mt_total": 9, "mw": 10,
       "qhead": 32, "qtail": 64, "pf": 96, "cq": 128, "ev_g1": 160, "dbg": 192, "xq": 256}

_lib = None


class MoeMkError(RuntimeError):
    def __init__(self, what: str, code: int):
        super().__init__(f"{what}: {moe_mk_status_str(code)} ({code})")
        self.code = code


class _RoutingView(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("hist", ctypes.c_void_p),
                ("exp_indptr", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("inv", ctypes.c_void_p),
                ("logits", ctypes.c_void_p), ("ctl", ctypes.c_void_p), ("mt_expert", ctypes.c_void_p),
                ("mt_row0", ctypes.c_void_p), ("mt_rows", ctypes.c_void_p), ("mt_cap", ctypes.c_int64)]


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with moe_groupgemm_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.moe_mk_plan.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int]
    L.moe_mk_plan.restype = ctypes.c_int
    L.moe_mk_plan_destroy.argtypes = [vp]
    L.moe_mk_plan_destroy.restype = None
    L.moe_mk_workspace_bytes.argtypes = [vp, i64]
    L.moe_mk_workspace_bytes.restype = sz
    L.moe_mk_workspace_init.argtypes = [vp, vp, sz, vp]
    L.moe_mk_workspace_init.restype = ctypes.c_int
    L.moe_mk_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, sz, vp]
    L.moe_mk_forward.restype = ctypes.c_int
    L.moe_mk_forward_unfused.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, sz, vp]
    L.moe_mk_forward_unfused.restype = ctypes.c_int
    L.moe_mk_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp]
    L.moe_mk_forward_noalloc.restype = ctypes.c_int
    L.moe_mk_routing_view.argtypes = [vp, i64, vp, sz, ctypes.POINTER(_RoutingView)]
    L.moe_mk_routing_view.restype = ctypes.c_int
    L.moe_mk_workspace_error.argtypes = [vp, vp, sz, vp, ctypes.POINTER(i32)]
    L.moe_mk_workspace_error.restype = ctypes.c_int
    L.moe_mk_plan_info.argtypes = [vp, ctypes.c_char_p]
    L.moe_mk_plan_info.restype = i64
    L.moe_mk_forward_info.argtypes = [vp, i64, ctypes.c_char_p]
    L.moe_mk_forward_info.restype = i64
    L.moe_mk_plan_set_debug.argtypes = [vp, i64, i32]
    L.moe_mk_plan_set_debug.restype = ctypes.c_int
    L.moe_mk_trace_view.argtypes = [vp, i64, vp, sz, ctypes.POINTER(vp), ctypes.POINTER(i64)]
    L.moe_mk_trace_view.restype = ctypes.c_int
    L.moe_mk_status_str.argtypes = [ctypes.c_int]
    L.moe_mk_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions the C header declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(moe_mk_[a-z_]+)\s*\(", text)))


def moe_mk_status_str(code: int) -> str:
    return lib().moe_mk_status_str(int(code)).decode()


def _check(code: int, what: str):
    if code != MOE_MK_OK:
        raise MoeMkError(what, code)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def moe_mk_plan(E: int, k: int, d: int, f: int, sched: int = MOE_MK_SCHED_STATIC) -> int:
    p = ctypes.c_void_p()
    _check(lib().moe_mk_plan(ctypes.byref(p), E, k, d, f, sched), "moe_mk_plan")
    return p.value


def moe_mk_plan_destroy(plan: int) -> None:
    _SHAPES.pop(plan, None)
    lib().moe_mk_plan_destroy(plan)


def moe_mk_workspace_bytes(plan: int, B: int) -> int:
    return int(lib().moe_mk_workspace_bytes(plan, B))


def moe_mk_workspace_init(plan: int, ws, stream=None) -> None:
    _check(lib().moe_mk_workspace_init(plan, _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_mk_workspace_init")


_SHAPES = {}


def _plan_shape(plan: int):
    """(E, k, d, f) of a plan (cached per plan handle)."""
    sh = _SHAPES.get(plan)
    if sh is None:
        sh = tuple(moe_mk_plan_info(plan, key) for key in ("E", "k", "d", "f"))
        _SHAPES[plan] = sh
    return sh


def _check_shape(t, name, shape):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_forward_args(plan, x, Wr, router_bias, W1, W3, W2, out, B, ws):
    """Shapes and devices of every tensor against the plan's (E, k, d, f) and B; the C ABI
    sees only pointers, so a mis-shaped tensor would be read or written out of bounds."""
    E, k, d, f = _plan_shape(plan)
    if B < 0:
        raise ValueError(f"B must be >= 0, got {B}")
    for t, name in ((x, "x"), (out, "out")):
        if t.dim() != 2 or t.shape[1] != d or t.shape[0] < B:
            raise ValueError(f"{name} must have shape (>= {B}, {d}), got {tuple(t.shape)}")
    _check_shape(Wr, "Wr", (d, E))
    _check_shape(router_bias, "router_bias", (E,))
    _check_shape(W1, "W1", (E, d, f))
    _check_shape(W3, "W3", (E, d, f))
    _check_shape(W2, "W2", (E, f, d))
    devs = {t.device for t in (x, Wr, router_bias, W1, W3, W2, out, ws) if t is not None}
    if len(devs) != 1:
        raise ValueError(f"every tensor must be on one device, got {sorted(str(v) for v in devs)}")


def moe_mk_forward(plan: int, x, Wr, router_bias, W1, W3, W2, out, B: int, ws, stream=None) -> None:
    import torch
    bf = torch.bfloat16
    _check_forward_args(plan, x, Wr, router_bias, W1, W3, W2, out, B, ws)
    _check(lib().moe_mk_forward(plan, _dev_ptr(x, "x", bf), _dev_ptr(Wr, "Wr", torch.float32),
                                _dev_ptr(router_bias, "router_bias", torch.float32), _dev_ptr(W1, "W1", bf),
                                _dev_ptr(W3, "W3", bf), _dev_ptr(W2, "W2", bf), _dev_ptr(out, "out", bf), B,
                                _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_mk_forward")


def moe_mk_forward_unfused(plan: int, x, Wr, router_bias, W1, W3, W2, out, B: int, ws, stream=None) -> None:
    """The layer as seven kernels, one per phase (the launch-per-phase baseline)."""
    import torch
    bf = torch.bfloat16
    _check_forward_args(plan, x, Wr, router_bias, W1, W3, W2, out, B, ws)
    _check(lib().moe_mk_forward_unfused(plan, _dev_ptr(x, "x", bf), _dev_ptr(Wr, "Wr", torch.float32),
                                        _dev_ptr(router_bias, "router_bias", torch.float32), _dev_ptr(W1, "W1", bf),
                                        _dev_ptr(W3, "W3", bf), _dev_ptr(W2, "W2", bf), _dev_ptr(out, "out", bf), B,
                                        _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_mk_forward_unfused")


def moe_mk_forward_noalloc(plan: int, x, Wr, router_bias, W1, W3, W2, out, B: int, err=None, stream=None) -> None:
    """moe_mk_forward on the library's static per-GPU scratch (allocates nothing); ``err``:
    optional int32 device tensor of one element receiving the forward's device error bits."""
    import torch
    bf = torch.bfloat16
    _check_forward_args(plan, x, Wr, router_bias, W1, W3, W2, out, B, err if err is not None else x)
    if err is not None and err.numel() < 1:
        raise ValueError("err must hold one int32")
    _check(lib().moe_mk_forward_noalloc(plan, _dev_ptr(x, "x", bf), _dev_ptr(Wr, "Wr", torch.float32),
                                        _dev_ptr(router_bias, "router_bias", torch.float32), _dev_ptr(W1, "W1", bf),
                                        _dev_ptr(W3, "W3", bf), _dev_ptr(W2, "W2", bf), _dev_ptr(out, "out", bf), B,
                                        _dev_ptr(err, "err", torch.int32), _stream(stream)),
           "moe_mk_forward_noalloc")


def moe_mk_routing_view(plan: int, B: int, ws) -> dict:
    """Views (no copies) of the routing arrays of the last forward with batch size B."""
    import torch
    v = _RoutingView()
    nbytes = ws.numel() * ws.element_size()
    _check(lib().moe_mk_routing_view(plan, B, ws.data_ptr(), nbytes, ctypes.byref(v)), "moe_mk_routing_view")
    E = moe_mk_plan_info(plan, "E")
    k = moe_mk_plan_info(plan, "k")
    raw = ws.view(torch.uint8).reshape(-1)
    base = ws.data_ptr()

    def part(ptr, n, dtype, shape):
        off = ptr - base
        size = n * torch.empty((), dtype=dtype).element_size()
        return raw[off:off + size].view(dtype).reshape(shape)

    return {"topk_idx": part(v.topk_idx, B * k, torch.int32, (B, k)),
            "topk_w": part(v.topk_w, B * k, torch.float32, (B, k)),
            "hist": part(v.hist, E, torch.int32, (E,)),
            "exp_indptr": part(v.exp_indptr, E + 1, torch.int32, (E + 1,)),
            "perm": part(v.perm, B * k, torch.int32, (B * k,)),
            "inv": part(v.inv, B * k, torch.int32, (B * k,)),
            "logits": part(v.logits, B * E, torch.float32, (B, E)),
            "ctl": part(v.ctl, CTL_WORDS, torch.int32, (CTL_WORDS,)),
            "mt_expert": part(v.mt_expert, v.mt_cap, torch.int32, (v.mt_cap,)),
            "mt_row0": part(v.mt_row0, v.mt_cap, torch.int32, (v.mt_cap,)),
            "mt_rows": part(v.mt_rows, v.mt_cap, torch.int32, (v.mt_cap,))}


def moe_mk_trace_view(plan: int, B: int, ws):
    """Device view (int64 [n, 8]) of the task trace of the last traced forward."""
    import torch
    ptr, n = ctypes.c_void_p(), ctypes.c_int64()
    _check(lib().moe_mk_trace_view(plan, B, ws.data_ptr(), ws.numel() * ws.element_size(), ctypes.byref(ptr),
                                   ctypes.byref(n)), "moe_mk_trace_view")
    off = ptr.value - ws.data_ptr()
    raw = ws.view(torch.uint8).reshape(-1)
    return raw[off:off + n.value * 64].view(torch.int64).reshape(n.value, 8)


def moe_mk_workspace_error(plan: int, ws, stream=None) -> int:
    err = ctypes.c_int32()
    _check(lib().moe_mk_workspace_error(plan, ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream),
                                        ctypes.byref(err)), "moe_mk_workspace_error")
    return int(err.value)


def moe_mk_plan_info(plan: int, key: str) -> int:
    v = int(lib().moe_mk_plan_info(plan, key.encode()))
    if v < 0:
        raise KeyError(key)
    return v


def moe_mk_forward_info(plan: int, B: int, key: str) -> int:
    v = int(lib().moe_mk_forward_info(plan, B, key.encode()))
    if v < 0:
        raise KeyError(key)
    return v


def moe_mk_plan_set_debug(plan: int, watchdog_ticks: int = 0, flags: int = 0) -> None:
    _check(lib().moe_mk_plan_set_debug(plan, watchdog_ticks, flags), "moe_mk_plan_set_debug")


class MoELayer:
    """A plan plus a workspace sized for ``max_batch`` tokens, bound to fixed weights."""

    def __init__(self, E, k, d, f, Wr, W1, W3, W2, router_bias=None, sched=MOE_MK_SCHED_STATIC,
                 max_batch: int = 1, device=None):
        import torch
        self.E, self.k, self.d, self.f = E, k, d, f
        self.Wr, self.W1, self.W3, self.W2, self.bias = Wr, W1, W3, W2, router_bias
        for t, name, shape in ((Wr, "Wr", (d, E)), (router_bias, "router_bias", (E,)), (W1, "W1", (E, d, f)),
                               (W3, "W3", (E, d, f)), (W2, "W2", (E, f, d))):
            _check_shape(t, name, shape)
        self.plan = moe_mk_plan(E, k, d, f, sched)
        nbytes = moe_mk_workspace_bytes(self.plan, max(1, max_batch))
        self.ws = torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device or "cuda")
        moe_mk_workspace_init(self.plan, self.ws)
        self.max_batch = max_batch

    def forward(self, x, out=None, stream=None):
        import torch
        if x.dim() != 2 or x.shape[1] != self.d:
            raise ValueError(f"x must have shape (B, {self.d}), got {tuple(x.shape)}")
        B = x.shape[0]
        if B > self.max_batch:
            raise ValueError(f"batch {B} exceeds the workspace capacity {self.max_batch}")
        if out is None:
            out = torch.empty((B, self.d), dtype=torch.bfloat16, device=x.device)
        moe_mk_forward(self.plan, x, self.Wr, self.bias, self.W1, self.W3, self.W2, out, B, self.ws, stream)
        return out

    __call__ = forward

    def forward_unfused(self, x, out=None, stream=None):
        """The same layer as one kernel per phase (the launch-per-phase baseline)."""
        import torch
        if x.dim() != 2 or x.shape[1] != self.d:
            raise ValueError(f"x must have shape (B, {self.d}), got {tuple(x.shape)}")
        B = x.shape[0]
        if B > self.max_batch:
            raise ValueError(f"batch {B} exceeds the workspace capacity {self.max_batch}")
        if out is None:
            out = torch.empty((B, self.d), dtype=torch.bfloat16, device=x.device)
        moe_mk_forward_unfused(self.plan, x, self.Wr, self.bias, self.W1, self.W3, self.W2, out, B, self.ws, stream)
        return out

    def routing(self, B):
        return moe_mk_routing_view(self.plan, B, self.ws)

    def error(self, stream=None) -> int:
        return moe_mk_workspace_error(self.plan, self.ws, stream)

    def reinit(self):
        moe_mk_workspace_init(self.plan, self.ws)

    def close(self):
        if self.plan:
            moe_mk_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
