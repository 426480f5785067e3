"""Python binding of libmoe_mi355x.so, the MI355X post-router MoE layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  The ctypes structures mirror include/moe.h field for field, and the
functions keep the C names.  Torch is used for device memory and the current
stream; helpers at the bottom turn torch tensors into the C descriptors.

The shared library is built in-tree (python -m moe_megakernel_amd.build); if
it is missing, load() raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_LAYOUT = 0, 1, 2, 3, 4
MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_ROUTE_OVERFLOW, MOE_ERR_HIP = 5, 6, 7, 8
MOE_ERR_ROUTE_INVALID = 9
MOE_BF16, MOE_FP32, MOE_MXFP8_E4M3 = 1, 2, 3
MOE_FLAG_HAS_SHARED = 1
MOE_FLAG_RECOMPUTE = 2
MOE_FLAG_TOPK_ROUTING = 4
MOE_FLAG_SHARED_GATE = 8

EXPORTED = ("moe_saved_bytes", "moe_workspace_bytes", "moe_saved_view", "moe_forward",
            "moe_forward_topk", "moe_forward_noalloc", "moe_backward", "moe_status_str",
            "moe_kernel_timer_enable", "moe_kernel_timer_read", "moe_mx_staging_view")
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class moe_problem(C.Structure):
    _fields_ = [("tokens", C.c_int64), ("hidden", C.c_int64), ("intermediate", C.c_int64),
                ("experts", C.c_int32), ("topk", C.c_int32), ("routed_dtype", C.c_int32),
                ("flags", C.c_uint32), ("swiglu_limit", C.c_float)]


class moe_mat(C.Structure):
    _fields_ = [("base", C.c_void_p), ("expert_stride", C.c_int64), ("table", C.c_void_p),
                ("ld", C.c_int64)]


class moe_weight(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("rows", C.c_int64), ("cols", C.c_int64),
                ("row_offset", C.c_int64), ("data", moe_mat), ("scale", moe_mat),
                ("col_data", moe_mat), ("col_scale", moe_mat)]


class moe_weights(C.Structure):
    _fields_ = [(n, moe_weight) for n in ("shared_gate", "shared_up", "shared_down",
                                          "routed_gate", "routed_up", "routed_down", "shared_out_gate")]


class moe_grad(C.Structure):
    _fields_ = [("base", C.c_void_p), ("expert_stride", C.c_int64), ("table", C.c_void_p),
                ("ld", C.c_int64), ("row_offset", C.c_int64), ("dtype", C.c_int32)]


class moe_main_grads(C.Structure):
    _fields_ = [(n, moe_grad) for n in ("shared_gate", "shared_up", "shared_down",
                                        "routed_gate", "routed_up", "routed_down", "shared_out_gate")]


class moe_saved_layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("top_experts", "router_weights", "counts", "offsets",
                                          "slot_of", "slot_token", "status_word")]


class moe_mx_staging_layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("x_codes", "x_scales", "h_codes", "h_scales",
                                          "dy_codes", "dy_scales", "dfc1_codes", "dfc1_scales")]


_lib = None


def load(path: str | None = None):
    """Load the in-tree shared library (raises FileNotFoundError if it was not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} is missing: build it with `python -m moe_megakernel_amd.build`")
    lib = C.CDLL(p)
    P = C.POINTER
    lib.moe_saved_bytes.argtypes = [P(moe_problem)]
    lib.moe_saved_bytes.restype = C.c_size_t
    lib.moe_workspace_bytes.argtypes = [P(moe_problem), C.c_int]
    lib.moe_workspace_bytes.restype = C.c_size_t
    lib.moe_saved_view.argtypes = [P(moe_problem), P(moe_saved_layout)]
    lib.moe_saved_view.restype = C.c_int
    lib.moe_forward.argtypes = [P(moe_problem), C.c_void_p, C.c_void_p, C.c_void_p, P(moe_weights),
                                C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.moe_forward.restype = C.c_int
    lib.moe_forward_topk.argtypes = lib.moe_forward.argtypes
    lib.moe_forward_topk.restype = C.c_int
    lib.moe_forward_noalloc.argtypes = [P(moe_problem), C.c_void_p, C.c_void_p, C.c_void_p, P(moe_weights),
                                        C.c_void_p, C.c_void_p, C.c_void_p]
    lib.moe_forward_noalloc.restype = C.c_int
    lib.moe_backward.argtypes = [P(moe_problem), C.c_void_p, C.c_void_p, P(moe_weights), C.c_void_p,
                                 C.c_void_p, C.c_void_p, P(moe_main_grads), C.c_void_p, C.c_size_t,
                                 C.c_void_p]
    lib.moe_backward.restype = C.c_int
    lib.moe_status_str.argtypes = [C.c_int]
    lib.moe_status_str.restype = C.c_char_p
    lib.moe_kernel_timer_enable.argtypes = [C.c_int]
    lib.moe_kernel_timer_enable.restype = None
    lib.moe_kernel_timer_read.argtypes = [P(C.c_char_p), P(C.c_int), P(C.c_double), C.c_int]
    lib.moe_kernel_timer_read.restype = C.c_int
    lib.moe_mx_staging_view.argtypes = [P(moe_problem), P(moe_mx_staging_layout)]
    lib.moe_mx_staging_view.restype = C.c_int
    if path is None:
        _lib = lib
    return lib


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({moe_status_str(status)})")
        self.status = status


# ------------------------------------------------------------------ C entry points
def moe_status_str(status: int) -> str:
    return load().moe_status_str(int(status)).decode()


def moe_saved_bytes(p: moe_problem) -> int:
    return int(load().moe_saved_bytes(C.byref(p)))


def moe_workspace_bytes(p: moe_problem, for_backward: bool) -> int:
    return int(load().moe_workspace_bytes(C.byref(p), int(bool(for_backward))))


def moe_saved_view(p: moe_problem) -> moe_saved_layout:
    out = moe_saved_layout()
    st = load().moe_saved_view(C.byref(p), C.byref(out))
    if st != MOE_OK:
        raise MoeError(st, "moe_saved_view")
    return out


def moe_mx_staging_view(p: moe_problem) -> moe_mx_staging_layout:
    out = moe_mx_staging_layout()
    st = load().moe_mx_staging_view(C.byref(p), C.byref(out))
    if st != MOE_OK:
        raise MoeError(st, "moe_mx_staging_view")
    return out


def moe_forward(p, hidden, probs, routing_map, weights, out, saved, workspace, workspace_bytes, stream) -> int:
    """Raw call with integer device addresses; returns the status code."""
    return load().moe_forward(C.byref(p), hidden, probs, routing_map, C.byref(weights), out, saved,
                              workspace, workspace_bytes, stream)


def moe_forward_noalloc(p, hidden, probs, routing_map, weights, out, saved, stream) -> int:
    """Raw call of the allocation-free forward (its scratch is the library's static per-GPU
    array); returns the status code."""
    return load().moe_forward_noalloc(C.byref(p), hidden, probs, routing_map, C.byref(weights), out, saved,
                                      stream)


def moe_forward_topk(p, hidden, top_experts, router_weights, weights, out, saved, workspace, workspace_bytes,
                     stream) -> int:
    """Raw call with integer device addresses (routing as the [T][K] table); returns the status."""
    return load().moe_forward_topk(C.byref(p), hidden, top_experts, router_weights, C.byref(weights), out,
                                   saved, workspace, workspace_bytes, stream)


def moe_backward(p, grad_out, hidden, weights, saved, grad_hidden, grad_probs, main_grads, workspace,
                 workspace_bytes, stream) -> int:
    return load().moe_backward(C.byref(p), grad_out, hidden, C.byref(weights), saved, grad_hidden,
                               grad_probs, C.byref(main_grads), workspace, workspace_bytes, stream)


def moe_kernel_timer_enable(on: bool) -> None:
    load().moe_kernel_timer_enable(int(bool(on)))


def moe_kernel_timer_read(cap: int = 64) -> dict:
    """{kernel name: (launches, total ms)} since the previous read."""
    names = (C.c_char_p * cap)()
    cnt = (C.c_int * cap)()
    ms = (C.c_double * cap)()
    n = load().moe_kernel_timer_read(names, cnt, ms, cap)
    return {names[i].decode(): (cnt[i], ms[i]) for i in range(min(n, cap))}


# ------------------------------------------------------------------ torch helpers
def problem(tokens, hidden, inter, experts, topk, routed_dtype=MOE_BF16, flags=MOE_FLAG_HAS_SHARED,
            swiglu_limit=0.0) -> moe_problem:
    return moe_problem(tokens, hidden, inter, experts, topk, routed_dtype, flags, swiglu_limit)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def mat(base=None, expert_stride=0, table=None, ld=0) -> moe_mat:
    """base/table: torch tensors (table: int64 device tensor of per-expert addresses)."""
    return moe_mat(_ptr(base), int(expert_stride), _ptr(table), int(ld))


def weight(dtype, rows, cols, data: moe_mat, row_offset=0, scale=None, col_data=None,
           col_scale=None) -> moe_weight:
    z = moe_mat(0, 0, 0, 0)
    return moe_weight(dtype, rows, cols, row_offset, data, scale or z, col_data or z, col_scale or z)


def grad(base=None, expert_stride=0, table=None, ld=0, row_offset=0, dtype=None) -> moe_grad:
    """main_grad view; dtype defaults to the tensor's (torch.float32 -> MOE_FP32,
    torch.bfloat16 -> MOE_BF16), else MOE_FP32."""
    if dtype is None:
        dtype = MOE_FP32
        t = base if base is not None else None
        if t is not None and hasattr(t, "dtype"):
            import torch
            dtype = MOE_BF16 if t.dtype == torch.bfloat16 else MOE_FP32
    return moe_grad(_ptr(base), int(expert_stride), _ptr(table), int(ld), int(row_offset), int(dtype))


def current_stream() -> int:
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


class Layer:
    """Caller-side convenience: holds the problem, the caller-owned `saved` and
    workspace tensors (allocated once with torch), and issues the two C calls
    on torch's current stream.  Raises MoeError on a non-OK status."""

    def __init__(self, p: moe_problem, device="cuda"):
        import torch
        self.p = p
        self.saved = torch.empty(max(moe_saved_bytes(p), 256), dtype=torch.uint8, device=device)
        fw = max(moe_workspace_bytes(p, False), 256)
        bw = max(moe_workspace_bytes(p, True), 256)
        self.ws_bytes = max(fw, bw)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        if moe_saved_bytes(p) == 0:
            raise MoeError(MOE_ERR_SHAPE, "moe_saved_bytes")

    def forward(self, hidden, probs, routing_map, weights: moe_weights, out):
        st = moe_forward(self.p, _ptr(hidden), _ptr(probs), _ptr(routing_map), weights, _ptr(out),
                         _ptr(self.saved), _ptr(self.workspace), self.ws_bytes, current_stream())
        if st != MOE_OK:
            raise MoeError(st, "moe_forward")
        return out

    def forward_noalloc(self, hidden, probs, routing_map, weights: moe_weights, out):
        """moe_forward_noalloc into this layer's `saved` (no workspace is passed)."""
        st = moe_forward_noalloc(self.p, _ptr(hidden), _ptr(probs), _ptr(routing_map), weights, _ptr(out),
                                 _ptr(self.saved), current_stream())
        if st != MOE_OK:
            raise MoeError(st, "moe_forward_noalloc")
        return out

    def forward_topk(self, hidden, top_experts, router_weights, weights: moe_weights, out):
        st = moe_forward_topk(self.p, _ptr(hidden), _ptr(top_experts), _ptr(router_weights), weights,
                              _ptr(out), _ptr(self.saved), _ptr(self.workspace), self.ws_bytes,
                              current_stream())
        if st != MOE_OK:
            raise MoeError(st, "moe_forward_topk")
        return out

    def backward(self, grad_out, hidden, weights: moe_weights, grad_hidden, grad_probs,
                 main_grads: moe_main_grads):
        st = moe_backward(self.p, _ptr(grad_out), _ptr(hidden), weights, _ptr(self.saved),
                          _ptr(grad_hidden), _ptr(grad_probs), main_grads, _ptr(self.workspace),
                          self.ws_bytes, current_stream())
        if st != MOE_OK:
            raise MoeError(st, "moe_backward")

    def routing_state(self):
        """Integer routing state from `saved` as torch views (device)."""
        import torch
        L = moe_saved_view(self.p)
        T, K, E = self.p.tokens, self.p.topk, self.p.experts

        def view(off, n, dt):
            nbytes = n * 4
            return self.saved[off:off + nbytes].view(dt)
        return {
            "top_experts": view(L.top_experts, T * K, torch.int32).view(T, K),
            "router_weights": view(L.router_weights, T * K, torch.float32).view(T, K),
            "counts": view(L.counts, E, torch.int32),
            "offsets": view(L.offsets, E + 1, torch.int32),
            "slot_of": view(L.slot_of, T * K, torch.int32).view(T, K),
            "slot_token": view(L.slot_token, T * K, torch.int32),
            "status_word": view(L.status_word, 1, torch.int32),
        }
