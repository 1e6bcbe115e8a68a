"""w4a4_rank_gemm_amd -- the fused W4A4 + low-rank linear of TwinQuant on MI355X.

A thin ctypes binding of libtwq (include/twq.h): it checks tensor dtypes and
devices, allocates outputs with torch on the input's device, and passes raw
pointers and the current HIP stream. Every step of the layer runs in the HIP
kernels of libtwq; there is no fallback. If libtwq.so has not been built, or no
GPU is present, the calls raise.

    Y = s_X s_W (Q_X Q_W) + (X L1) L2

(TwinQuant, page 1, section 2, eqs. (1)-(3); fused as in page 1, section 4.3.)
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libtwq.so")

TWQ_OK = 0
STATUS_NAMES = {0: "TWQ_OK", 1: "TWQ_ERR_NULL", 2: "TWQ_ERR_SHAPE", 3: "TWQ_ERR_ALIGN",
                4: "TWQ_ERR_UNSUPPORTED", 5: "TWQ_ERR_HIP", 6: "TWQ_ERR_WORKSPACE"}

# every symbol include/twq.h declares
EXPORTS = ("twq_status_string", "twq_last_error_string", "twq_last_hip_error", "twq_version",
           "twq_quantize_act_workspace_bytes", "twq_quantize_act", "twq_pack_weight",
           "twq_dual_linear", "twq_debug_residual_acc", "twq_linear_workspace_bytes",
           "twq_linear", "twq_quantize_act_grouped", "twq_pack_weight_grouped", "twq_dual_linear_grouped",
           "twq_linear_grouped_workspace_bytes", "twq_linear_grouped", "twq_quantize_act_a8",
           "twq_dual_linear_a8", "twq_linear_a8_workspace_bytes", "twq_linear_a8", "twq_debug_residual_acc_a8",
           "twq_pack_lowrank_int4",
           "twq_quantize_act_lr4", "twq_debug_lr4_h", "twq_dual_linear_lr4", "twq_linear_lr4_workspace_bytes",
           "twq_linear_lr4", "twq_debug_linear_lr4_main", "twq_debug_linear_main",
           "twq_debug_linear_grouped_main", "twq_debug_linear_a8_main", "twq_linear_noalloc_max_bytes",
           "twq_linear_noalloc", "twq_fold_workspace_bytes", "twq_fold_lowrank")

GROUP = 128  # group size of the group-wise entry points


class TwqError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = f"{where}: {STATUS_NAMES.get(status, status)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


_lib = None
_lock = threading.Lock()
_P, _I, _S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded libtwq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(f"libtwq.so is not built ({LIB_PATH}); run "
                                      "`python -m w4a4_rank_gemm_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                L.twq_status_string.restype = ctypes.c_char_p
                L.twq_status_string.argtypes = [ctypes.c_int]
                L.twq_last_error_string.restype = ctypes.c_char_p
                L.twq_last_error_string.argtypes = []
                L.twq_last_hip_error.restype = ctypes.c_char_p
                L.twq_last_hip_error.argtypes = []
                L.twq_version.restype = ctypes.c_int
                L.twq_quantize_act_workspace_bytes.restype = _S
                L.twq_quantize_act_workspace_bytes.argtypes = [_I, _I, _I]
                L.twq_quantize_act.restype = ctypes.c_int
                L.twq_quantize_act.argtypes = [_P, _I, _I, _P, _P, _P, _I, _P, _P, _S, _P]
                L.twq_pack_weight.restype = ctypes.c_int
                L.twq_pack_weight.argtypes = [_P, _I, _I, _P, _P, _P]
                L.twq_dual_linear.restype = ctypes.c_int
                L.twq_dual_linear.argtypes = [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P]
                L.twq_debug_residual_acc.restype = ctypes.c_int
                L.twq_debug_residual_acc.argtypes = [_P, _P, _P, _I, _I, _I, _P]
                L.twq_linear_workspace_bytes.restype = _S
                L.twq_linear_workspace_bytes.argtypes = [_I, _I, _I, _I]
                L.twq_linear.restype = ctypes.c_int
                L.twq_linear.argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _S, _P]
                L.twq_quantize_act_grouped.restype = ctypes.c_int
                L.twq_quantize_act_grouped.argtypes = [_P, _I, _I, _I, _P, _P, _P, _I, _P, _P, _S, _P]
                L.twq_pack_weight_grouped.restype = ctypes.c_int
                L.twq_pack_weight_grouped.argtypes = [_P, _I, _I, _I, _P, _P, _P]
                L.twq_dual_linear_grouped.restype = ctypes.c_int
                L.twq_dual_linear_grouped.argtypes = [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _P]
                L.twq_linear_grouped_workspace_bytes.restype = _S
                L.twq_linear_grouped_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
                L.twq_linear_grouped.restype = ctypes.c_int
                L.twq_linear_grouped.argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _P, _S, _P]
                L.twq_quantize_act_a8.restype = ctypes.c_int
                L.twq_quantize_act_a8.argtypes = [_P, _I, _I, _P, _P, _P, _I, _P, _P, _S, _P]
                L.twq_dual_linear_a8.restype = ctypes.c_int
                L.twq_dual_linear_a8.argtypes = [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P]
                L.twq_linear_a8_workspace_bytes.restype = _S
                L.twq_linear_a8_workspace_bytes.argtypes = [_I, _I, _I, _I]
                L.twq_linear_a8.restype = ctypes.c_int
                L.twq_linear_a8.argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _S, _P]
                L.twq_debug_residual_acc_a8.restype = ctypes.c_int
                L.twq_debug_residual_acc_a8.argtypes = [_P, _P, _P, _I, _I, _I, _P]
                L.twq_pack_lowrank_int4.restype = ctypes.c_int
                L.twq_pack_lowrank_int4.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P]
                L.twq_quantize_act_lr4.restype = ctypes.c_int
                L.twq_quantize_act_lr4.argtypes = [_P, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P]
                L.twq_debug_lr4_h.restype = ctypes.c_int
                L.twq_debug_lr4_h.argtypes = [_P, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P]
                L.twq_linear_lr4_workspace_bytes.restype = _S
                L.twq_linear_lr4_workspace_bytes.argtypes = [_I, _I, _I, _I]
                for nm in ("twq_linear_lr4", "twq_debug_linear_lr4_main"):
                    getattr(L, nm).restype = ctypes.c_int
                    getattr(L, nm).argtypes = [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _S, _P]
                L.twq_dual_linear_lr4.restype = ctypes.c_int
                L.twq_dual_linear_lr4.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P]
                for nm in ("twq_debug_linear_main", "twq_debug_linear_a8_main"):
                    getattr(L, nm).restype = ctypes.c_int
                    getattr(L, nm).argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _S, _P]
                L.twq_fold_workspace_bytes.restype = _S
                L.twq_fold_workspace_bytes.argtypes = [_I, _I, _I]
                L.twq_fold_lowrank.restype = ctypes.c_int
                L.twq_fold_lowrank.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _S, _P]
                L.twq_linear_noalloc_max_bytes.restype = _S
                L.twq_linear_noalloc_max_bytes.argtypes = []
                L.twq_linear_noalloc.restype = ctypes.c_int
                L.twq_linear_noalloc.argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P]
                L.twq_debug_linear_grouped_main.restype = ctypes.c_int
                L.twq_debug_linear_grouped_main.argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _P, _S, _P]
                _lib = L
    return _lib


def _check(status: int, where: str):
    if status != TWQ_OK:
        detail = lib().twq_last_error_string().decode() if status == 5 else ""
        raise TwqError(status, where, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# One workspace per (device, stream): calls sharing a workspace must not overlap,
# and calls enqueued on one stream never do. New workspaces start zeroed.
_workspaces: dict = {}


def _workspace(dev: torch.device, nbytes: int):
    if nbytes == 0:
        return None, 0
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws, ws.numel()


def quantize_act(x: torch.Tensor, l1t: torch.Tensor | None = None):
    """X fp16 [b][m] -> (Q_X u8 [b][m/2], s_X f32 [b], T f32 [b][r] or None)."""
    _need(x, "x", torch.float16, 2)
    b, m = x.shape
    r = 0
    if l1t is not None:
        _need(l1t, "l1t", torch.float16, 2)
        r = l1t.shape[0]
        if l1t.shape[1] != m or l1t.device != x.device:
            raise ValueError("l1t must be [r][m] on x's device")
    dev = x.device
    qx = torch.empty((b, m // 2), dtype=torch.uint8, device=dev)
    sx = torch.empty((b,), dtype=torch.float32, device=dev)
    t = torch.empty((b, r), dtype=torch.float32, device=dev) if r else None
    L = lib()
    ws, wsb = _workspace(dev, L.twq_quantize_act_workspace_bytes(b, m, r))
    _check(L.twq_quantize_act(_ptr(x), b, m, _ptr(qx), _ptr(sx), _ptr(l1t), r, _ptr(t),
                              _ptr(ws), wsb, _stream(dev)), "twq_quantize_act")
    return qx, sx, t


def pack_weight(w_res: torch.Tensor):
    """W_res f32 [n][m] -> (Q_W u8 [n][m/2], s_W f32 [n]).

    Q_W's n*m/2 bytes are in the library's 16-channel panel layout (twq.h), not one
    channel per row: the tensor's shape only records n and m."""
    _need(w_res, "w_res", torch.float32, 2)
    n, m = w_res.shape
    dev = w_res.device
    qw = torch.empty((n, m // 2), dtype=torch.uint8, device=dev)
    sw = torch.empty((n,), dtype=torch.float32, device=dev)
    _check(lib().twq_pack_weight(_ptr(w_res), n, m, _ptr(qw), _ptr(sw), _stream(dev)),
           "twq_pack_weight")
    return qw, sw


def dual_linear(qx, sx, qw, sw, t=None, l2t=None, out: torch.Tensor | None = None):
    """The fused layer: Y fp16 [b][n] from the packed operands and the low-rank pair."""
    _need(qx, "qx", torch.uint8, 2)
    _need(qw, "qw", torch.uint8, 2)
    _need(sx, "sx", torch.float32, 1)
    _need(sw, "sw", torch.float32, 1)
    b, kb = qx.shape
    n = qw.shape[0]
    m = 2 * kb
    if qw.shape[1] != kb or sx.shape[0] != b or sw.shape[0] != n:
        raise ValueError("inconsistent shapes of qx/sx/qw/sw")
    r = 0
    if l2t is not None or t is not None:
        _need(t, "t", torch.float32, 2)
        _need(l2t, "l2t", torch.float16, 2)
        r = l2t.shape[1]
        if t.shape != (b, r) or l2t.shape[0] != n:
            raise ValueError("t must be [b][r] and l2t [n][r]")
    dev = qx.device
    for name, ten in (("sx", sx), ("qw", qw), ("sw", sw), ("t", t), ("l2t", l2t)):
        if ten is not None and ten.device != dev:
            raise ValueError(f"{name} is on {ten.device}, qx on {dev}")
    y = out if out is not None else torch.empty((b, n), dtype=torch.float16, device=dev)
    _need(y, "out", torch.float16, 2)
    if y.shape != (b, n):
        raise ValueError("out must be [b][n]")
    _check(lib().twq_dual_linear(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(t), _ptr(l2t), r,
                                 _ptr(y), b, m, n, _stream(dev)), "twq_dual_linear")
    return y


def linear(x: torch.Tensor, qw, sw, l1t=None, l2t=None, out: torch.Tensor | None = None):
    """The whole layer in one call (twq_linear): Y fp16 [b][n] from fp16 X, the packed
    residual weight and the fp16 low-rank pair; Q_X, s_X and T live in the workspace."""
    _need(x, "x", torch.float16, 2)
    _need(qw, "qw", torch.uint8, 2)
    _need(sw, "sw", torch.float32, 1)
    b, m = x.shape
    n = qw.shape[0]
    if qw.shape[1] != m // 2 or sw.shape[0] != n:
        raise ValueError("inconsistent shapes of x/qw/sw")
    r = 0
    if l1t is not None or l2t is not None:
        _need(l1t, "l1t", torch.float16, 2)
        _need(l2t, "l2t", torch.float16, 2)
        r = l1t.shape[0]
        if l1t.shape[1] != m or l2t.shape != (n, r):
            raise ValueError("l1t must be [r][m] and l2t [n][r]")
    dev = x.device
    for name, ten in (("qw", qw), ("sw", sw), ("l1t", l1t), ("l2t", l2t)):
        if ten is not None and ten.device != dev:
            raise ValueError(f"{name} is on {ten.device}, x on {dev}")
    y = out if out is not None else torch.empty((b, n), dtype=torch.float16, device=dev)
    _need(y, "out", torch.float16, 2)
    if y.shape != (b, n):
        raise ValueError("out must be [b][n]")
    L = lib()
    ws, wsb = _workspace(dev, L.twq_linear_workspace_bytes(b, m, n, r))
    _check(L.twq_linear(_ptr(x), _ptr(qw), _ptr(sw), _ptr(l1t), _ptr(l2t), r, _ptr(y), b, m, n,
                        _ptr(ws), wsb, _stream(dev)), "twq_linear")
    return y


def linear_noalloc(x: torch.Tensor, qw, sw, l1t=None, l2t=None, out: torch.Tensor | None = None):
    """twq_linear_noalloc: the one-call layer on the library's own per-GPU scratch array
    (no workspace, no allocation inside the call). Only `out`, if not given, is allocated
    here, before the call; pass `out` to allocate nothing. Calls that may overlap on one
    GPU share the scratch and must be serialized by the caller."""
    _need(x, "x", torch.float16, 2)
    _need(qw, "qw", torch.uint8, 2)
    _need(sw, "sw", torch.float32, 1)
    b, m = x.shape
    n = qw.shape[0]
    if qw.shape[1] != m // 2 or sw.shape[0] != n:
        raise ValueError("inconsistent shapes of x/qw/sw")
    r = 0
    if l1t is not None or l2t is not None:
        _need(l1t, "l1t", torch.float16, 2)
        _need(l2t, "l2t", torch.float16, 2)
        r = l1t.shape[0]
        if l1t.shape[1] != m or l2t.shape != (n, r):
            raise ValueError("l1t must be [r][m] and l2t [n][r]")
    dev = x.device
    for name, ten in (("qw", qw), ("sw", sw), ("l1t", l1t), ("l2t", l2t)):
        if ten is not None and ten.device != dev:
            raise ValueError(f"{name} is on {ten.device}, x on {dev}")
    y = out if out is not None else torch.empty((b, n), dtype=torch.float16, device=dev)
    _need(y, "out", torch.float16, 2)
    if y.shape != (b, n):
        raise ValueError("out must be [b][n]")
    with torch.cuda.device(dev):
        _check(lib().twq_linear_noalloc(_ptr(x), _ptr(qw), _ptr(sw), _ptr(l1t), _ptr(l2t), r, _ptr(y), b, m, n,
                                        _stream(dev)), "twq_linear_noalloc")
    return y


# ---- group-wise scales (groups of GROUP along K; scales group-major) ----

def quantize_act_grouped(x: torch.Tensor, l1t: torch.Tensor | None = None, g: int = GROUP):
    """X fp16 [b][m] -> (Q_X u8 [b][m/2], s_X f32 [m/g][b], T f32 [b][r] or None)."""
    _need(x, "x", torch.float16, 2)
    b, m = x.shape
    r = 0
    if l1t is not None:
        _need(l1t, "l1t", torch.float16, 2)
        r = l1t.shape[0]
        if l1t.shape[1] != m or l1t.device != x.device:
            raise ValueError("l1t must be [r][m] on x's device")
    dev = x.device
    qx = torch.empty((b, m // 2), dtype=torch.uint8, device=dev)
    sx = torch.empty((m // g, b), dtype=torch.float32, device=dev)
    t = torch.empty((b, r), dtype=torch.float32, device=dev) if r else None
    L = lib()
    ws, wsb = _workspace(dev, L.twq_quantize_act_workspace_bytes(b, m, r))
    _check(L.twq_quantize_act_grouped(_ptr(x), b, m, g, _ptr(qx), _ptr(sx), _ptr(l1t), r, _ptr(t),
                                      _ptr(ws), wsb, _stream(dev)), "twq_quantize_act_grouped")
    return qx, sx, t


def pack_weight_grouped(w_res: torch.Tensor, g: int = GROUP):
    """W_res f32 [n][m] -> (Q_W u8 [n][m/2] in the panel layout, s_W f32 [m/g][n])."""
    _need(w_res, "w_res", torch.float32, 2)
    n, m = w_res.shape
    dev = w_res.device
    qw = torch.empty((n, m // 2), dtype=torch.uint8, device=dev)
    sw = torch.empty((m // g, n), dtype=torch.float32, device=dev)
    _check(lib().twq_pack_weight_grouped(_ptr(w_res), n, m, g, _ptr(qw), _ptr(sw), _stream(dev)),
           "twq_pack_weight_grouped")
    return qw, sw


def dual_linear_grouped(qx, sx, qw, sw, t=None, l2t=None, out: torch.Tensor | None = None, g: int = GROUP):
    """The fused layer with group-wise scales: Y fp16 [b][n]."""
    _need(qx, "qx", torch.uint8, 2)
    _need(qw, "qw", torch.uint8, 2)
    _need(sx, "sx", torch.float32, 2)
    _need(sw, "sw", torch.float32, 2)
    b, kb = qx.shape
    n = qw.shape[0]
    m = 2 * kb
    if qw.shape[1] != kb or sx.shape != (m // g, b) or sw.shape != (m // g, n):
        raise ValueError("inconsistent shapes of qx/sx/qw/sw")
    r = 0
    if l2t is not None or t is not None:
        _need(t, "t", torch.float32, 2)
        _need(l2t, "l2t", torch.float16, 2)
        r = l2t.shape[1]
        if t.shape != (b, r) or l2t.shape[0] != n:
            raise ValueError("t must be [b][r] and l2t [n][r]")
    dev = qx.device
    y = out if out is not None else torch.empty((b, n), dtype=torch.float16, device=dev)
    _need(y, "out", torch.float16, 2)
    if y.shape != (b, n):
        raise ValueError("out must be [b][n]")
    _check(lib().twq_dual_linear_grouped(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(t), _ptr(l2t), r,
                                         _ptr(y), b, m, n, g, _stream(dev)), "twq_dual_linear_grouped")
    return y


def linear_grouped(x: torch.Tensor, qw, sw, l1t=None, l2t=None, out: torch.Tensor | None = None, g: int = GROUP):
    """The whole group-wise layer in one call (twq_linear_grouped): Y fp16 [b][n]."""
    _need(x, "x", torch.float16, 2)
    _need(qw, "qw", torch.uint8, 2)
    _need(sw, "sw", torch.float32, 2)
    b, m = x.shape
    n = qw.shape[0]
    if qw.shape[1] != m // 2 or sw.shape != (m // g, n):
        raise ValueError("inconsistent shapes of x/qw/sw")
    r = 0
    if l1t is not None or l2t is not None:
        _need(l1t, "l1t", torch.float16, 2)
        _need(l2t, "l2t", torch.float16, 2)
        r = l1t.shape[0]
        if l1t.shape[1] != m or l2t.shape != (n, r):
            raise ValueError("l1t must be [r][m] and l2t [n][r]")
    dev = x.device
    y = out if out is not None else torch.empty((b, n), dtype=torch.float16, device=dev)
    _need(y, "out", torch.float16, 2)
    if y.shape != (b, n):
        raise ValueError("out must be [b][n]")
    L = lib()
    ws, wsb = _workspace(dev, L.twq_linear_grouped_workspace_bytes(b, m, n, r, g))
    _check(L.twq_linear_grouped(_ptr(x), _ptr(qw), _ptr(sw), _ptr(l1t), _ptr(l2t), r, _ptr(y), b, m, n, g,
                                _ptr(ws), wsb, _stream(dev)), "twq_linear_grouped")
    return y


# ---- W4A8: 8-bit activation codes (int8 [b][m]), 4-bit residual weight ----

def quantize_act_a8(x: torch.Tensor, l1t: torch.Tensor | None = None):
    """X fp16 [b][m] -> (Q_X int8 [b][m], s_X f32 [b], T f32 [b][r] or None)."""
    _need(x, "x", torch.float16, 2)
    b, m = x.shape
    r = 0
    if l1t is not None:
        _need(l1t, "l1t", torch.float16, 2)
        r = l1t.shape[0]
        if l1t.shape[1] != m or l1t.device != x.device:
            raise ValueError("l1t must be [r][m] on x's device")
    dev = x.device
    qx = torch.empty((b, m), dtype=torch.int8, device=dev)
    sx = torch.empty((b,), dtype=torch.float32, device=dev)
    t = torch.empty((b, r), dtype=torch.float32, device=dev) if r else None
    L = lib()
    ws, wsb = _workspace(dev, L.twq_quantize_act_workspace_bytes(b, m, r))
    _check(L.twq_quantize_act_a8(_ptr(x), b, m, _ptr(qx), _ptr(sx), _ptr(l1t), r, _ptr(t),
                                 _ptr(ws), wsb, _stream(dev)), "twq_quantize_act_a8")
    return qx, sx, t


def dual_linear_a8(qx, sx, qw, sw, t=None, l2t=None, out: torch.Tensor | None = None):
    """The fused W4A8 layer: Y fp16 [b][n]."""
    _need(qx, "qx", torch.int8, 2)
    _need(qw, "qw", torch.uint8, 2)
    _need(sx, "sx", torch.float32, 1)
    _need(sw, "sw", torch.float32, 1)
    b, m = qx.shape
    n = qw.shape[0]
    if qw.shape[1] != m // 2 or sx.shape[0] != b or sw.shape[0] != n:
        raise ValueError("inconsistent shapes of qx/sx/qw/sw")
    r = 0
    if l2t is not None or t is not None:
        _need(t, "t", torch.float32, 2)
        _need(l2t, "l2t", torch.float16, 2)
        r = l2t.shape[1]
        if t.shape != (b, r) or l2t.shape[0] != n:
            raise ValueError("t must be [b][r] and l2t [n][r]")
    dev = qx.device
    y = out if out is not None else torch.empty((b, n), dtype=torch.float16, device=dev)
    _need(y, "out", torch.float16, 2)
    if y.shape != (b, n):
        raise ValueError("out must be [b][n]")
    _check(lib().twq_dual_linear_a8(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(t), _ptr(l2t), r,
                                    _ptr(y), b, m, n, _stream(dev)), "twq_dual_linear_a8")
    return y


def linear_a8(x: torch.Tensor, qw, sw, l1t=None, l2t=None, out: torch.Tensor | None = None):
    """The whole W4A8 layer in one call (twq_linear_a8): Y fp16 [b][n]."""
    _need(x, "x", torch.float16, 2)
    _need(qw, "qw", torch.uint8, 2)
    _need(sw, "sw", torch.float32, 1)
    b, m = x.shape
    n = qw.shape[0]
    if qw.shape[1] != m // 2 or sw.shape[0] != n:
        raise ValueError("inconsistent shapes of x/qw/sw")
    r = 0
    if l1t is not None or l2t is not None:
        _need(l1t, "l1t", torch.float16, 2)
        _need(l2t, "l2t", torch.float16, 2)
        r = l1t.shape[0]
        if l1t.shape[1] != m or l2t.shape != (n, r):
            raise ValueError("l1t must be [r][m] and l2t [n][r]")
    dev = x.device
    y = out if out is not None else torch.empty((b, n), dtype=torch.float16, device=dev)
    _need(y, "out", torch.float16, 2)
    if y.shape != (b, n):
        raise ValueError("out must be [b][n]")
    L = lib()
    ws, wsb = _workspace(dev, L.twq_linear_a8_workspace_bytes(b, m, n, r))
    _check(L.twq_linear_a8(_ptr(x), _ptr(qw), _ptr(sw), _ptr(l1t), _ptr(l2t), r, _ptr(y), b, m, n,
                           _ptr(ws), wsb, _stream(dev)), "twq_linear_a8")
    return y


def debug_residual_acc_a8(qx, qw):
    """int32 [b][n] = Q_X (8-bit) . Q_W^T (4-bit) computed by the W4A8 main loop."""
    _need(qx, "qx", torch.int8, 2)
    _need(qw, "qw", torch.uint8, 2)
    b, m = qx.shape
    n = qw.shape[0]
    acc = torch.empty((b, n), dtype=torch.int32, device=qx.device)
    _check(lib().twq_debug_residual_acc_a8(_ptr(qx), _ptr(qw), _ptr(acc), b, m, n, _stream(qx.device)),
           "twq_debug_residual_acc_a8")
    return acc


def debug_residual_acc(qx, qw):
    """int32 [b][n] = Q_X . Q_W^T computed by the fused kernel's main loop."""
    _need(qx, "qx", torch.uint8, 2)
    _need(qw, "qw", torch.uint8, 2)
    b, kb = qx.shape
    n = qw.shape[0]
    acc = torch.empty((b, n), dtype=torch.int32, device=qx.device)
    _check(lib().twq_debug_residual_acc(_ptr(qx), _ptr(qw), _ptr(acc), b, 2 * kb, n,
                                        _stream(qx.device)), "twq_debug_residual_acc")
    return acc


def pack_lowrank_int4(l1t: torch.Tensor, l2t: torch.Tensor):
    """fp16 L1^T [r][m], L2^T [n][r] -> dict ql1 [r][m/2], sl1 [r], ql2 [n][r/2], sl2 [r], c [r].

    ql1 is in the panel layout of pack_weight (it is the weight operand of H = Q_X Q_L1^T)."""
    _need(l1t, "l1t", torch.float16, 2)
    _need(l2t, "l2t", torch.float16, 2)
    r, m = l1t.shape
    n = l2t.shape[0]
    if l2t.shape[1] != r:
        raise ValueError("l2t must be [n][r]")
    dev = l1t.device
    out = {"ql1": torch.empty((r, m // 2), dtype=torch.uint8, device=dev),
           "sl1": torch.empty((r,), dtype=torch.float32, device=dev),
           "ql2": torch.empty((n, r // 2), dtype=torch.uint8, device=dev),
           "sl2": torch.empty((r,), dtype=torch.float32, device=dev),
           "c": torch.empty((r,), dtype=torch.float32, device=dev)}
    _check(lib().twq_pack_lowrank_int4(_ptr(l1t), _ptr(l2t), r, m, n, _ptr(out["ql1"]), _ptr(out["sl1"]),
                                       _ptr(out["ql2"]), _ptr(out["sl2"]), _ptr(out["c"]), _stream(dev)),
           "twq_pack_lowrank_int4")
    return out


def quantize_act_lr4(x: torch.Tensor, lp: dict, debug_h: bool = False):
    """X fp16 [b][m] and the packed int4 factors (pack_lowrank_int4) -> (Q_X u8 [b][m/2],
    s_X f32 [b], Q_H u8 [b][r/2], s_H f32 [b]); H = Q_X Q_L1^T is requantized on chip.
    debug_h: through the test export twq_debug_lr4_h, which also returns the int32 H."""
    _need(x, "x", torch.float16, 2)
    ql1, c = lp["ql1"], lp["c"]
    _need(ql1, "ql1", torch.uint8, 2)
    _need(c, "c", torch.float32, 1)
    b, m = x.shape
    r = ql1.shape[0]
    if ql1.shape[1] != m // 2 or c.shape[0] != r:
        raise ValueError("ql1 must be [r][m/2] and c [r]")
    dev = x.device
    qx = torch.empty((b, m // 2), dtype=torch.uint8, device=dev)
    sx = torch.empty((b,), dtype=torch.float32, device=dev)
    qh = torch.empty((b, r // 2), dtype=torch.uint8, device=dev)
    sh = torch.empty((b,), dtype=torch.float32, device=dev)
    if debug_h:
        h = torch.empty((b, r), dtype=torch.int32, device=dev)
        _check(lib().twq_debug_lr4_h(_ptr(x), b, m, _ptr(ql1), _ptr(c), r, _ptr(h), _ptr(qx), _ptr(sx), _ptr(qh),
                                     _ptr(sh), _stream(dev)), "twq_debug_lr4_h")
        return qx, sx, qh, sh, h
    _check(lib().twq_quantize_act_lr4(_ptr(x), b, m, _ptr(ql1), _ptr(c), r, _ptr(qx), _ptr(sx), _ptr(qh), _ptr(sh),
                                      _stream(dev)), "twq_quantize_act_lr4")
    return qx, sx, qh, sh


def linear_lr4(x: torch.Tensor, qw, sw, lp: dict, out: torch.Tensor | None = None):
    """The whole layer with the int4 low-rank branch in one call (twq_linear_lr4)."""
    _need(x, "x", torch.float16, 2)
    _need(qw, "qw", torch.uint8, 2)
    _need(sw, "sw", torch.float32, 1)
    b, m = x.shape
    n = qw.shape[0]
    ql1, c, ql2 = lp["ql1"], lp["c"], lp["ql2"]
    r = ql1.shape[0]
    if qw.shape[1] != m // 2 or sw.shape[0] != n or ql1.shape[1] != m // 2 or ql2.shape != (n, r // 2):
        raise ValueError("inconsistent shapes of x/qw/sw/ql1/ql2")
    dev = x.device
    y = out if out is not None else torch.empty((b, n), dtype=torch.float16, device=dev)
    _need(y, "out", torch.float16, 2)
    L = lib()
    ws, wsb = _workspace(dev, L.twq_linear_lr4_workspace_bytes(b, m, n, r))
    _check(L.twq_linear_lr4(_ptr(x), _ptr(qw), _ptr(sw), _ptr(ql1), _ptr(c), _ptr(ql2), r, _ptr(y), b, m, n,
                            _ptr(ws), wsb, _stream(dev)), "twq_linear_lr4")
    return y


def dual_linear_lr4(qx, sx, qw, sw, qh, sh, ql2, out: torch.Tensor | None = None):
    """The fused layer with the int4 low-rank branch: Y fp16 [b][n]."""
    for name, t, dt in (("qx", qx, torch.uint8), ("qw", qw, torch.uint8), ("qh", qh, torch.uint8),
                        ("ql2", ql2, torch.uint8)):
        _need(t, name, dt, 2)
    _need(sx, "sx", torch.float32, 1)
    _need(sw, "sw", torch.float32, 1)
    _need(sh, "sh", torch.float32, 1)
    b, kb = qx.shape
    n = qw.shape[0]
    r = 2 * qh.shape[1]
    if ql2.shape != (n, r // 2) or sh.shape[0] != b:
        raise ValueError("qh must be [b][r/2], ql2 [n][r/2], sh [b]")
    y = out if out is not None else torch.empty((b, n), dtype=torch.float16, device=qx.device)
    _check(lib().twq_dual_linear_lr4(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(qh), _ptr(sh), _ptr(ql2), r,
                                     _ptr(y), b, 2 * kb, n, _stream(qx.device)), "twq_dual_linear_lr4")
    return y


class DualLinear:
    """A packed layer: Q_W, s_W and the fp16 low-rank pair, resident on one GPU."""

    def __init__(self, w_res: torch.Tensor, l1t: torch.Tensor | None, l2t: torch.Tensor | None):
        self.qw, self.sw = pack_weight(w_res)
        self.l1t = l1t
        self.l2t = l2t
        self.n, self.m = w_res.shape
        self.r = 0 if l1t is None else l1t.shape[0]

    def __call__(self, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        return linear(x, self.qw, self.sw, self.l1t if self.r else None, self.l2t if self.r else None, out=out)
