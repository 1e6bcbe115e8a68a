"""CPU oracle for the fused W4A4 + low-rank linear layer -- TEST INFRASTRUCTURE ONLY.

A ctypes binding of ``twq_oracle.c``: the plain C definition of the layer of
TwinQuant (page 1, section 2, eqs. (1)-(3); page 1, section 4.3 for the int4
low-rank variant), binary32 where a float decides an integer, int64 for integer
sums and binary64 for everything else. Only ``tests/``, the smoke check and the
benchmark's CPU-baseline leg may import this package; the HIP library never
does, and the two share no code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "twq_oracle.c")
# TWQ_ORACLE_LIB names another build of twq_oracle.c to load (the CPU sanitizer test
# runs the oracle's pins against an AddressSanitizer/UBSan build this way)
LIB_PATH = os.environ.get("TWQ_ORACLE_LIB") or os.path.join(_HERE, "libtwq_oracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-std=c11",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no contraction) into LIB_PATH."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.orc_half_to_double.restype = ctypes.c_double
        lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_quantize_act.argtypes = [_P, _I, _I, _P, _P, _P]
        lib.orc_quantize_weight.argtypes = [_P, _I, _I, _P, _P, _P]
        lib.orc_residual_acc.argtypes = [_P, _P, _I, _I, _I, _P]
        lib.orc_lowrank_t.argtypes = [_P, _P, _I, _I, _I, _P]
        lib.orc_lowrank_out.argtypes = [_P, _P, _I, _I, _I, _P]
        lib.orc_dual_linear.restype = ctypes.c_int
        lib.orc_dual_linear.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
        lib.orc_dual_linear_sampled.restype = ctypes.c_int
        lib.orc_dual_linear_sampled.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P, _P]
        lib.orc_quantize_lowrank.restype = ctypes.c_int
        lib.orc_quantize_lowrank.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
        lib.orc_lowrank_requant.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P]
        lib.orc_dual_linear_lr4.restype = ctypes.c_int
        lib.orc_dual_linear_lr4.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P]
        lib.orc_dual_linear_lr4_sampled.restype = ctypes.c_int
        lib.orc_dual_linear_lr4_sampled.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P]
        lib.orc_quantize_act_grouped.argtypes = [_P, _I, _I, _I, _P, _P, _P]
        lib.orc_quantize_weight_grouped.argtypes = [_P, _I, _I, _I, _P, _P, _P]
        lib.orc_residual_acc_grouped.argtypes = [_P, _P, _I, _I, _I, _I, _P]
        lib.orc_dual_linear_grouped.restype = ctypes.c_int
        lib.orc_dual_linear_grouped.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]
        lib.orc_dual_linear_grouped_sampled.restype = ctypes.c_int
        lib.orc_dual_linear_grouped_sampled.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _P]
        lib.orc_quantize_act_a8.argtypes = [_P, _I, _I, _P, _P]
        lib.orc_dual_linear_a8.restype = ctypes.c_int
        lib.orc_dual_linear_a8.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
        lib.orc_dual_linear_a8_sampled.restype = ctypes.c_int
        lib.orc_dual_linear_a8_sampled.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P, _P]
        lib.orc_max_threads.restype = ctypes.c_int
        lib.orc_require_i32.restype = ctypes.c_int64
        lib.orc_require_i32.argtypes = [_I]
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _h(a):
    """fp16 array -> its uint16 bit pattern (the C side decodes the format itself)."""
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


FP16_MAX = 65504.0


def _fp16_range(y, t=None):
    """The layer stores Y in fp16 and feeds T to fp16 matrix cores, so the error budget
    of the comparison assumes neither leaves the fp16 range; an input that breaks this
    is rejected here, where Y and T are formed."""
    if y.size and not np.abs(y).max() < FP16_MAX:
        raise AssertionError(f"oracle Y reaches {np.abs(y).max():.6g}, outside the fp16 range")
    if t is not None and t.size and not np.abs(t).max() < FP16_MAX:
        raise AssertionError(f"oracle T reaches {np.abs(t).max():.6g}, outside the fp16 range")
    return y


def max_threads() -> int:
    return int(_load().orc_max_threads())


def half_to_double(h) -> np.ndarray:
    bits = _h(h).ravel()
    lib = _load()
    return np.array([lib.orc_half_to_double(int(v)) for v in bits], np.float64).reshape(np.shape(h))


def quantize_act(x):
    """X fp16 [b][m] -> (codes int8 [b][m], packed u8 [b][m/2], s_X f32 [b])."""
    xb = _h(x)
    b, m = xb.shape
    q = np.empty((b, m), np.int8)
    qp = np.empty((b, m // 2), np.uint8)
    s = np.empty(b, np.float32)
    _load().orc_quantize_act(_p(xb), b, m, _p(q), _p(qp), _p(s))
    return q, qp, s


def quantize_weight(w):
    """W_res f32 [n][m] -> (codes int8 [n][m], packed u8 [n][m/2], s_W f32 [n])."""
    w = _c(w, np.float32)
    n, m = w.shape
    q = np.empty((n, m), np.int8)
    qp = np.empty((n, m // 2), np.uint8)
    s = np.empty(n, np.float32)
    _load().orc_quantize_weight(_p(w), n, m, _p(q), _p(qp), _p(s))
    return q, qp, s


def residual_acc(qx, qw):
    """int64 [b][n] = Q_X [b][m] . Q_W[n][m]^T."""
    qx = _c(qx, np.int8)
    qw = _c(qw, np.int8)
    b, m = qx.shape
    n = qw.shape[0]
    acc = np.empty((b, n), np.int64)
    _load().orc_residual_acc(_p(qx), _p(qw), b, m, n, _p(acc))
    return acc


def lowrank_t(x, l1t):
    """T f64 [b][r] = X . L1 with L1 given transposed [r][m]."""
    xb, lb = _h(x), _h(l1t)
    b, m = xb.shape
    r = lb.shape[0]
    t = np.empty((b, r), np.float64)
    _load().orc_lowrank_t(_p(xb), _p(lb), b, m, r, _p(t))
    return t


def lowrank_out(t, l2t):
    """LR f64 [b][n] = T . L2 with L2 given transposed [n][r]."""
    t = _c(t, np.float64)
    lb = _h(l2t)
    b, r = t.shape
    n = lb.shape[0]
    lr = np.empty((b, n), np.float64)
    _load().orc_lowrank_out(_p(t), _p(lb), b, n, r, _p(lr))
    return lr


def dual_linear(x, w_res, l1t, l2t):
    """The whole layer. Returns dict: qx_packed, sx, qw_packed, sw, acc (int64), t, y (f64)."""
    xb = _h(x)
    w = _c(w_res, np.float32)
    b, m = xb.shape
    n = w.shape[0]
    l1 = _h(l1t) if l1t is not None else np.zeros((0, m), np.uint16)
    l2 = _h(l2t) if l2t is not None else np.zeros((n, 0), np.uint16)
    r = l1.shape[0]
    out = {
        "qx_packed": np.empty((b, m // 2), np.uint8), "sx": np.empty(b, np.float32),
        "qw_packed": np.empty((n, m // 2), np.uint8), "sw": np.empty(n, np.float32),
        "acc": np.empty((b, n), np.int64), "t": np.zeros((b, r), np.float64),
        "y": np.empty((b, n), np.float64),
    }
    rc = _load().orc_dual_linear(_p(xb), _p(w), _p(l1), _p(l2), b, m, n, r,
                                 _p(out["qx_packed"]), _p(out["sx"]), _p(out["qw_packed"]),
                                 _p(out["sw"]), _p(out["acc"]), _p(out["t"]), _p(out["y"]))
    if rc:
        raise MemoryError("oracle allocation failed")
    _fp16_range(out["y"], out["t"])
    return out


def dual_linear_sampled(x, w_res, l1t, l2t, rows, cols):
    """Y and acc at the positions (rows[p], cols[p]) only."""
    xb = _h(x)
    w = _c(w_res, np.float32)
    b, m = xb.shape
    n = w.shape[0]
    l1, l2 = _h(l1t), _h(l2t)
    r = l1.shape[0]
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    assert rows.shape == cols.shape and rows.ndim == 1
    assert ((0 <= rows) & (rows < b)).all() and ((0 <= cols) & (cols < n)).all()
    acc = np.empty(rows.shape[0], np.int64)
    y = np.empty(rows.shape[0], np.float64)
    rc = _load().orc_dual_linear_sampled(_p(xb), _p(w), _p(l1), _p(l2), b, m, n, r,
                                         _p(rows), _p(cols), rows.shape[0], _p(acc), _p(y))
    if rc:
        raise MemoryError("oracle allocation failed")
    return acc, _fp16_range(y)


def quantize_lowrank(l1t, l2t):
    """int4 low-rank factors: dict ql1 [r][m], ql1_packed [r][m/2], sl1 [r],
    ql2 [n][r], ql2_packed [n][r/2], sl2 [r], c [r] (= sl1 * sl2)."""
    l1, l2 = _h(l1t), _h(l2t)
    r, m = l1.shape
    n = l2.shape[0]
    out = {
        "ql1": np.empty((r, m), np.int8), "ql1_packed": np.empty((r, m // 2), np.uint8),
        "sl1": np.empty(r, np.float32), "ql2": np.empty((n, r), np.int8),
        "ql2_packed": np.empty((n, r // 2), np.uint8), "sl2": np.empty(r, np.float32),
        "c": np.empty(r, np.float32),
    }
    rc = _load().orc_quantize_lowrank(_p(l1), _p(l2), r, m, n, _p(out["ql1"]),
                                      _p(out["ql1_packed"]), _p(out["sl1"]), _p(out["ql2"]),
                                      _p(out["ql2_packed"]), _p(out["sl2"]), _p(out["c"]))
    if rc:
        raise MemoryError("oracle allocation failed")
    return out


def lowrank_requant(qx, sx, ql1, c):
    """dict qh [b][r], qh_packed [b][r/2], sh [b], h (int64 H) [b][r]."""
    qx = _c(qx, np.int8)
    sx = _c(sx, np.float32)
    ql1 = _c(ql1, np.int8)
    c = _c(c, np.float32)
    b, m = qx.shape
    r = ql1.shape[0]
    out = {"qh": np.empty((b, r), np.int8), "qh_packed": np.empty((b, r // 2), np.uint8),
           "sh": np.empty(b, np.float32), "h": np.empty((b, r), np.int64)}
    _load().orc_lowrank_requant(_p(qx), _p(sx), _p(ql1), _p(c), b, m, r, _p(out["qh"]),
                                _p(out["qh_packed"]), _p(out["sh"]), _p(out["h"]))
    return out


def dual_linear_lr4(x, w_res, l1t, l2t):
    """The layer with the int4 low-rank branch: dict qh_packed, sh, h, acc2, y."""
    xb = _h(x)
    w = _c(w_res, np.float32)
    b, m = xb.shape
    n = w.shape[0]
    l1, l2 = _h(l1t), _h(l2t)
    r = l1.shape[0]
    out = {"qh_packed": np.empty((b, r // 2), np.uint8), "sh": np.empty(b, np.float32),
           "h": np.empty((b, r), np.int64), "acc2": np.empty((b, n), np.int64),
           "y": np.empty((b, n), np.float64)}
    rc = _load().orc_dual_linear_lr4(_p(xb), _p(w), _p(l1), _p(l2), b, m, n, r,
                                     _p(out["qh_packed"]), _p(out["sh"]), _p(out["h"]),
                                     _p(out["acc2"]), _p(out["y"]))
    if rc:
        raise MemoryError("oracle allocation failed")
    _fp16_range(out["y"])
    return out


def dual_linear_lr4_sampled(x, w_res, l1t, l2t, rows, cols):
    """The int4 low-rank layer at the positions (rows[p], cols[p]): (acc, acc2, y)."""
    xb = _h(x)
    w = _c(w_res, np.float32)
    b, m = xb.shape
    n = w.shape[0]
    l1, l2 = _h(l1t), _h(l2t)
    r = l1.shape[0]
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    assert rows.shape == cols.shape and rows.ndim == 1
    assert ((0 <= rows) & (rows < b)).all() and ((0 <= cols) & (cols < n)).all()
    acc = np.empty(rows.shape[0], np.int64)
    acc2 = np.empty(rows.shape[0], np.int64)
    y = np.empty(rows.shape[0], np.float64)
    rc = _load().orc_dual_linear_lr4_sampled(_p(xb), _p(w), _p(l1), _p(l2), b, m, n, r, _p(rows), _p(cols),
                                             rows.shape[0], _p(acc), _p(acc2), _p(y))
    if rc:
        raise MemoryError("oracle allocation failed")
    return acc, acc2, _fp16_range(y)


def _check_group(m, g):
    if g <= 0 or g % 2 or m % g:
        raise ValueError(f"group size {g} must be even and divide m = {m}")


def quantize_act_grouped(x, g):
    """Group-wise activation quantizer: (codes int8 [b][m], packed u8 [b][m/2], s_X f32 [b][m/g])."""
    xb = _h(x)
    b, m = xb.shape
    _check_group(m, g)
    q = np.empty((b, m), np.int8)
    qp = np.empty((b, m // 2), np.uint8)
    s = np.empty((b, m // g), np.float32)
    _load().orc_quantize_act_grouped(_p(xb), b, m, g, _p(q), _p(qp), _p(s))
    return q, qp, s


def quantize_weight_grouped(w, g):
    """Group-wise weight quantizer: (codes int8 [n][m], packed u8 [n][m/2], s_W f32 [n][m/g])."""
    w = _c(w, np.float32)
    n, m = w.shape
    _check_group(m, g)
    q = np.empty((n, m), np.int8)
    qp = np.empty((n, m // 2), np.uint8)
    s = np.empty((n, m // g), np.float32)
    _load().orc_quantize_weight_grouped(_p(w), n, m, g, _p(q), _p(qp), _p(s))
    return q, qp, s


def residual_acc_grouped(qx, qw, g):
    """int64 [b][n][m/g]: the integer sum of each group of K separately."""
    qx = _c(qx, np.int8)
    qw = _c(qw, np.int8)
    b, m = qx.shape
    n = qw.shape[0]
    _check_group(m, g)
    acc = np.empty((b, n, m // g), np.int64)
    _load().orc_residual_acc_grouped(_p(qx), _p(qw), b, m, n, g, _p(acc))
    return acc


def dual_linear_grouped(x, w_res, l1t, l2t, g):
    """The layer with group-wise scales: dict qx_packed, sx [b][m/g], qw_packed, sw [n][m/g], y."""
    xb = _h(x)
    w = _c(w_res, np.float32)
    b, m = xb.shape
    n = w.shape[0]
    _check_group(m, g)
    l1 = _h(l1t) if l1t is not None else np.zeros((0, m), np.uint16)
    l2 = _h(l2t) if l2t is not None else np.zeros((n, 0), np.uint16)
    r = l1.shape[0]
    out = {"qx_packed": np.empty((b, m // 2), np.uint8), "sx": np.empty((b, m // g), np.float32),
           "qw_packed": np.empty((n, m // 2), np.uint8), "sw": np.empty((n, m // g), np.float32),
           "y": np.empty((b, n), np.float64)}
    rc = _load().orc_dual_linear_grouped(_p(xb), _p(w), _p(l1), _p(l2), b, m, n, r, g,
                                         _p(out["qx_packed"]), _p(out["sx"]), _p(out["qw_packed"]),
                                         _p(out["sw"]), _p(out["y"]))
    if rc:
        raise MemoryError("oracle allocation failed")
    _fp16_range(out["y"])
    return out


def dual_linear_grouped_sampled(x, w_res, l1t, l2t, g, rows, cols):
    """Y of the group-wise layer at the positions (rows[p], cols[p])."""
    xb = _h(x)
    w = _c(w_res, np.float32)
    b, m = xb.shape
    n = w.shape[0]
    _check_group(m, g)
    l1 = _h(l1t) if l1t is not None else np.zeros((0, m), np.uint16)
    l2 = _h(l2t) if l2t is not None else np.zeros((n, 0), np.uint16)
    r = l1.shape[0]
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    assert rows.shape == cols.shape and rows.ndim == 1
    assert ((0 <= rows) & (rows < b)).all() and ((0 <= cols) & (cols < n)).all()
    y = np.empty(rows.shape[0], np.float64)
    rc = _load().orc_dual_linear_grouped_sampled(_p(xb), _p(w), _p(l1), _p(l2), b, m, n, r, g, _p(rows),
                                                 _p(cols), rows.shape[0], _p(y))
    if rc:
        raise MemoryError("oracle allocation failed")
    return _fp16_range(y)


def quantize_act_a8(x):
    """8-bit activation quantizer (q_max = 127): (codes int8 [b][m], s_X f32 [b])."""
    xb = _h(x)
    b, m = xb.shape
    q = np.empty((b, m), np.int8)
    s = np.empty(b, np.float32)
    _load().orc_quantize_act_a8(_p(xb), b, m, _p(q), _p(s))
    return q, s


def dual_linear_a8(x, w_res, l1t, l2t):
    """The W4A8 layer: dict qx (int8 [b][m]), sx, qw_packed, sw, acc (int64), y (f64)."""
    xb = _h(x)
    w = _c(w_res, np.float32)
    b, m = xb.shape
    n = w.shape[0]
    l1 = _h(l1t) if l1t is not None else np.zeros((0, m), np.uint16)
    l2 = _h(l2t) if l2t is not None else np.zeros((n, 0), np.uint16)
    r = l1.shape[0]
    out = {"qx": np.empty((b, m), np.int8), "sx": np.empty(b, np.float32),
           "qw_packed": np.empty((n, m // 2), np.uint8), "sw": np.empty(n, np.float32),
           "acc": np.empty((b, n), np.int64), "y": np.empty((b, n), np.float64)}
    rc = _load().orc_dual_linear_a8(_p(xb), _p(w), _p(l1), _p(l2), b, m, n, r, _p(out["qx"]), _p(out["sx"]),
                                    _p(out["qw_packed"]), _p(out["sw"]), _p(out["acc"]), _p(out["y"]))
    if rc:
        raise MemoryError("oracle allocation failed")
    _fp16_range(out["y"])
    return out


def dual_linear_a8_sampled(x, w_res, l1t, l2t, rows, cols):
    """The W4A8 layer at the positions (rows[p], cols[p]): (acc, y)."""
    xb = _h(x)
    w = _c(w_res, np.float32)
    b, m = xb.shape
    n = w.shape[0]
    l1 = _h(l1t) if l1t is not None else np.zeros((0, m), np.uint16)
    l2 = _h(l2t) if l2t is not None else np.zeros((n, 0), np.uint16)
    r = l1.shape[0]
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    assert rows.shape == cols.shape and rows.ndim == 1
    assert ((0 <= rows) & (rows < b)).all() and ((0 <= cols) & (cols < n)).all()
    acc = np.empty(rows.shape[0], np.int64)
    y = np.empty(rows.shape[0], np.float64)
    rc = _load().orc_dual_linear_a8_sampled(_p(xb), _p(w), _p(l1), _p(l2), b, m, n, r, _p(rows), _p(cols),
                                            rows.shape[0], _p(acc), _p(y))
    if rc:
        raise MemoryError("oracle allocation failed")
    return acc, _fp16_range(y)


def unpack_codes(packed):
    """Canonical packed bytes -> int8 codes (low nibble = even element), for tests."""
    p = np.asarray(packed, np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---- offline preparation: SVD split and folding of given transforms -------------------
#
# TwinQuant page 1, section 4.1 (eq. (6) and the factors defined below it): with an
# orthogonal Q (m x m) acting on the activations and an invertible G (r x r) acting on
# the rank space, the layer's factors become U' = Q^-1 U G, V' = G^-1 V and R' = Q^-1 R,
# and the layer is fed X Q, so that (X Q)(U' V' + R') = X (U V + R) = X W. Learning Q and
# G needs calibration data and is not done here; they are inputs.

def fold_split(w_nm, r, q=None, g=None):
    """Plain fp64 definition. w_nm: W^T (fp32 [n][m], nn.Linear layout), r: rank,
    q: orthogonal [m][m] or None (identity), g: invertible [r][r] or None (identity).
    U S V^T = W (LAPACK SVD), U_r = U[:, :r] sqrt(S_r), V_r = sqrt(S_r) V^T[:r];
    U' = Q^T U_r G and V' = G^-1 V_r rounded to fp16; R' = Q^T W - U' V' from those
    rounded factors, rounded to fp32. Returns (l1t' fp16 [r][m], l2t' fp16 [n][r],
    w_res' fp32 [n][m])."""
    w = np.asarray(w_nm, np.float64).T  # m x n
    m, n = w.shape
    qm = np.eye(m) if q is None else np.asarray(q, np.float64)
    gm = np.eye(r) if g is None else np.asarray(g, np.float64)
    u, s, vt = np.linalg.svd(w, full_matrices=False)
    rs = np.sqrt(s[:r])
    u_r = u[:, :r] * rs[None, :]
    v_r = rs[:, None] * vt[:r]
    u_f = (qm.T @ u_r @ gm).astype(np.float16)
    v_f = np.linalg.solve(gm, v_r).astype(np.float16)
    r_f = (qm.T @ w - u_f.astype(np.float64) @ v_f.astype(np.float64)).astype(np.float32)
    return np.ascontiguousarray(u_f.T), np.ascontiguousarray(v_f.T), np.ascontiguousarray(r_f.T)
