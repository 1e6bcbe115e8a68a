"""Seeded synthetic inputs for the fused W4A4 + low-rank linear layer.

This module only *draws* inputs: activations X, the weight W, and the split of W
into a low-rank pair (L1, L2) plus a residual W_res that the layer consumes. It
holds none of the layer's own arithmetic (no quantizer, no integer GEMM, no
merge), so both the CPU oracle and the HIP path can take their inputs from here
without sharing any of the computation they are compared on.

Shapes follow the linear layer of the TwinQuant pages (page 1, section 2,
eqs. (2)-(3)): X is b x m, W is m x n, the low-rank factors are U (m x r) and
V (r x n). Storage is row-major and K-contiguous for every operand:

  x     fp16 [b][m]      activations, one row per token
  w_res fp32 [n][m]      residual weight, one row per output channel
                          (the transpose of the pages' m x n W, nn.Linear layout)
  l1t   fp16 [r][m]      L1 transposed, L1 = U_r sqrt(S_r)   (m x r)
  l2t   fp16 [n][r]      L2 transposed, L2 = sqrt(S_r) V_r^T (r x n)

The value distributions stand in for LLM layers: heavy-tailed weights with a
slowly decaying spectrum (TwinQuant page 1, section 3, observation 1) and
activations with a few outlier channels (page 1, section 1).
"""
from __future__ import annotations

import dataclasses
import numpy as np

GEN_VERSION = 1
SEED_BASE = 20260601


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    index: int
    name: str
    b: int
    m: int
    n: int
    r: int
    x_dist: str            # "normal": N(0,1); "t4": raw Student-t with 4 degrees of freedom
    x_outlier_frac: float  # fraction of input channels that carry outliers
    x_outlier_scale: float
    w_outlier_frac: float  # fraction of input channels (rows of the m x n W) scaled up
    w_outlier_scale: float
    b_gen: int             # X is drawn at this many rows and sliced to b
    svd: str               # "exact" or "randomized"
    lowrank: str = "fp16"  # "fp16", or "int4" for the quantized low-rank variant


def _cfg(index, name, b, m, n, r, x_dist, xf, xs, wf, ws, b_gen, svd, lowrank="fp16"):
    return LayerConfig(index, name, b, m, n, r, x_dist, xf, xs, wf, ws, b_gen, svd, lowrank)


# The five layer shapes (LLaMA3-8B attention / MLP and a 70B-size MLP layer).
# Config 4 runs at two token counts; both slice the same 8192-row X.
CONFIGS = {
    "tiny": _cfg(0, "tiny", 16, 512, 512, 16, "normal", 4 / 512, 30.0, 0.0, 20.0, 16, "exact"),
    "o_proj_decode": _cfg(1, "o_proj_decode", 16, 4096, 4096, 32, "normal", 0.005, 50.0,
                          0.001, 20.0, 16, "randomized"),
    "gate_up_prefill": _cfg(2, "gate_up_prefill", 2048, 4096, 14336, 32, "normal", 0.005, 50.0,
                            0.001, 20.0, 2048, "randomized"),
    "down_prefill": _cfg(3, "down_prefill", 4096, 14336, 4096, 64, "t4", 0.01, 40.0,
                         0.001, 20.0, 4096, "randomized"),
    "70b_gate_up_decode": _cfg(4, "70b_gate_up_decode", 32, 8192, 28672, 128, "normal", 0.005,
                               50.0, 0.001, 20.0, 8192, "randomized"),
    "70b_gate_up_prefill": _cfg(4, "70b_gate_up_prefill", 8192, 8192, 28672, 128, "normal",
                                0.005, 50.0, 0.001, 20.0, 8192, "randomized"),
}


def outlier_count(frac: float, dim: int) -> int:
    """Number of outlier channels: frac * dim rounded half-to-even."""
    return int(np.rint(frac * dim))


def _children(index: int, seed_base: int):
    ss = np.random.SeedSequence(seed_base, spawn_key=(index,))
    # 0: X values, 1: X outlier channels, 2: W values, 3: W outlier channels,
    # 4: randomized-SVD test matrix
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(5)]


def draw_x(rng_vals, rng_out, b: int, m: int, dist: str, frac: float, scale: float):
    """fp16 [b][m]: N(0,1) or raw t_4, with round(frac*m) channels multiplied by scale.

    Values are drawn in fp64, outlier channels scaled, then cast to fp16 once."""
    if dist == "normal":
        x = rng_vals.standard_normal((b, m))
    elif dist == "t4":
        x = rng_vals.standard_t(4, size=(b, m))
    else:
        raise ValueError(dist)
    k = outlier_count(frac, m)
    if k:
        ch = np.sort(rng_out.choice(m, size=k, replace=False))
        x[:, ch] *= scale
    x16 = x.astype(np.float16)
    assert np.isfinite(x16).all()
    return x16


def draw_w(rng_vals, rng_out, n: int, m: int, frac: float, scale: float):
    """fp64 [n][m]: raw Student-t(3) * 0.02, with round(frac*m) input channels
    (rows of the m x n weight, so columns of this storage) multiplied by scale."""
    w = rng_vals.standard_t(3, size=(n, m))
    w *= 0.02
    k = outlier_count(frac, m)
    if k:
        ch = np.sort(rng_out.choice(m, size=k, replace=False))
        w[:, ch] *= scale
    return w


def truncated_svd(a: np.ndarray, r: int, method: str, rng=None):
    """Top-r singular triplets of a (fp64): returns (left [rows][r], s [r], right_t [r][cols])."""
    if method == "exact":
        u, s, vt = np.linalg.svd(a, full_matrices=False)
        return u[:, :r], s[:r], vt[:r]
    # randomized range finder with power iterations (Halko, Martinsson, Tropp 2011,
    # algorithms 4.4 and 5.1): oversampling 16, 4 power iterations, fp64 throughout
    p, q = 16, 4
    k = min(r + p, min(a.shape))
    omega = rng.standard_normal((a.shape[1], k))
    y, _ = np.linalg.qr(a @ omega)
    for _ in range(q):
        z, _ = np.linalg.qr(a.T @ y)
        y, _ = np.linalg.qr(a @ z)
    bmat = y.T @ a
    ub, s, vt = np.linalg.svd(bmat, full_matrices=False)
    u = y @ ub
    return u[:, :r], s[:r], vt[:r]


def split_lowrank(w_nm: np.ndarray, r: int, method: str, rng=None):
    """Split the weight into fp16 low-rank factors and an fp32 residual.

    With W = w_nm^T (m x n) = U S V^T, L1 = U_r sqrt(S_r) and L2 = sqrt(S_r) V_r^T
    (TwinQuant page 1, section 2, eq. (3)). The residual is formed from the
    fp16-rounded factors, W_res = W - L1 L2 in fp64, then cast to fp32, so the
    split is exact against the factors the layer is given.

    Returns (l1t fp16 [r][m], l2t fp16 [n][r], w_res fp32 [n][m])."""
    n, m = w_nm.shape
    if r > min(n, m):
        raise ValueError(f"rank {r} exceeds min(n, m) = {min(n, m)}: the split has no such component")
    if r == 0:
        return (np.zeros((0, m), np.float16), np.zeros((n, 0), np.float16),
                w_nm.astype(np.float32))
    # w_nm = A S B^T with A (n x r) = V_r and B (m x r) = U_r
    a_left, s, b_t = truncated_svd(w_nm, r, method, rng)
    rs = np.sqrt(s)
    l1t = (rs[:, None] * b_t).astype(np.float16)          # sqrt(S) U^T   [r][m]
    l2t = (a_left * rs[None, :]).astype(np.float16)       # V sqrt(S)     [n][r]
    lr = l2t.astype(np.float64) @ l1t.astype(np.float64)  # (L1 L2)^T     [n][m]
    w_res = (w_nm - lr).astype(np.float32)
    return l1t, l2t, w_res


FP16_MAX = 65504.0


def check_fp16_headroom(x: np.ndarray, w_nm: np.ndarray, l1t: np.ndarray):
    """Reject inputs whose unquantized products could leave the fp16 range.

    By Cauchy-Schwarz, |X_i . W_j| <= |X_i| |W_j| and |X_i . L1_t| <= |X_i| |L1_t|
    (Euclidean norms of rows), so max row norms bound every output of X W and every
    T = X L1 without forming either. The layer stores Y in fp16 and feeds T to fp16
    matrix cores; the quantized Y itself is checked where it is formed (the oracle)."""
    xn = np.sqrt(np.square(x.astype(np.float64)).sum(axis=1)).max(initial=0.0)
    wn = np.sqrt(np.square(w_nm.astype(np.float64)).sum(axis=1)).max(initial=0.0)
    ln = np.sqrt(np.square(l1t.astype(np.float64)).sum(axis=1)).max(initial=0.0)
    assert xn * wn < FP16_MAX, f"|X W| may reach {xn * wn:.6g}, outside the fp16 range"
    assert xn * ln < FP16_MAX, f"|X L1| may reach {xn * ln:.6g}, outside the fp16 range"


def make_layer(cfg: LayerConfig | str, seed_base: int = SEED_BASE, b: int | None = None,
               keep_w: bool = False):
    """All inputs of one configuration, deterministic in (config index, seed_base).

    Returns a dict with x, w_res, l1t, l2t (and w, fp32 [n][m], if keep_w)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rx, rxo, rw, rwo, rsvd = _children(cfg.index, seed_base)
    x = draw_x(rx, rxo, cfg.b_gen, cfg.m, cfg.x_dist, cfg.x_outlier_frac, cfg.x_outlier_scale)
    bb = cfg.b if b is None else b
    assert bb <= cfg.b_gen
    x = np.ascontiguousarray(x[:bb])
    w = draw_w(rw, rwo, cfg.n, cfg.m, cfg.w_outlier_frac, cfg.w_outlier_scale)
    l1t, l2t, w_res = split_lowrank(w, cfg.r, cfg.svd, rsvd)
    check_fp16_headroom(x, w, l1t)
    out = {"x": x, "w_res": w_res, "l1t": np.ascontiguousarray(l1t),
           "l2t": np.ascontiguousarray(l2t), "cfg": cfg}
    if keep_w:
        out["w"] = w.astype(np.float32)
    return out


def make_random(b: int, m: int, n: int, r: int, seed: int, x_dist: str = "normal",
                x_outlier_frac: float = 0.01, x_outlier_scale: float = 30.0,
                w_outlier_frac: float = 0.01, w_outlier_scale: float = 20.0):
    """Inputs of an arbitrary shape (ragged and edge cases), same distributions."""
    cfg = LayerConfig(1000 + seed, f"random_{b}x{m}x{n}_r{r}", b, m, n, r, x_dist,
                      x_outlier_frac, x_outlier_scale, w_outlier_frac, w_outlier_scale,
                      b, "exact" if max(m, n) <= 1024 else "randomized")
    return make_layer(cfg, seed_base=SEED_BASE)


def rng_for(seed: int) -> np.random.Generator:
    """A PCG64 stream for test-local draws (sample positions, permutations)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED_BASE, spawn_key=(7, seed))))
