"""Offline preparation of a TwinQuant layer on the GPU: the rank-r SVD split of the
weight and the folding of given transforms into its factors.

TwinQuant page 1, section 2, eq. (3): W = U V + R with a rank-r low-rank pair from the
SVD and a residual R. Page 1, section 4.1 (eq. (6) and the factors below it): an
orthogonal Q (m x m) on the activations and an invertible G (r x r) on the rank space
give U' = Q^-1 U G, V' = G^-1 V and R' = Q^-1 R, and the layer is fed X Q; the real
product is unchanged, (X Q)(U' V' + R') = X W. Learning Q and G needs calibration data
and is not part of this library: they come in as inputs.

Only the SVD runs on the platform's dense linear algebra (torch.linalg, fp64); the
folding -- the scalings, Q^T U_r G, G^-1 (Gauss-Jordan) V_r, the fp16 rounding of the
factors and R' = Q^T W - U' V' -- is libtwq's twq_fold_lowrank (HIP kernels, binary64).
This runs once per layer, before serving; its outputs feed twq_pack_weight and the
fused layer.
"""
from __future__ import annotations

import torch


def _top_svd(w: torch.Tensor, r: int, method: str, seed: int):
    """Top-r singular triplets of w (fp64, on its device): (u [m][r], s [r], vt [r][n])."""
    if method == "exact":
        u, s, vt = torch.linalg.svd(w, full_matrices=False)
        return u[:, :r], s[:r], vt[:r]
    # randomized range finder with power iterations (Halko, Martinsson and Tropp 2011,
    # algorithms 4.4 and 5.1): oversampling 16, 4 power iterations
    k = min(r + 16, min(w.shape))
    gen = torch.Generator(device=w.device).manual_seed(seed)
    omega = torch.randn((w.shape[1], k), generator=gen, device=w.device, dtype=w.dtype)
    y = torch.linalg.qr(w @ omega).Q
    for _ in range(4):
        z = torch.linalg.qr(w.T @ y).Q
        y = torch.linalg.qr(w @ z).Q
    ub, s, vt = torch.linalg.svd(y.T @ w, full_matrices=False)
    return (y @ ub)[:, :r], s[:r], vt[:r]


def fold_split(w_nm: torch.Tensor, r: int, q: torch.Tensor | None = None, g: torch.Tensor | None = None,
               method: str = "auto", seed: int = 0):
    """Split and fold one layer on the GPU.

    w_nm: W^T, fp32 [n][m] (nn.Linear layout); r: rank; q: orthogonal [m][m] or None
    (identity); g: invertible [r][r] or None (identity). U' = Q^T U_r G and V' =
    G^-1 V_r are rounded to fp16, and R' = Q^T W - U' V' is formed from those rounded
    factors in fp64 and rounded to fp32, so the split is exact against the factors the
    layer is given. method: "exact" (dense SVD), "randomized", or "auto" (exact up to
    4096 on the longer side). Returns (l1t' fp16 [r][m], l2t' fp16 [n][r], w_res' fp32
    [n][m]) on w_nm's device; the layer is then called on X Q."""
    if w_nm.dim() != 2 or w_nm.device.type != "cuda":
        raise ValueError("w_nm must be a 2-D GPU tensor")
    n, m = w_nm.shape
    if not 0 <= r <= min(m, n):
        raise ValueError(f"rank {r} must lie in [0, min(m, n) = {min(m, n)}]")
    dev = w_nm.device
    if q is not None and q.shape != (m, m):
        raise ValueError("q must be [m][m]")
    if g is not None and g.shape != (r, r):
        raise ValueError("g must be [r][r]")
    w_nm64 = w_nm.to(torch.float64).contiguous()
    if method == "auto":
        method = "exact" if max(m, n) <= 4096 else "randomized"
    if r > 0:  # the SVD of W (m x n) on the platform library
        u, sv, vt = _top_svd(w_nm64.T, r, method, seed)
        u, sv, vt = u.contiguous(), sv.contiguous(), vt.contiguous()
    else:
        u = sv = vt = None
    qd = None if q is None else q.to(dev, torch.float64).contiguous()
    gd = None if (g is None or r == 0) else g.to(dev, torch.float64).contiguous()
    return fold_lowrank(w_nm64, u, sv, vt, qd, gd, r)


def fold_lowrank(w_nm64: torch.Tensor, u, sv, vt, q, g, r: int):
    """twq_fold_lowrank: the folded split from the top-r SVD factors of W (u fp64 [m][r],
    sv [r], vt [r][n]; None when r == 0), W^T fp64 [n][m], and q fp64 [m][m] / g fp64
    [r][r] or None. Returns (l1t' fp16 [r][m], l2t' fp16 [n][r], w_res' fp32 [n][m])."""
    import w4a4_rank_gemm_amd as twq
    n, m = w_nm64.shape
    dev = w_nm64.device
    for name, t, shape in (("w", w_nm64, (n, m)), ("u", u, (m, r)), ("s", sv, (r,)), ("vt", vt, (r, n)),
                           ("q", q, (m, m)), ("g", g, (r, r))):
        if t is None:
            continue
        if t.dtype != torch.float64 or not t.is_contiguous() or t.device != dev or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be contiguous fp64 {shape} on {dev}")
    l1t = torch.empty((r, m), dtype=torch.float16, device=dev)
    l2t = torch.empty((n, r), dtype=torch.float16, device=dev)
    w_res = torch.empty((n, m), dtype=torch.float32, device=dev)
    L = twq.lib()
    need = L.twq_fold_workspace_bytes(m, n, r)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    P = twq._ptr
    twq._check(L.twq_fold_lowrank(P(w_nm64), P(u), P(sv), P(vt), P(q), P(g), m, n, r, P(l1t) if r else None,
                                  P(l2t) if r else None, P(w_res), P(ws), need, twq._stream(dev)),
               "twq_fold_lowrank")
    return l1t, l2t, w_res
