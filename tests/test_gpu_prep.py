"""Offline split and folding on the GPU (TwinQuant page 1, section 4.1: U' = Q^-1 U G,
V' = G^-1 V, R' = Q^-1 R, the layer fed X Q) against the oracle's plain fp64
definition, and the fused layer on the folded operands against the oracle.

The singular vectors of an SVD are unique only up to sign, so the factors are compared
through their product U' V' (and the residual), which is unique when the r-th and
(r+1)-th singular values are apart (the test weights have a decaying spectrum)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a4_rank_gemm_amd as twq
from w4a4_rank_gemm_amd import prep

pytestmark = pytest.mark.gpu


def _case(n, m, r, seed, gap=False):
    rng = synth.rng_for(seed)
    k = min(n, m)
    # gap: the top r singular values well above the rest, so that the randomized range
    # finder (four power iterations) converges to the same subspace as a dense SVD
    spectrum = (np.concatenate([np.geomspace(4.0, 1.0, r), np.geomspace(0.02, 0.001, k - r)]) if gap
                else np.geomspace(4.0, 0.05, k))
    a, _ = np.linalg.qr(rng.standard_normal((n, min(n, m))))
    b, _ = np.linalg.qr(rng.standard_normal((m, min(n, m))))
    w = ((a * spectrum[None, :]) @ b.T).astype(np.float32)
    q, _ = np.linalg.qr(rng.standard_normal((m, m)))
    # an invertible G of condition number at most 4 (a rotation times scales in [0.5, 2]):
    # the fp16 T of the layer is exact only to 2^-11 |T|, and T L2 with T = (X Q) U' G
    # amplifies that by the conditioning of G, which a learned G keeps small
    rot, _ = np.linalg.qr(rng.standard_normal((r, r)))
    g = rot * rng.uniform(0.5, 2.0, r)[None, :]
    x = (rng.standard_normal((24, m)) * 2).astype(np.float16)
    return w, q, g, x


@pytest.mark.parametrize("n,m,r,method", [(384, 512, 32, "exact"), (1024, 2048, 64, "randomized")])
def test_fold_split_matches_oracle_and_layer(n, m, r, method):
    w, q, g, x = _case(n, m, r, 900 + r, gap=method == "randomized")
    dev = torch.device("cuda:0")
    l1t, l2t, w_res = prep.fold_split(torch.from_numpy(w).to(dev), r, torch.from_numpy(q).to(dev),
                                      torch.from_numpy(g).to(dev), method=method, seed=1)
    torch.cuda.synchronize()
    ol1t, ol2t, ow_res = oracle.fold_split(w, r, q, g)
    uv = l1t.double().T @ l2t.double().T
    ou, ov = torch.from_numpy(ol1t.astype(np.float64)).to(dev).T, torch.from_numpy(ol2t.astype(np.float64)).to(dev).T
    ouv = ou @ ov
    # Both sides hold the exact U' V' up to the fp16 rounding of their own factors, which
    # is at most 2^-11 relative per element, so each product lies within 2^-10 |U'| |V'|
    # (elementwise) of the exact one. The factors themselves may differ between the
    # sides (singular vectors are defined up to sign, and G mixes the rank space), so the
    # two rounding bounds add; G also makes |U'| |V'| much larger than |U' V'|.
    gu, gv = l1t.double().T, l2t.double().T
    bound = 2.0 ** -10 * (ou.abs() @ ov.abs() + gu.abs() @ gv.abs()) + 1e-9
    assert ((uv - ouv).abs() <= bound).all()
    assert ((w_res.double().T - torch.from_numpy(ow_res).to(dev).double().T).abs() <= bound + 1e-6).all()
    # the fold leaves the real product unchanged: (X Q)(U' V' + R') = X W
    xd = torch.from_numpy(x.astype(np.float64)).to(dev)
    xq = xd @ torch.from_numpy(q).to(dev)
    ref = xd @ torch.from_numpy(w.astype(np.float64)).to(dev).T
    got = xq @ (uv + w_res.double().T)
    assert (got - ref).abs().max().item() <= 1e-5 * ref.abs().max().item()
    # the fused layer on the folded operands, fed X Q, against the oracle on the same operands
    xq16 = xq.to(torch.float16)
    qw, sw = twq.pack_weight(w_res)
    y = twq.linear(xq16, qw, sw, l1t, l2t)
    torch.cuda.synchronize()
    ref_layer = oracle.dual_linear(xq16.cpu().numpy(), w_res.cpu().numpy(), l1t.cpu().numpy(), l2t.cpu().numpy())
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref_layer["y"]).max()
    assert err <= 2e-3 * np.abs(ref_layer["y"]).max()


def test_fold_split_identity_is_plain_split():
    w, _, _, _ = _case(96, 128, 16, 950)
    dev = torch.device("cuda:0")
    l1t, l2t, w_res = prep.fold_split(torch.from_numpy(w).to(dev), 16)
    torch.cuda.synchronize()
    back = w_res.double() + l2t.double() @ l1t.double()
    assert (back - torch.from_numpy(w).to(dev).double()).abs().max().item() <= 1e-6


def _ulp16(a):
    """Spacing of fp16 at |a| (the distance to the next fp16 away from zero)."""
    a = np.abs(a.astype(np.float16))
    return (np.nextafter(a, np.float16(np.inf)).astype(np.float64) - a.astype(np.float64))


@pytest.mark.parametrize("n,m,r,with_q,with_g", [(384, 512, 32, True, True), (200, 128, 64, False, True),
                                                  (96, 256, 16, True, False), (64, 64, 0, True, False),
                                                  (300, 256, 256, True, True)])
def test_fold_kernels_match_oracle_on_the_same_svd(n, m, r, with_q, with_g):
    """twq_fold_lowrank given the very SVD factors the oracle uses (so no sign ambiguity):
    the fp16 factors equal the oracle's up to one fp16 step (the binary64 products differ
    only in summation order, which can move a value across a rounding boundary), R' is
    exact against the factors it was given (R' + L1 L2 = Q^T W within the fp32 rounding
    of R'), and G^-1 from the kernel's elimination satisfies G V' = V_r."""
    w, q, g, _ = _case(n, m, max(r, 1), 970 + r)
    q = q if with_q else None
    g = (g if with_g else None) if r else None
    wmn = w.astype(np.float64).T  # m x n
    u, s, vt = np.linalg.svd(wmn, full_matrices=False)
    dev = torch.device("cuda:0")
    T = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float64)).to(dev)
    l1t, l2t, w_res = prep.fold_lowrank(T(wmn.T), T(u[:, :r]) if r else None, T(s[:r]) if r else None,
                                        T(vt[:r]) if r else None, T(q), T(g), r)
    torch.cuda.synchronize()
    ol1t, ol2t, ow_res = oracle.fold_split(w, r, q, g)
    for got, want in ((l1t.cpu().numpy(), ol1t), (l2t.cpu().numpy(), ol2t)):
        diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
        assert (diff <= _ulp16(want) * 1.0001).all(), diff.max()
    # exactness of the split against its own factors
    qm = np.eye(m) if q is None else q
    rot = qm.T @ wmn
    back = w_res.cpu().numpy().astype(np.float64).T + l1t.cpu().numpy().astype(np.float64).T @ \
        l2t.cpu().numpy().astype(np.float64).T
    assert np.abs(back - rot).max() <= 2.0 ** -23 * np.abs(rot).max() + 1e-12
    if g is not None:  # G V' = V_r up to the fp16 rounding of V'
        v_r = np.sqrt(s[:r])[:, None] * vt[:r]
        gv = g @ l2t.cpu().numpy().astype(np.float64).T
        bound = 2.0 ** -11 * (np.abs(g) @ np.abs(l2t.cpu().numpy().astype(np.float64).T)) + 1e-12
        assert (np.abs(gv - v_r) <= bound * 1.0001).all()
