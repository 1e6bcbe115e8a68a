"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value is a
hand-worked vector of eq. (1)-(3) of TwinQuant (page 1, section 2), an exact
rational model of binary32 rounding, a pure-Python brute force, an invariant of
the quantizer, or an identity that reduces the layer to a library routine.
"""
import json
import os
from fractions import Fraction as F

import numpy as np
import pytest

import synth
from tests import ratmodel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_vectors():
    cases = []
    with open(os.path.join(GOLDEN, "quantizer_vectors.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, xs, s, q, _why = [p.strip() for p in line.split("|")]
            cases.append((name, [float(v) for v in xs.split()], float(s), [int(v) for v in q.split()]))
    return cases


VECTORS = _load_vectors()


# ---------------------------------------------------------------- fp16 decoding

def test_half_decode_all_bit_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_lib.half_to_double(bits.view(np.float16))
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == want[~nan]).all()


# ---------------------------------------------------------------- quantizer, eq. (1)

@pytest.mark.parametrize("case", VECTORS, ids=[c[0] for c in VECTORS])
def test_quantizer_hand_vectors(oracle_lib, case):
    name, xs, s_want, q_want = case
    x = np.array([xs], np.float16)
    assert (x.astype(np.float64)[0] == np.array(xs)).all(), "fixture values must be exact in fp16"
    # the fixture itself re-derived from exact rationals
    s_rat, q_rat = ratmodel.quantize([F(v) for v in xs])
    assert float(s_rat) == s_want and q_rat == q_want
    q, _, s = oracle_lib.quantize_act(x)
    assert float(s[0]) == s_want
    assert q[0].tolist() == q_want
    # the same vector as a weight row (binary32 input path)
    qw, _, sw = oracle_lib.quantize_weight(x.astype(np.float32))
    assert float(sw[0]) == s_want and qw[0].tolist() == q_want


def test_reciprocal_form_differs_on_e4():
    """eq. (1) divides by s; the reciprocal form would round E4 the other way."""
    amax, x = F(1.9453125), F(0.97265625)
    s = ratmodel.rnd32(amax / 7)
    assert ratmodel.rne_int(ratmodel.rnd32(x / s)) == 3
    assert ratmodel.rne_int(ratmodel.rnd32(x * ratmodel.rnd32(7 / amax))) == 4


def _rows_with_near_ties(rng, rows, cols):
    """fp16 rows that include values landing within an ulp of k + 1/2 after division."""
    out = rng.standard_normal((rows, cols)) * rng.choice([0.01, 1.0, 30.0], size=(rows, 1))
    for i in range(rows):
        amax = np.float32(np.abs(out[i]).max())
        s = np.float64(np.float32(amax / np.float32(7)))
        ks = rng.integers(-7, 7, size=cols // 4) + 0.5
        pos = rng.choice(cols, size=cols // 4, replace=False)
        out[i, pos] = ks * s
    return out.astype(np.float16)


def test_quantizer_matches_rational_model(oracle_lib):
    rng = synth.rng_for(1)
    x = _rows_with_near_ties(rng, 48, 64)
    q, _, s = oracle_lib.quantize_act(x)
    for i in range(x.shape[0]):
        s_rat, q_rat = ratmodel.quantize([F(float(v)) for v in x[i]])
        assert float(s[i]) == float(s_rat)
        assert q[i].tolist() == q_rat, i
    w = (rng.standard_t(3, size=(32, 48)) * 0.02).astype(np.float32)
    qw, _, sw = oracle_lib.quantize_weight(w)
    for j in range(w.shape[0]):
        s_rat, q_rat = ratmodel.quantize([F(float(v)) for v in w[j]])
        assert float(sw[j]) == float(s_rat) and qw[j].tolist() == q_rat


def test_max_code_is_seven_for_every_fp16_amax(oracle_lib):
    """For every positive finite fp16 amax, amax / fl32(amax / 7) rounds to 7, so the
    clamp to [-7, 7] never acts and every nonzero row reaches q_max exactly."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)  # all positive finite fp16 values
    a = bits.view(np.float16)
    x = np.stack([a, np.zeros_like(a)], axis=1)
    q, _, s = oracle_lib.quantize_act(x)
    assert (q[:, 0] == 7).all() and (q[:, 1] == 0).all()
    # the exact-rational model agrees on a strided subset (every value is slow in Python)
    for v in a[::97]:
        fv = F(float(v))
        sv = ratmodel.rnd32(fv / 7)
        assert ratmodel.rne_int(ratmodel.rnd32(fv / sv)) == 7


def test_quantizer_invariants(oracle_lib):
    d = synth.make_layer("tiny")
    x = d["x"].astype(np.float16)
    q, _, s = oracle_lib.quantize_act(x)
    xf = x.astype(np.float64)
    # codes in range, every nonzero row reaches q_max
    assert np.abs(q).max() <= 7 and (np.abs(q).max(axis=1) == 7).all()
    # odd symmetry q(-x) = -q(x), same scale
    qn, _, sn = oracle_lib.quantize_act(-x)
    assert (qn == -q).all() and (sn == s).all()
    # scaling by a power of two scales s exactly and leaves codes unchanged
    for e in (1, 2):  # upward in fp16 stays exact (no subnormal loss, no overflow here)
        xe = (xf * 2.0 ** e).astype(np.float16)
        assert (xe.astype(np.float64) == xf * 2.0 ** e).all()
        qe, _, se = oracle_lib.quantize_act(xe)
        assert (qe == q).all() and (se.astype(np.float64) == s.astype(np.float64) * 2.0 ** e).all()
    w = d["w_res"]
    qw, _, sw = oracle_lib.quantize_weight(w)
    for e in (-9, 5):  # binary32 weights: exact both ways at these magnitudes
        qe, _, se = oracle_lib.quantize_weight(w * np.float32(2.0 ** e))
        assert (qe == qw).all() and (se.astype(np.float64) == sw.astype(np.float64) * 2.0 ** e).all()
    # rounding error of the dequantized value: |x - s q| <= (s/2)(1 + 2^-20)
    err = np.abs(xf - s[:, None].astype(np.float64) * q)
    assert (err <= s[:, None] / 2 * (1 + 2.0 ** -20)).all()
    # all-zero rows: scale 0, codes 0
    z = np.zeros((3, 128), np.float16)
    qz, pz, sz = oracle_lib.quantize_act(z)
    assert (qz == 0).all() and (pz == 0).all() and (sz == 0).all()


def test_quantizer_nearest_integer_bound(oracle_lib):
    """Against exact rationals: each code is within 1/2 (+ one binary32 rounding) of x/s,
    and it is the unique nearest integer wherever x/s is not within 2^-20 of a half."""
    rng = synth.rng_for(2)
    x = (rng.standard_normal((16, 256)) * 3).astype(np.float16)
    q, _, s = oracle_lib.quantize_act(x)
    for i in range(x.shape[0]):
        si = F(float(s[i]))
        for k in range(x.shape[1]):
            ratio = F(float(x[i, k])) / si
            d = abs(ratio - q[i, k])
            assert d <= F(1, 2) + F(1, 2 ** 20)
            if abs(abs(ratio - int(ratio)) - F(1, 2)) > F(1, 2 ** 20):
                assert q[i, k] == ratmodel.rne_int(ratio)


# ---------------------------------------------------------------- packing

def test_packed_layout(oracle_lib):
    x = np.array([[1, 2, 3, -4], [0.5, -1.75, 3.5, -7]], np.float16)
    q, p, _ = oracle_lib.quantize_act(x)
    # byte t: code 2t in the low nibble, code 2t+1 in the high nibble, two's complement
    assert p.tolist() == [[0x32, 0x95], [0xE0, 0x94]]
    assert (oracle_lib.unpack_codes(p) == q).all()
    d = synth.make_layer("tiny")
    q, p, _ = oracle_lib.quantize_act(d["x"])
    assert (oracle_lib.unpack_codes(p) == q).all()


# ---------------------------------------------------------------- integer GEMM, eq. (2)

def test_residual_acc_bruteforce(oracle_lib):
    rng = synth.rng_for(3)
    for b, m, n in [(1, 2, 1), (3, 8, 5), (7, 16, 9)]:
        qx = rng.integers(-7, 8, size=(b, m)).astype(np.int8)
        qw = rng.integers(-7, 8, size=(n, m)).astype(np.int8)
        acc = oracle_lib.residual_acc(qx, qw)
        for i in range(b):
            for j in range(n):
                assert acc[i, j] == sum(int(qx[i, k]) * int(qw[j, k]) for k in range(m))


def test_residual_acc_library_and_permutation(oracle_lib):
    rng = synth.rng_for(4)
    qx = rng.integers(-7, 8, size=(19, 256)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(33, 256)).astype(np.int8)
    acc = oracle_lib.residual_acc(qx, qw)
    assert (acc == qx.astype(np.int64) @ qw.astype(np.int64).T).all()
    perm = rng.permutation(256)
    assert (oracle_lib.residual_acc(qx[:, perm], qw[:, perm]) == acc).all()
    # extreme codes reach 49 m
    full = np.full((1, 14336), 7, np.int8)
    assert oracle_lib.residual_acc(full, -full)[0, 0] == -49 * 14336


# ---------------------------------------------------------------- whole layer, eqs. (2)-(3)

def _e6():
    with open(os.path.join(GOLDEN, "e6_layer.json")) as f:
        return json.load(f)


def test_e6_whole_layer(oracle_lib):
    g = _e6()
    x = np.array(g["x"], np.float16)
    out = oracle_lib.dual_linear(x, np.array(g["w_res"], np.float32),
                                 np.array(g["l1t"], np.float16), np.array(g["l2t"], np.float16))
    assert out["qx_packed"].tolist() == g["qx_packed"]
    assert (oracle_lib.unpack_codes(out["qx_packed"]) == np.array(g["qx"])).all()
    assert (oracle_lib.unpack_codes(out["qw_packed"]) == np.array(g["qw"])).all()
    assert out["sx"].astype(np.float64).tolist() == g["sx"]
    assert out["sw"].astype(np.float64).tolist() == g["sw"]
    assert out["acc"].tolist() == g["acc"]
    assert out["t"].tolist() == g["t"]
    np.testing.assert_allclose(out["y"], np.array(g["y"]), rtol=0, atol=1e-12)
    assert out["y"].astype(np.float16).astype(np.float64).tolist() == g["y_fp16"]


def test_identity_rank0_is_plain_w4a4(oracle_lib):
    """r = 0: Y = diag(s_X) (Q_X Q_W^T) diag(s_W), checked with a library int64 matmul."""
    rng = synth.rng_for(5)
    x = (rng.standard_normal((9, 64)) * 2).astype(np.float16)
    w = (rng.standard_t(3, size=(12, 64)) * 0.02).astype(np.float32)
    out = oracle_lib.dual_linear(x, w, None, None)
    qx = oracle_lib.unpack_codes(out["qx_packed"]).astype(np.int64)
    qw = oracle_lib.unpack_codes(out["qw_packed"]).astype(np.int64)
    ref = out["sx"].astype(np.float64)[:, None] * out["sw"].astype(np.float64)[None, :] * (qx @ qw.T)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-15, atol=0)


def test_identity_zero_residual_is_pure_lowrank(oracle_lib):
    """W_res = 0: s_W = 0, Q_W = 0 and Y = X L1 L2, checked with a library fp64 matmul on
    non-square shapes so that a transposed operand cannot pass."""
    rng = synth.rng_for(6)
    b, m, n, r = 5, 24, 10, 3
    x = rng.standard_normal((b, m)).astype(np.float16)
    l1t = rng.standard_normal((r, m)).astype(np.float16)
    l2t = rng.standard_normal((n, r)).astype(np.float16)
    out = oracle_lib.dual_linear(x, np.zeros((n, m), np.float32), l1t, l2t)
    assert (out["sw"] == 0).all() and (out["qw_packed"] == 0).all() and (out["acc"] == 0).all()
    ref_t = x.astype(np.float64) @ l1t.astype(np.float64).T
    ref = ref_t @ l2t.astype(np.float64).T
    np.testing.assert_allclose(out["t"], ref_t, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_sampled_matches_full(oracle_lib):
    d = synth.make_layer("tiny")
    full = oracle_lib.dual_linear(d["x"], d["w_res"], d["l1t"], d["l2t"])
    rng = synth.rng_for(7)
    rows = rng.integers(0, 16, 64)
    cols = rng.integers(0, 512, 64)
    acc, y = oracle_lib.dual_linear_sampled(d["x"], d["w_res"], d["l1t"], d["l2t"], rows, cols)
    assert (acc == full["acc"][rows, cols]).all()
    assert (y == full["y"][rows, cols]).all()


def test_layer_split_reconstructs_weight():
    """The inputs are a split of W: W_res + L1 L2 = W up to one binary32 rounding."""
    d = synth.make_layer("tiny", keep_w=True)
    rec = d["w_res"].astype(np.float64) + d["l2t"].astype(np.float64) @ d["l1t"].astype(np.float64)
    np.testing.assert_allclose(rec, d["w"].astype(np.float64), rtol=0, atol=2.0 ** -20)


# ---------------------------------------------------------------- int4 low-rank variant

def _lr4():
    with open(os.path.join(GOLDEN, "lr4_layer.json")) as f:
        return json.load(f)


def test_lr4_hand_worked(oracle_lib):
    g = _lr4()
    x = np.array(g["x"], np.float16)
    l1t = np.array(g["l1t"], np.float16)
    l2t = np.array(g["l2t"], np.float16)
    w = np.array(g["w_res"], np.float32)
    f = oracle_lib.quantize_lowrank(l1t, l2t)
    assert f["ql1"].tolist() == g["ql1"] and f["ql2"].tolist() == g["ql2"]
    assert f["sl1"].astype(np.float64).tolist() == g["sl1"]
    assert f["sl2"].astype(np.float64).tolist() == g["sl2"]
    assert f["c"].astype(np.float64).tolist() == g["c"]
    assert (oracle_lib.unpack_codes(f["ql1_packed"]) == f["ql1"]).all()
    assert (oracle_lib.unpack_codes(f["ql2_packed"]) == f["ql2"]).all()
    out = oracle_lib.dual_linear_lr4(x, w, l1t, l2t)
    assert out["h"].tolist() == g["h"]
    assert (oracle_lib.unpack_codes(out["qh_packed"]) == np.array(g["qh"])).all()
    assert out["sh"].astype(np.float64).tolist() == g["sh"]
    assert out["acc2"].tolist() == g["acc2"]
    np.testing.assert_allclose(out["y"], np.array(g["y"]), rtol=0, atol=1e-12)
    assert out["y"].astype(np.float16).astype(np.float64).tolist() == g["y_fp16"]


def test_lr4_hand_worked_rational(oracle_lib):
    """The lr4 fixture re-derived with the exact binary32 model."""
    g = _lr4()
    sx, qx = ratmodel.quantize([F(v) for v in g["x"][0]])
    ql1 = [ratmodel.quantize([F(v) for v in row]) for row in g["l1t"]]
    l2t = g["l2t"]
    ql2 = [ratmodel.quantize([F(l2t[j][t]) for j in range(len(l2t))]) for t in range(len(l2t[0]))]
    c = [ratmodel.rnd32(ql1[t][0] * ql2[t][0]) for t in range(len(ql1))]
    assert [float(v) for v in c] == g["c"]
    H = [sum(qx[k] * ql1[t][1][k] for k in range(len(qx))) for t in range(len(ql1))]
    assert H == g["h"][0]
    h = [ratmodel.rnd32(ratmodel.rnd32(sx * H[t]) * c[t]) for t in range(len(H))]
    sh, qh = ratmodel.quantize(h)
    assert float(sh) == g["sh"][0] and qh == g["qh"][0]


def test_lr4_bruteforce_and_bound(oracle_lib):
    """H and acc2 by pure-Python brute force; the int4 branch stays within its derived
    requantization bound of the exactly dequantized product Q(X) Q(L1) Q(L2)."""
    rng = synth.rng_for(8)
    b, m, n, r = 3, 16, 6, 4
    x = rng.standard_normal((b, m)).astype(np.float16)
    l1t = rng.standard_normal((r, m)).astype(np.float16)
    l2t = rng.standard_normal((n, r)).astype(np.float16)
    w = np.zeros((n, m), np.float32)
    f = oracle_lib.quantize_lowrank(l1t, l2t)
    qx, _, sx = oracle_lib.quantize_act(x)
    rq = oracle_lib.lowrank_requant(qx, sx, f["ql1"], f["c"])
    out = oracle_lib.dual_linear_lr4(x, w, l1t, l2t)
    qh = oracle_lib.unpack_codes(out["qh_packed"])
    assert (qh == rq["qh"]).all() and (out["sh"] == rq["sh"]).all()
    for i in range(b):
        for t in range(r):
            assert out["h"][i, t] == sum(int(qx[i, k]) * int(f["ql1"][t, k]) for k in range(m))
        for j in range(n):
            assert out["acc2"][i, j] == sum(int(qh[i, t]) * int(f["ql2"][j, t]) for t in range(r))
    assert (np.abs(qh).max(axis=1) == 7).all()
    # exact dequantized reference and the bound |h_t - s_H Q_H,t| <= (s_H/2)(1 + 2^-20)
    # propagated through |Q_L2| (plus the binary32 roundings of h, far below it)
    deq_x = sx.astype(np.float64)[:, None] * qx
    deq_l1 = (f["sl1"].astype(np.float64)[:, None] * f["ql1"]).T       # m x r
    deq_l2 = (f["sl2"].astype(np.float64)[None, :] * f["ql2"]).T       # r x n
    exact = deq_x @ deq_l1 @ deq_l2
    sh = out["sh"].astype(np.float64)
    bound = (sh[:, None] / 2 * (1 + 2.0 ** -20) + np.abs(deq_x @ deq_l1).max(axis=1, keepdims=True) * 2.0 ** -22) \
        * np.abs(f["ql2"]).sum(axis=1)[None, :]
    assert (np.abs(out["y"] - exact) <= bound).all()


def test_lr4_rank1_identity(oracle_lib):
    """r = 1: Q_H = +-7 so s_H Q_H = h up to one rounding, and the branch equals
    Q(X) Q(L1) Q(L2) to binary32 precision."""
    rng = synth.rng_for(9)
    b, m, n = 4, 32, 8
    x = rng.standard_normal((b, m)).astype(np.float16)
    l1t = rng.standard_normal((1, m)).astype(np.float16)
    l2t = rng.standard_normal((n, 1)).astype(np.float16)
    out = oracle_lib.dual_linear_lr4(x, np.zeros((n, m), np.float32), l1t, l2t)
    f = oracle_lib.quantize_lowrank(l1t, l2t)
    qx, _, sx = oracle_lib.quantize_act(x)
    exact = (sx.astype(np.float64)[:, None] * qx) @ (f["sl1"][0] * f["ql1"][0].astype(np.float64))
    exact = exact[:, None] * (f["sl2"][0] * f["ql2"][:, 0].astype(np.float64))[None, :]
    np.testing.assert_allclose(out["y"], exact, rtol=4e-7, atol=0)


def test_lr4_sampled_matches_full(oracle_lib):
    d = synth.make_random(12, 256, 48, 32, seed=21)
    full = oracle_lib.dual_linear_lr4(d["x"], d["w_res"], d["l1t"], d["l2t"])
    rng = synth.rng_for(22)
    rows = rng.integers(0, 12, 40)
    cols = rng.integers(0, 48, 40)
    acc, acc2, y = oracle_lib.dual_linear_lr4_sampled(d["x"], d["w_res"], d["l1t"], d["l2t"], rows, cols)
    assert (acc2 == full["acc2"][rows, cols]).all()
    assert (y == full["y"][rows, cols]).all()
    ref_acc = oracle_lib.dual_linear(d["x"], d["w_res"], d["l1t"], d["l2t"])["acc"]
    assert (acc == ref_acc[rows, cols]).all()


# ---------------------------------------------------------------- generators

def test_generators_deterministic_and_outliers():
    a = synth.make_layer("tiny")
    b = synth.make_layer("tiny")
    for k in ("x", "w_res", "l1t", "l2t"):
        assert a[k].tobytes() == b[k].tobytes()
    assert synth.outlier_count(0.005, 4096) == 20 and synth.outlier_count(0.01, 14336) == 143
    assert synth.outlier_count(0.001, 8192) == 8 and synth.outlier_count(4 / 512, 512) == 4
    with pytest.raises(ValueError):
        synth.make_random(4, 128, 16, 32, seed=0)  # rank above min(n, m)
    # the 4 outlier channels of the tiny config dominate the column maxima
    colmax = np.abs(a["x"].astype(np.float64)).max(axis=0)
    assert (np.sort(colmax)[-4:] > 10 * np.median(colmax)).all()


# ---------------------------------------------------------------- group-wise scales (g = 128 in the pages' experiments)

def _grouped():
    with open(os.path.join(GOLDEN, "grouped_layer.json")) as f:
        return json.load(f)


def test_grouped_hand_worked(oracle_lib):
    gd = _grouped()
    g = gd["g"]
    x = np.array(gd["x"], np.float16)
    w = np.array(gd["w_res"], np.float32)
    qx, qxp, sx = oracle_lib.quantize_act_grouped(x, g)
    qw, qwp, sw = oracle_lib.quantize_weight_grouped(w, g)
    assert qx.tolist() == gd["qx"] and qxp.tolist() == gd["qx_packed"]
    assert qw.tolist() == gd["qw"] and qwp.tolist() == gd["qw_packed"]
    assert sx.astype(np.float64).tolist() == gd["sx"] and sw.astype(np.float64).tolist() == gd["sw"]
    assert oracle_lib.residual_acc_grouped(qx, qw, g).tolist() == gd["acc_grouped"]
    out = oracle_lib.dual_linear_grouped(x, w, None, None, g)
    assert out["y"].tolist() == gd["y"]
    assert out["qx_packed"].tolist() == gd["qx_packed"] and out["sw"].astype(np.float64).tolist() == gd["sw"]
    # one scale per token gives different codes for the first group
    assert oracle_lib.quantize_act(x)[0][0].tolist() == gd["qx_per_token_row0"]


def test_grouped_rational_bruteforce(oracle_lib):
    """Codes, scales and Y of the group-wise layer from exact rationals (binary32 roundings
    decided by the rational model), including the low-rank branch."""
    rng = synth.rng_for(40)
    b, m, n, r, g = 3, 16, 5, 2, 4
    x = (rng.standard_normal((b, m)) * np.array([1, 1, 1, 30] * 4)).astype(np.float16)
    x[1, 4:8] = 0  # an all-zero group
    w = (rng.standard_t(3, size=(n, m)) * 0.02).astype(np.float32)
    w[2, 8:12] = 0
    l1t = rng.standard_normal((r, m)).astype(np.float16)
    l2t = rng.standard_normal((n, r)).astype(np.float16)
    out = oracle_lib.dual_linear_grouped(x, w, l1t, l2t, g)
    qx = oracle_lib.unpack_codes(out["qx_packed"])
    qw = oracle_lib.unpack_codes(out["qw_packed"])
    xf = [[F(float(v)) for v in row] for row in x]
    wf = [[F(float(v)) for v in row] for row in w]
    for i in range(b):
        for G in range(m // g):
            s, q = ratmodel.quantize(xf[i][G * g:(G + 1) * g])
            assert F(float(out["sx"][i, G])) == s and qx[i, G * g:(G + 1) * g].tolist() == q
    for j in range(n):
        for G in range(m // g):
            s, q = ratmodel.quantize(wf[j][G * g:(G + 1) * g])
            assert F(float(out["sw"][j, G])) == s and qw[j, G * g:(G + 1) * g].tolist() == q
    l1 = [[F(float(v)) for v in row] for row in l1t]
    l2 = [[F(float(v)) for v in row] for row in l2t]
    for i in range(b):
        t = [sum(xf[i][k] * l1[u][k] for k in range(m)) for u in range(r)]
        for j in range(n):
            y = sum(F(float(out["sx"][i, G])) * F(float(out["sw"][j, G])) *
                    sum(int(qx[i, k]) * int(qw[j, k]) for k in range(G * g, (G + 1) * g))
                    for G in range(m // g))
            y += sum(t[u] * l2[j][u] for u in range(r))
            assert abs(float(y) - out["y"][i, j]) <= 1e-12 * max(1.0, abs(float(y)))


def test_grouped_one_group_is_per_token(oracle_lib):
    """g = m: one group per row, which is the per-token / per-channel layer exactly."""
    d = synth.make_random(6, 96, 20, 16, seed=41)
    m = d["x"].shape[1]
    gl = oracle_lib.dual_linear_grouped(d["x"], d["w_res"], d["l1t"], d["l2t"], m)
    pl = oracle_lib.dual_linear(d["x"], d["w_res"], d["l1t"], d["l2t"])
    assert (gl["qx_packed"] == pl["qx_packed"]).all() and (gl["qw_packed"] == pl["qw_packed"]).all()
    assert (gl["sx"][:, 0] == pl["sx"]).all() and (gl["sw"][:, 0] == pl["sw"]).all()
    assert (gl["y"] == pl["y"]).all()


def test_grouped_rows_are_per_row_quantization(oracle_lib):
    """Each group is eq. (1) on its own: the group-wise quantizer of a [rows][m] matrix is the
    per-row quantizer of the same matrix cut into [rows m / g][g]."""
    d = synth.make_random(4, 512, 24, 16, seed=42)
    for g in (128, 32, 512):
        qx, _, sx = oracle_lib.quantize_act_grouped(d["x"], g)
        qx1, _, sx1 = oracle_lib.quantize_act(d["x"].reshape(-1, g))
        assert (qx.reshape(-1, g) == qx1).all() and (sx.reshape(-1) == sx1).all()
        qw, _, sw = oracle_lib.quantize_weight_grouped(d["w_res"], g)
        qw1, _, sw1 = oracle_lib.quantize_weight(d["w_res"].reshape(-1, g))
        assert (qw.reshape(-1, g) == qw1).all() and (sw.reshape(-1) == sw1).all()


def test_grouped_scales_are_local(oracle_lib):
    """An outlier changes the codes and scale of its own group and nothing else."""
    rng = synth.rng_for(43)
    x = rng.standard_normal((2, 512)).astype(np.float16)
    q0, _, s0 = oracle_lib.quantize_act_grouped(x, 128)
    x2 = x.copy()
    x2[0, 300] = 900.0  # group 2 of row 0
    q1, _, s1 = oracle_lib.quantize_act_grouped(x2, 128)
    changed = s1 != s0
    assert changed.tolist() == [[False, False, True, False], [False, False, False, False]]
    keep = np.ones((2, 512), bool)
    keep[0, 256:384] = False
    assert (q0[keep] == q1[keep]).all() and (q0[0, 256:384] != q1[0, 256:384]).any()


def test_grouped_acc_sums_to_whole_acc(oracle_lib):
    rng = synth.rng_for(44)
    qx = rng.integers(-7, 8, size=(5, 256)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(7, 256)).astype(np.int8)
    accg = oracle_lib.residual_acc_grouped(qx, qw, 64)
    assert (accg.sum(axis=2) == oracle_lib.residual_acc(qx, qw)).all()
    i, j, G = 3, 5, 2
    assert accg[i, j, G] == sum(int(qx[i, k]) * int(qw[j, k]) for k in range(128, 192))


def test_grouped_sampled_matches_full(oracle_lib):
    d = synth.make_random(10, 384, 40, 16, seed=45)
    full = oracle_lib.dual_linear_grouped(d["x"], d["w_res"], d["l1t"], d["l2t"], 128)
    rng = synth.rng_for(46)
    rows = rng.integers(0, 10, 50)
    cols = rng.integers(0, 40, 50)
    y = oracle_lib.dual_linear_grouped_sampled(d["x"], d["w_res"], d["l1t"], d["l2t"], 128, rows, cols)
    assert (y == full["y"][rows, cols]).all()


# ---------------------------------------------------------------- W4A8 (8-bit activations, q_max = 127)

def test_a8_hand_worked(oracle_lib):
    with open(os.path.join(GOLDEN, "w4a8_layer.json")) as f:
        gd = json.load(f)
    x = np.array(gd["x"], np.float16)
    out = oracle_lib.dual_linear_a8(x, np.array(gd["w_res"], np.float32), None, None)
    assert out["qx"].tolist() == gd["qx"] and out["sx"].astype(np.float64).tolist() == gd["sx"]
    assert oracle_lib.unpack_codes(out["qw_packed"]).tolist() == gd["qw"]
    assert out["sw"].astype(np.float64).tolist() == gd["sw"]
    assert out["acc"].tolist() == gd["acc"] and out["y"].tolist() == gd["y"]


def test_a8_rational_bruteforce(oracle_lib):
    """Codes and scales of the 8-bit quantizer from exact rationals (binary32 roundings
    decided by the rational model), the integer sum by brute force, Y exactly."""
    rng = synth.rng_for(50)
    b, m, n, r = 4, 24, 6, 3
    x = (rng.standard_normal((b, m)) * np.array([1.0] * 20 + [40.0] * 4)).astype(np.float16)
    x[2] = 0
    w = (rng.standard_t(3, size=(n, m)) * 0.02).astype(np.float32)
    l1t = rng.standard_normal((r, m)).astype(np.float16)
    l2t = rng.standard_normal((n, r)).astype(np.float16)
    out = oracle_lib.dual_linear_a8(x, w, l1t, l2t)
    qw = oracle_lib.unpack_codes(out["qw_packed"])
    xf = [[F(float(v)) for v in row] for row in x]
    for i in range(b):
        s, q = ratmodel.quantize(xf[i], q_max=127)
        assert F(float(out["sx"][i])) == s and out["qx"][i].tolist() == q
    l1 = [[F(float(v)) for v in row] for row in l1t]
    l2 = [[F(float(v)) for v in row] for row in l2t]
    for i in range(b):
        t = [sum(xf[i][k] * l1[u][k] for k in range(m)) for u in range(r)]
        for j in range(n):
            acc = sum(int(out["qx"][i, k]) * int(qw[j, k]) for k in range(m))
            assert out["acc"][i, j] == acc
            y = F(float(out["sx"][i])) * F(float(out["sw"][j])) * acc + sum(t[u] * l2[j][u] for u in range(r))
            assert abs(float(y) - out["y"][i, j]) <= 1e-12 * max(1.0, abs(float(y)))


def test_a8_max_code_is_127_for_every_fp16_amax(oracle_lib):
    bits = np.arange(1, 0x7C00, dtype=np.uint16)  # every positive finite fp16
    amax = bits.view(np.float16)
    x = np.stack([amax, -amax, np.zeros_like(amax)], axis=1)
    q, s = oracle_lib.quantize_act_a8(x)
    assert (q[:, 0] == 127).all() and (q[:, 1] == -127).all() and (q[:, 2] == 0).all()
    assert (s == (amax.astype(np.float32) / np.float32(127))).all()


def test_a8_invariants(oracle_lib):
    rng = synth.rng_for(51)
    x = rng.standard_normal((32, 64)).astype(np.float16)
    q, s = oracle_lib.quantize_act_a8(x)
    qn, sn = oracle_lib.quantize_act_a8(-x)
    assert (qn == -q).all() and (sn == s).all()
    for e in (-3, 4):
        q2, s2 = oracle_lib.quantize_act_a8((x.astype(np.float32) * 2.0 ** e).astype(np.float16))
        assert (q2 == q).all() and (s2 == s * np.float32(2.0 ** e)).all()
    # within half a step: |x - s q| <= s / 2
    assert (np.abs(x.astype(np.float64) - s[:, None].astype(np.float64) * q) <= s[:, None] / 2 * (1 + 1e-6)).all()


def test_a8_library_matmul_and_sampled(oracle_lib):
    d = synth.make_random(9, 256, 40, 16, seed=52)
    out = oracle_lib.dual_linear_a8(d["x"], d["w_res"], d["l1t"], d["l2t"])
    qw = oracle_lib.unpack_codes(out["qw_packed"]).astype(np.int64)
    assert (out["acc"] == out["qx"].astype(np.int64) @ qw.T).all()
    lr = oracle_lib.lowrank_out(oracle_lib.lowrank_t(d["x"], d["l1t"]), d["l2t"])
    ref = out["sx"].astype(np.float64)[:, None] * out["sw"].astype(np.float64)[None, :] * out["acc"] + lr
    np.testing.assert_allclose(out["y"], ref, rtol=1e-15, atol=1e-12)
    rng = synth.rng_for(53)
    rows, cols = rng.integers(0, 9, 40), rng.integers(0, 40, 40)
    acc, y = oracle_lib.dual_linear_a8_sampled(d["x"], d["w_res"], d["l1t"], d["l2t"], rows, cols)
    assert (acc == out["acc"][rows, cols]).all() and (y == out["y"][rows, cols]).all()


# ---------------------------------------------------------------- offline folding of Q and G

def _qg(m, r, seed):
    rng = synth.rng_for(seed)
    q, _ = np.linalg.qr(rng.standard_normal((m, m)))
    g = np.eye(r) + 0.3 * rng.standard_normal((r, r))
    return q, g


def test_fold_invariance_and_eckart_young(oracle_lib):
    """(X Q)(U' V' + R') = X W for any orthogonal Q and invertible G (the split is exact
    against the stored factors); U' V' = Q^T U V does not depend on G; and ||R'||_F is the
    tail of the spectrum (Eckart-Young) up to the fp16 rounding of the factors."""
    rng = synth.rng_for(60)
    n, m, r = 40, 48, 8
    w = (rng.standard_normal((n, m)) * np.linspace(2.0, 0.1, m)[None, :]).astype(np.float32)
    x = rng.standard_normal((5, m))
    q, g = _qg(m, r, 61)
    l1t, l2t, w_res = oracle_lib.fold_split(w, r, q, g)
    uv = l1t.T.astype(np.float64) @ l2t.T.astype(np.float64)          # U' V'  (m x n)
    total = uv + w_res.T.astype(np.float64)                            # U' V' + R'
    ref = x @ w.T.astype(np.float64)
    np.testing.assert_allclose((x @ q) @ total, ref, rtol=0, atol=1e-5 * np.abs(ref).max())
    # G cancels in the product of the factors
    l1b, l2b, _ = oracle_lib.fold_split(w, r, q, np.eye(r))
    uv_b = l1b.T.astype(np.float64) @ l2b.T.astype(np.float64)
    np.testing.assert_allclose(uv, uv_b, rtol=0, atol=5e-3 * np.abs(uv_b).max())
    s = np.linalg.svd(w.astype(np.float64), compute_uv=False)
    tail = np.sqrt((s[r:] ** 2).sum())
    assert abs(np.linalg.norm(w_res.astype(np.float64)) - tail) <= 2e-3 * s[0]


def test_fold_identity_and_rank_zero(oracle_lib):
    """Q = I and G = I give the plain split: the factors span the top-r singular space and
    the residual is W minus their product; r = 0 leaves W whole."""
    rng = synth.rng_for(62)
    w = rng.standard_normal((24, 32)).astype(np.float32)
    l1t, l2t, w_res = oracle_lib.fold_split(w, 4, None, None)
    np.testing.assert_allclose(w_res.astype(np.float64) + l2t.astype(np.float64) @ l1t.astype(np.float64),
                               w.astype(np.float64), rtol=0, atol=1e-6)
    u, s, vt = np.linalg.svd(w.T.astype(np.float64))
    proj = u[:, :4] @ u[:, :4].T  # the factors' column space is the top-4 left singular space of W
    np.testing.assert_allclose(proj @ l1t.T.astype(np.float64), l1t.T.astype(np.float64), atol=2e-3)
    l1t0, l2t0, w_res0 = oracle_lib.fold_split(w, 0, None, None)
    assert l1t0.shape == (0, 32) and l2t0.shape == (24, 0) and (w_res0 == w).all()


# ---- range guards of the error budget (the int32 accumulator, the fp16 outputs) ----

def test_require_i32_accepts_the_accumulator_range(oracle_lib):
    lib = oracle_lib._load()
    for v in (0, 1, -1, 49 * 131072, -(49 * 131072), (1 << 31) - 1, -(1 << 31) + 1):
        assert lib.orc_require_i32(v) == v


@pytest.mark.parametrize("v", [1 << 31, -(1 << 31), 1 << 40])
def test_require_i32_aborts_outside_int32(oracle_lib, v):
    """An integer sum the int32 accumulator could not hold stops the oracle (in a child
    process, so the abort does not take the test runner with it)."""
    import subprocess
    import sys
    code = ("import oracle; oracle._load().orc_require_i32(%d); print('returned')" % v)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode != 0 and "returned" not in r.stdout
    assert "outside the int32 accumulator range" in r.stderr


def test_oracle_rejects_outputs_beyond_fp16(oracle_lib):
    """A layer whose exact output exceeds the fp16 range is refused where Y is formed."""
    x = np.zeros((1, 128), np.float16)
    x[0, 0] = 60000.0
    w = np.zeros((16, 128), np.float32)
    w[0, 0] = 2.0  # Y[0][0] ~ 1.2e5
    with pytest.raises(AssertionError, match="fp16 range"):
        oracle_lib.dual_linear(x, w, None, None)
    w[0, 0] = 0.5  # Y[0][0] ~ 3e4: accepted
    assert np.isfinite(oracle_lib.dual_linear(x, w, None, None)["y"]).all()


def test_synth_headroom_check():
    """The generator's Cauchy-Schwarz bound accepts the configs and rejects a layer whose
    products could overflow fp16."""
    import synth
    d = synth.make_layer("tiny", keep_w=True)
    synth.check_fp16_headroom(d["x"], d["w"], d["l1t"])
    with pytest.raises(AssertionError, match="fp16 range"):
        synth.check_fp16_headroom(d["x"], d["w"] * 1000.0, d["l1t"])
    with pytest.raises(AssertionError, match="fp16 range"):
        synth.check_fp16_headroom(d["x"], d["w"], d["l1t"] * 1000.0)
