"""Parity of the int4 low-rank variant (TwinQuant page 1, section 4.3) with the oracle.

Bit for bit: the low-rank codes and scales, c, the integer H, Q_H and s_H; Y within
2e-3 * max|Y_oracle|.
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import w4a4_rank_gemm_amd as twq
from tests import layers
from tests.panels import from_panels, to_panels

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
Y_TOL = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.cpu().numpy()


def run_lr4(d):
    """The int4 low-rank layer on the GPU: the activation launch through the product entry
    point and through the test export that also stores H (they must agree bit for bit),
    the fused launch, and the one-call layer (bitwise equal to the two calls)."""
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    dev = torch.device("cuda:0")
    x = torch.from_numpy(d["x"]).to(dev)
    w = torch.from_numpy(d["w_res"]).to(dev)
    l1t = torch.from_numpy(d["l1t"]).to(dev)
    l2t = torch.from_numpy(d["l2t"]).to(dev)
    qw, sw = twq.pack_weight(w)
    f = twq.pack_lowrank_int4(l1t, l2t)
    qx, sx, qh, sh = twq.quantize_act_lr4(x, f)
    qx_d, sx_d, qh_d, sh_d, h = twq.quantize_act_lr4(x, f, debug_h=True)
    y = twq.dual_linear_lr4(qx, sx, qw, sw, qh, sh, f["ql2"])
    y1 = twq.linear_lr4(x, qw, sw, f)
    torch.cuda.synchronize()
    for name, a_, b_ in (("qx", qx, qx_d), ("sx", sx, sx_d), ("qh", qh, qh_d), ("sh", sh, sh_d)):
        assert torch.equal(a_, b_), f"{name}: product entry point and test export differ"
    assert torch.equal(y, y1), "twq_linear_lr4 differs from twq_quantize_act_lr4 + twq_dual_linear_lr4"
    return {"qx": qx, "sx": sx, "f": f, "h": h, "qh": qh, "sh": sh, "y": y}


def check_factors(d, g):
    ref = oracle.quantize_lowrank(d["l1t"], d["l2t"])
    for k in ("ql1_packed", "sl1", "ql2_packed", "sl2", "c"):
        gk = k.replace("_packed", "")
        want = to_panels(ref[k]) if k == "ql1_packed" else ref[k]  # Q_L1 is H's weight operand
        assert np.array_equal(_np(g["f"][gk]), want), k
    return ref


def test_lr4_hand_worked_padded():
    """The hand-worked int4 low-rank layer, zero-padded to m = 128, n = 16, r = 32:
    padded ranks have zero factors (c = 0, h = 0), which changes no value."""
    with open(os.path.join(GOLDEN, "lr4_layer.json")) as fh:
        gld = json.load(fh)
    x = np.zeros((1, 128), np.float16)
    x[:, :4] = np.array(gld["x"])
    w = np.zeros((16, 128), np.float32)
    w[:2, :4] = np.array(gld["w_res"])
    l1t = np.zeros((32, 128), np.float16)
    l1t[:2, :4] = np.array(gld["l1t"])
    l2t = np.zeros((16, 32), np.float16)
    l2t[:2, :2] = np.array(gld["l2t"])
    g = run_lr4({"x": x, "w_res": w, "l1t": l1t, "l2t": l2t})
    ql1 = oracle.unpack_codes(from_panels(_np(g["f"]["ql1"])))
    assert ql1[:2, :4].tolist() == gld["ql1"] and (ql1[2:] == 0).all()
    ql2 = oracle.unpack_codes(_np(g["f"]["ql2"]))
    assert ql2[:2, :2].tolist() == gld["ql2"] and (ql2[:, 2:] == 0).all()
    assert _np(g["f"]["sl1"])[:2].astype(np.float64).tolist() == gld["sl1"]
    assert _np(g["f"]["sl2"])[:2].astype(np.float64).tolist() == gld["sl2"]
    assert _np(g["f"]["c"])[:2].astype(np.float64).tolist() == gld["c"]
    assert _np(g["h"])[:, :2].tolist() == gld["h"] and (_np(g["h"])[:, 2:] == 0).all()
    qh = oracle.unpack_codes(_np(g["qh"]))
    assert qh[:, :2].tolist() == gld["qh"] and (qh[:, 2:] == 0).all()
    assert _np(g["sh"]).astype(np.float64).tolist() == gld["sh"]
    y = _np(g["y"]).astype(np.float64)
    want = np.array(gld["y"])
    assert np.abs(y[:, :2] - want).max() <= Y_TOL * np.abs(want).max()
    assert (y[:, 2:] == 0).all()


SHAPES = [(16, 512, 512, 32), (17, 384, 80, 64), (1, 256, 256, 256), (130, 640, 144, 96),
          (32, 1024, 8192, 128), (64, 512, 8192, 32), (200, 256, 176, 160),
          # the remaining few-token tilings (2x1 blocks; 4x4, pipelined) and b just above 64
          (16, 512, 8192, 32), (64, 256, 12304, 64), (90, 384, 272, 32)]


@pytest.mark.parametrize("b,m,n,r", SHAPES)
def test_lr4_full_compare(b, m, n, r):
    _say(f"lr4 b={b} m={m} n={n} r={r}")
    d = synth.make_random(b, m, n, r, seed=3 * b + r)
    g = run_lr4(d)
    check_factors(d, g)
    _, qxp_ref, sx_ref = oracle.quantize_act(d["x"])
    assert np.array_equal(_np(g["qx"]), qxp_ref) and np.array_equal(_np(g["sx"]), sx_ref), "Q_X, s_X"
    ref = oracle.dual_linear_lr4(d["x"], d["w_res"], d["l1t"], d["l2t"])
    assert np.array_equal(_np(g["h"]).astype(np.int64), ref["h"]), "H"
    assert np.array_equal(_np(g["qh"]), ref["qh_packed"]), "Q_H"
    assert np.array_equal(_np(g["sh"]), ref["sh"]), "s_H"
    yo = ref["y"]
    err = np.abs(_np(g["y"]).astype(np.float64) - yo).max()
    assert err <= Y_TOL * np.abs(yo).max(), (err, np.abs(yo).max())


def test_lr4_rank0_is_plain_w4a4():
    d = synth.make_random(20, 512, 64, 0, seed=31)
    dev = torch.device("cuda:0")
    qx, sx, _ = twq.quantize_act(torch.from_numpy(d["x"]).to(dev))
    qw, sw = twq.pack_weight(torch.from_numpy(d["w_res"]).to(dev))
    L = twq.lib()
    y = torch.empty((20, 64), dtype=torch.float16, device=dev)
    p = twq._ptr
    assert L.twq_dual_linear_lr4(p(qx), p(sx), p(qw), p(sw), None, None, None, 0, p(y), 20, 512, 64, None) == 0
    y_plain = twq.dual_linear(qx, sx, qw, sw)
    torch.cuda.synchronize()
    assert torch.equal(y, y_plain)


@pytest.mark.parametrize("name", ["70b_gate_up_decode", "70b_gate_up_prefill", "gate_up_prefill", "down_prefill"])
def test_lr4_full_size_sampled(name):
    """Full-size layers with the int4 low-rank branch (the 70B-size gate/up layer at both
    token counts, the 8B gate/up and down layers at prefill): factors, Q_X, s_X, H, Q_H
    and s_H compared whole, Y at 384 sampled positions."""
    _say(f"lr4 {name}: generating inputs")
    d = layers.layer(name)
    b, m = d["x"].shape
    n, r = d["w_res"].shape[0], d["l1t"].shape[0]
    _say(f"lr4 {name}: GPU b={b} m={m} n={n} r={r}")
    g = run_lr4(d)
    ref_f = check_factors(d, g)
    qx, qxp, sx = oracle.quantize_act(d["x"])
    assert np.array_equal(_np(g["qx"]), qxp) and np.array_equal(_np(g["sx"]), sx), "Q_X, s_X"
    rq = oracle.lowrank_requant(qx, sx, ref_f["ql1"], ref_f["c"])
    assert np.array_equal(_np(g["h"]).astype(np.int64), rq["h"]), "H"
    assert np.array_equal(_np(g["qh"]), rq["qh_packed"]), "Q_H"
    assert np.array_equal(_np(g["sh"]), rq["sh"]), "s_H"
    rng = synth.rng_for(200 + b)
    rows = rng.integers(0, b, 384)
    cols = rng.integers(0, n, 384)
    top = int(torch.argmax(g["y"].abs().float()).item())
    rows[:5] = [0, 0, b - 1, b - 1, top // n]
    cols[:5] = [0, n - 1, 0, n - 1, top % n]
    _, _, y_ref = oracle.dual_linear_lr4_sampled(d["x"], d["w_res"], d["l1t"], d["l2t"], rows, cols)
    ri = torch.from_numpy(rows).to(g["y"].device)
    ci = torch.from_numpy(cols).to(g["y"].device)
    y = g["y"][ri, ci].cpu().numpy().astype(np.float64)
    scale = np.abs(y_ref).max()
    err = np.abs(y - y_ref).max()
    assert err <= Y_TOL * scale, (err, scale)
    _say(f"  sampled max|Y-Y_or| = {err:.3g}, max|Y_or| over samples = {scale:.3g}")
