"""Parity of the W4A8 path (8-bit per-token activations, q_max = 127, 4-bit residual
weight; TwinQuant page 1, section 5.1) with the CPU oracle, through the C ABI, on an
MI355X.

Bar: the 8-bit codes, the scales and the int32 accumulator bit for bit; Y within
2e-3 * max|Y_oracle|; the one-call layer bitwise equal to the split calls.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import w4a4_rank_gemm_amd as twq
from tests import layers
from tests.test_gpu_parity import _random_shapes
from tests.panels import to_panels

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np(t):
    return None if t is None else t.cpu().numpy()


def run_a8(d, debug_acc=True):
    dev = torch.device("cuda:0")
    x = torch.from_numpy(d["x"]).to(dev)
    w = torch.from_numpy(d["w_res"]).to(dev)
    r = d["l1t"].shape[0]
    l1t = torch.from_numpy(d["l1t"]).to(dev) if r else None
    l2t = torch.from_numpy(d["l2t"]).to(dev) if r else None
    qx, sx, t = twq.quantize_act_a8(x, l1t)
    qw, sw = twq.pack_weight(w)
    y = twq.dual_linear_a8(qx, sx, qw, sw, t, l2t)
    y1 = twq.linear_a8(x, qw, sw, l1t, l2t)
    acc = twq.debug_residual_acc_a8(qx, qw) if debug_acc else None
    torch.cuda.synchronize()
    return {"qx": qx, "sx": sx, "qw": qw, "sw": sw, "y": y, "y1": y1, "acc": acc}


def check_y(y_gpu, y_ref):
    y = y_gpu.astype(np.float64)
    assert np.isfinite(y).all()
    err = np.abs(y - y_ref).max() if y_ref.size else 0.0
    scale = np.abs(y_ref).max() if y_ref.size else 0.0
    assert err <= Y_TOL * scale + 1e-30, f"max|Y - Y_or| = {err} > {Y_TOL} * {scale}"
    return err, scale


SHAPES = [
    (1, 128, 16, 0), (16, 4096, 4096, 32), (17, 384, 48, 32), (33, 512, 80, 48), (64, 1024, 128, 128),
    (130, 640, 144, 16), (200, 256, 272, 256), (129, 1152, 208, 64), (32, 1024, 8192, 64),
    (16, 512, 16384, 16), (5, 2048, 16384, 64), (300, 4096, 1040, 32), (27, 512, 8208, 48),
    # wide few-token grids: 2x2 and 4x4 blocks of 16 per CTA, a partial last channel tile
    (27, 384, 24592, 32), (64, 256, 12304, 48), (48, 512, 8192, 32),
    # rows past 16384 elements (two-pass quantizer) and 128-chunk few-token slices
    (3, 32768, 48, 32), (130, 20480, 80, 16), (16, 8192, 96, 32),
]


@pytest.mark.parametrize("b,m,n,r", SHAPES + _random_shapes(8, seed=2028))
def test_a8_matches_oracle(b, m, n, r):
    _say(f"a8 b={b} m={m} n={n} r={r}")
    d = synth.make_random(b, m, n, r, seed=700 + b + n)
    g = run_a8(d)
    ref = oracle.dual_linear_a8(d["x"], d["w_res"], d["l1t"], d["l2t"])
    assert np.array_equal(_np(g["qx"]), ref["qx"]), "Q_X codes"
    assert np.array_equal(_np(g["sx"]), ref["sx"]), "s_X"
    assert np.array_equal(_np(g["qw"]), to_panels(ref["qw_packed"])) and np.array_equal(_np(g["sw"]), ref["sw"])
    assert np.array_equal(_np(g["acc"]).astype(np.int64), ref["acc"]), "int32 accumulator"
    err, scale = check_y(_np(g["y"]), ref["y"])
    assert torch.equal(g["y1"], g["y"]), "twq_linear_a8 differs from the split calls"
    _say(f"  max|Y-Y_or| = {err:.3g}, max|Y_or| = {scale:.3g}")


def test_a8_extreme_codes_and_zero_rows():
    """Codes of +-127 on every element (the largest accumulator), an all-zero token and an
    all-zero output channel."""
    d = synth.make_random(40, 2048, 96, 16, seed=801)
    d["x"][0] = np.float16(3.0)
    d["x"][1] = np.float16(-3.0)
    d["x"][5] = 0
    d["w_res"][0] = np.float32(0.5)
    d["w_res"][7] = 0
    g = run_a8(d)
    ref = oracle.dual_linear_a8(d["x"], d["w_res"], d["l1t"], d["l2t"])
    assert np.array_equal(_np(g["qx"]), ref["qx"]) and np.array_equal(_np(g["acc"]).astype(np.int64), ref["acc"])
    assert ref["acc"][0, 0] == 127 * 7 * 2048 and ref["acc"][1, 0] == -127 * 7 * 2048
    check_y(_np(g["y"]), ref["y"])


def test_a8_quantizer_ties():
    """Rows holding exact ties and fp16 neighbours of the half-integers of their scale at
    q_max = 127 (the fast quantizer's division fallback band)."""
    rng = synth.rng_for(811)
    rows = []
    for j in range(64):
        amax = np.float16(127 * 2.0 ** rng.integers(-8, 6)) if j % 2 == 0 else np.float16(rng.uniform(0.05, 4000.0))
        s = np.float32(np.float32(amax) / np.float32(127))
        vals = [amax, -amax]
        for k in range(-127, 127, 5):
            h = np.float16((k + 0.5) * float(s))
            for _ in range(2):
                h = np.nextafter(h, np.float16(-np.inf))
            for _ in range(5):
                if abs(float(h)) <= float(amax):
                    vals.append(h)
                h = np.nextafter(h, np.float16(np.inf))
        row = (rng.uniform(-1, 1, 512) * float(amax)).astype(np.float16)
        row[:len(vals)] = np.array(vals, np.float16)[:512]
        row[np.abs(row.astype(np.float32)) > np.float32(amax)] = amax
        rows.append(row)
    x = np.stack(rows)
    q_ref, s_ref = oracle.quantize_act_a8(x)
    qx, sx, _ = twq.quantize_act_a8(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_np(sx), s_ref) and np.array_equal(_np(qx), q_ref)


@pytest.mark.parametrize("name", ["o_proj_decode", "gate_up_prefill", "70b_gate_up_decode", "down_prefill",
                                  "70b_gate_up_prefill"])
def test_a8_full_size_sampled(name):
    _say(f"a8 {name}: generating inputs")
    d = layers.layer(name)
    b, m = d["x"].shape
    n = d["w_res"].shape[0]
    _say(f"a8 {name}: GPU b={b} m={m} n={n} r={d['l1t'].shape[0]}")
    g = run_a8(d, debug_acc=False)
    q_ref, s_ref = oracle.quantize_act_a8(d["x"])
    assert np.array_equal(_np(g["qx"]), q_ref) and np.array_equal(_np(g["sx"]), s_ref)
    assert torch.equal(g["y1"], g["y"])
    rng = synth.rng_for(300 + b)
    rows = rng.integers(0, b, 384)
    cols = rng.integers(0, n, 384)
    top = int(torch.argmax(g["y"].abs().float()).item())
    rows[:5] = [0, 0, b - 1, b - 1, top // n]
    cols[:5] = [0, n - 1, 0, n - 1, top % n]
    acc_ref, y_ref = oracle.dual_linear_a8_sampled(d["x"], d["w_res"], d["l1t"], d["l2t"], rows, cols)
    acc = twq.debug_residual_acc_a8(g["qx"], g["qw"])
    ri = torch.from_numpy(rows).to(acc.device)
    ci = torch.from_numpy(cols).to(acc.device)
    assert np.array_equal(acc[ri, ci].cpu().numpy().astype(np.int64), acc_ref)
    err, scale = check_y(g["y"][ri, ci].cpu().numpy(), y_ref)
    _say(f"  sampled max|Y-Y_or| = {err:.3g}, max|Y_or| over samples = {scale:.3g}")
