"""Parity of the group-wise path (groups of 128 along K, as in TwinQuant page 1, section
5.1 and page 2, section 5.1) with the CPU oracle, through the C ABI, on an MI355X.

Bar: the 4-bit codes and every group scale bit for bit (the library's scales are
group-major, the oracle's row-major, so they are compared transposed); Y within
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
from tests.test_gpu_quant_ties import _row

pytestmark = pytest.mark.gpu

G = 128
Y_TOL = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np(t):
    return None if t is None else t.cpu().numpy()


def run_grouped(d):
    dev = torch.device("cuda:0")
    x = torch.from_numpy(d["x"]).to(dev)
    w = torch.from_numpy(d["w_res"]).to(dev)
    r = d["l1t"].shape[0]
    l1t = torch.from_numpy(d["l1t"]).to(dev) if r else None
    l2t = torch.from_numpy(d["l2t"]).to(dev) if r else None
    qx, sx, t = twq.quantize_act_grouped(x, l1t)
    qw, sw = twq.pack_weight_grouped(w)
    y = twq.dual_linear_grouped(qx, sx, qw, sw, t, l2t)
    y1 = twq.linear_grouped(x, qw, sw, l1t, l2t)
    torch.cuda.synchronize()
    return {"qx": qx, "sx": sx, "qw": qw, "sw": sw, "y": y, "y1": y1}


def check_codes(d, g):
    _, qxp, sx = oracle.quantize_act_grouped(d["x"], G)
    assert np.array_equal(_np(g["qx"]), qxp), "Q_X bytes"
    assert np.array_equal(_np(g["sx"]), sx.T), "s_X"
    _, qwp, sw = oracle.quantize_weight_grouped(d["w_res"], G)
    assert np.array_equal(_np(g["qw"]), to_panels(qwp)), "Q_W bytes"
    assert np.array_equal(_np(g["sw"]), sw.T), "s_W"
    assert torch.equal(g["y1"], g["y"]), "twq_linear_grouped differs from the split calls"


def check_y(y_gpu, y_ref):
    y = y_gpu.astype(np.float64)
    assert np.isfinite(y).all()
    err = np.abs(y - y_ref).max() if y_ref.size else 0.0
    scale = np.abs(y_ref).max() if y_ref.size else 0.0
    assert err <= Y_TOL * scale + 1e-30, f"max|Y - Y_or| = {err} > {Y_TOL} * {scale}"
    return err, scale


# decode and prefill launches, ragged tokens and channels, a single group, rank 0 and
# the largest rank, ranks not a multiple of 32, few-token shapes with wide channel tiles
SHAPES = [
    (1, 128, 16, 0), (16, 4096, 4096, 32), (17, 384, 48, 32), (33, 512, 80, 48), (64, 1024, 128, 128),
    (130, 640, 144, 16), (200, 256, 272, 256), (129, 1152, 208, 64), (32, 1024, 8192, 64),
    (16, 512, 16384, 16), (5, 2048, 16384, 64), (300, 4096, 1040, 32), (27, 512, 8208, 48),
    # wide few-token grids: 2x2 and 4x4 blocks of 16 per CTA, a partial last channel tile
    (27, 384, 24592, 32), (64, 256, 12304, 48), (48, 512, 8192, 32),
    # tilings that read Q_X from LDS at m <= 4096: 2x1, 2x2 and 4x4 blocks, ragged tokens
    (9, 2048, 8192, 32), (30, 3072, 24576, 32), (61, 640, 12304, 16),
    # rows past 16384 elements, few and many tokens
    (3, 32768, 48, 32), (130, 20480, 80, 16),
]


@pytest.mark.parametrize("b,m,n,r", SHAPES + _random_shapes(8, seed=2027))
def test_grouped_matches_oracle(b, m, n, r):
    _say(f"grouped b={b} m={m} n={n} r={r}")
    d = synth.make_random(b, m, n, r, seed=500 + b + n)
    g = run_grouped(d)
    check_codes(d, g)
    ref = oracle.dual_linear_grouped(d["x"], d["w_res"], d["l1t"], d["l2t"], G)
    err, scale = check_y(_np(g["y"]), ref["y"])
    _say(f"  max|Y-Y_or| = {err:.3g}, max|Y_or| = {scale:.3g}")


def test_grouped_zero_groups_and_rows():
    """All-zero groups (s = 0, codes 0) next to non-zero ones, an all-zero token and an
    all-zero output channel."""
    d = synth.make_random(40, 512, 96, 32, seed=601)
    d["x"][3] = 0
    d["x"][7, 128:256] = 0
    d["w_res"][5] = 0
    d["w_res"][9, 256:384] = 0
    g = run_grouped(d)
    check_codes(d, g)
    assert (_np(g["sx"])[1, 7] == 0) and (_np(g["sw"])[2, 9] == 0)
    ref = oracle.dual_linear_grouped(d["x"], d["w_res"], d["l1t"], d["l2t"], G)
    check_y(_np(g["y"]), ref["y"])


@pytest.mark.parametrize("b", [3, 256])
def test_grouped_quantizer_ties(b):
    """Every group holds exact ties and fp16 neighbours of the half-integers of its own
    scale; the group-wise quantizer must round them as the oracle does."""
    rng = synth.rng_for(4300 + b)
    m = 1024
    rows = []
    for i in range(b):
        amaxes = [np.float16(7 * 2.0 ** rng.integers(-6, 5)) if k % 2 == 0 else np.float16(rng.uniform(0.01, 600.0))
                  for k in range(m // G)]
        rows.append(np.concatenate([_row(a, G, rng) for a in amaxes]))
    x = np.stack(rows)
    _, qxp, sx = oracle.quantize_act_grouped(x, G)
    qx_g, sx_g, _ = twq.quantize_act_grouped(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_np(sx_g), sx.T)
    assert np.array_equal(_np(qx_g), qxp)


def test_grouped_repeat_bitwise():
    d = synth.make_random(48, 2048, 1024, 64, seed=602)
    a = run_grouped(d)
    b = run_grouped(d)
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["y1"], b["y1"])


BIG = ["o_proj_decode", "gate_up_prefill", "70b_gate_up_decode", "down_prefill", "70b_gate_up_prefill"]


@pytest.mark.parametrize("name", BIG)
def test_grouped_full_size_sampled(name):
    """Full-size layer shapes: every code and group scale compared whole, Y at 384 sampled
    positions (plus the corners and the largest |Y|)."""
    _say(f"grouped {name}: generating inputs")
    d = layers.layer(name)
    b, m = d["x"].shape
    n = d["w_res"].shape[0]
    _say(f"grouped {name}: GPU b={b} m={m} n={n} r={d['l1t'].shape[0]}")
    g = run_grouped(d)
    check_codes(d, g)
    rng = synth.rng_for(200 + b)
    rows = rng.integers(0, b, 384)
    cols = rng.integers(0, n, 384)
    top = int(torch.argmax(g["y"].abs().float()).item())
    rows[:5] = [0, 0, b - 1, b - 1, top // n]
    cols[:5] = [0, n - 1, 0, n - 1, top % n]
    y_ref = oracle.dual_linear_grouped_sampled(d["x"], d["w_res"], d["l1t"], d["l2t"], G, rows, cols)
    ri = torch.from_numpy(rows).to(g["y"].device)
    ci = torch.from_numpy(cols).to(g["y"].device)
    err, scale = check_y(g["y"][ri, ci].cpu().numpy(), y_ref)
    _say(f"  sampled max|Y-Y_or| = {err:.3g}, max|Y_or| over samples = {scale:.3g}")
