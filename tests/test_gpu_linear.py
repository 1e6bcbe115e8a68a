"""The one-call layer (twq_linear) against the oracle and against the separate calls.

twq_linear adds the partial sums of T in the epilogue for few tokens (in slice order,
as twq_quantize_act does), so its Y equals twq_quantize_act + twq_dual_linear value for
value; both are checked against the oracle to 2e-3 * max|Y_oracle|.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import w4a4_rank_gemm_amd as twq

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(d):
    dev = torch.device("cuda:0")
    x = torch.from_numpy(d["x"]).to(dev)
    qw, sw = twq.pack_weight(torch.from_numpy(d["w_res"]).to(dev))
    r = d["l1t"].shape[0]
    l1t = torch.from_numpy(d["l1t"]).to(dev) if r else None
    l2t = torch.from_numpy(d["l2t"]).to(dev) if r else None
    y1 = twq.linear(x, qw, sw, l1t, l2t)
    qx, sx, t = twq.quantize_act(x, l1t)
    y2 = twq.dual_linear(qx, sx, qw, sw, t, l2t)
    torch.cuda.synchronize()
    return y1.cpu().numpy(), y2.cpu().numpy()


# few tokens (partial sums of T added in the epilogue, 2 to 16 slices, one or two
# channel tiles per CTA), the decode shapes that need T whole, and many tokens
SHAPES = [(16, 4096, 4096, 32), (16, 512, 512, 16), (1, 4096, 272, 32), (5, 2048, 16384, 64),
          (16, 8192, 1024, 128), (24, 4096, 4096, 32), (32, 1024, 8192, 64), (48, 2048, 512, 16),
          (64, 4096, 2048, 32), (200, 1024, 528, 48), (16, 4096, 4096, 0), (3, 16384, 256, 256),
          (29, 4096, 12304, 32),  # 2x2 blocks reading Q_X from LDS with T's slices in the epilogue
          # many tokens on grids of at least 4 x 256 tiles (the two-stage ring of the 32 x 32
          # kernel): ragged tokens and channels, a single K stage, a half low-rank step (r = 48)
          (1000, 128, 16400, 48), (1100, 384, 15008, 16),
          # the three-stage ring with a single K stage
          (300, 128, 272, 48)]


@pytest.mark.parametrize("b,m,n,r", SHAPES)
def test_linear_matches_split_calls_and_oracle(b, m, n, r):
    _say(f"twq_linear b={b} m={m} n={n} r={r}")
    d = synth.make_random(b, m, n, r, seed=11 * b + r)
    y1, y2 = _run(d)
    assert np.array_equal(y1, y2), "twq_linear differs from twq_quantize_act + twq_dual_linear"
    ref = oracle.dual_linear(d["x"], d["w_res"], d["l1t"], d["l2t"])["y"]
    err = np.abs(y1.astype(np.float64) - ref).max()
    assert err <= Y_TOL * np.abs(ref).max(), (err, np.abs(ref).max())


def test_linear_headline_config_full():
    """The o_proj decode layer (b=16, m=n=4096, r=32), every output against the oracle."""
    d = synth.make_layer("o_proj_decode")
    y1, y2 = _run(d)
    assert np.array_equal(y1, y2)
    ref = oracle.dual_linear(d["x"], d["w_res"], d["l1t"], d["l2t"])["y"]
    err = np.abs(y1.astype(np.float64) - ref).max()
    assert err <= Y_TOL * np.abs(ref).max(), (err, np.abs(ref).max())


def test_linear_repeat_bitwise():
    d = synth.make_random(16, 4096, 1024, 32, seed=5)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(d["x"]).to(dev)
    qw, sw = twq.pack_weight(torch.from_numpy(d["w_res"]).to(dev))
    l1t, l2t = torch.from_numpy(d["l1t"]).to(dev), torch.from_numpy(d["l2t"]).to(dev)
    ys = [twq.linear(x, qw, sw, l1t, l2t).cpu() for _ in range(3)]
    assert all(torch.equal(ys[0], y) for y in ys[1:])


@pytest.mark.parametrize("name", ["70b_gate_up_decode", "70b_gate_up_prefill"])
def test_linear_70b_full_size(name):
    """twq_linear at both 70B-size gate/up shapes, as the benchmark runs it: Y bitwise
    equal to twq_quantize_act + twq_dual_linear, and within 2e-3 * max|Y_or| of the oracle
    at 384 sampled positions (plus the corners and the largest |Y|)."""
    from tests import layers
    _say(f"twq_linear {name}: generating inputs")
    d = layers.layer(name)
    b, m = d["x"].shape
    n, r = d["w_res"].shape[0], d["l1t"].shape[0]
    _say(f"twq_linear {name}: GPU b={b} m={m} n={n} r={r}")
    y1, y2 = _run(d)
    assert np.array_equal(y1, y2), "twq_linear differs from twq_quantize_act + twq_dual_linear"
    rng = synth.rng_for(900 + b)
    rows = rng.integers(0, b, 384)
    cols = rng.integers(0, n, 384)
    top = int(np.argmax(np.abs(y1.astype(np.float32))))
    rows[:5] = [0, 0, b - 1, b - 1, top // n]
    cols[:5] = [0, n - 1, 0, n - 1, top % n]
    _, y_ref = oracle.dual_linear_sampled(d["x"], d["w_res"], d["l1t"], d["l2t"], rows, cols)
    y = y1[rows, cols].astype(np.float64)
    scale = np.abs(y_ref).max()
    err = np.abs(y - y_ref).max()
    assert err <= Y_TOL * scale, (err, scale)
    _say(f"  sampled max|Y-Y_or| = {err:.3g}, max|Y_or| over samples = {scale:.3g}")
