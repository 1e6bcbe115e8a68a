"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Bar: the 4-bit codes, the scales and the int32 accumulator bit for bit; T within
its fp32 summation bound; Y within 2e-3 * max|Y_oracle| (eqs. (1)-(3) of
TwinQuant, page 1, section 2; fused epilogue of page 1, section 4.3).
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
from tests.panels import to_panels, from_panels

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
Y_TOL = 2e-3


def _dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(d, debug_acc=True):
    dev = _dev()
    x = torch.from_numpy(d["x"]).to(dev)
    w = torch.from_numpy(d["w_res"]).to(dev)
    r = d["l1t"].shape[0]
    l1t = torch.from_numpy(d["l1t"]).to(dev) if r else None
    l2t = torch.from_numpy(d["l2t"]).to(dev) if r else None
    qx, sx, t = twq.quantize_act(x, l1t)
    qw, sw = twq.pack_weight(w)
    y = twq.dual_linear(qx, sx, qw, sw, t, l2t)
    acc = twq.debug_residual_acc(qx, qw) if debug_acc else None
    torch.cuda.synchronize()
    out = {"qx": qx, "sx": sx, "qw": qw, "sw": sw, "t": t, "y": y, "acc": acc}
    return out


def _np(t):
    return None if t is None else t.cpu().numpy()


def check_t(t_gpu, d):
    if t_gpu is None:
        return
    ref = oracle.lowrank_t(d["x"], d["l1t"])
    mag = np.abs(d["x"].astype(np.float64)) @ np.abs(d["l1t"].astype(np.float64)).T
    m = d["x"].shape[1]
    bound = 2.0 * m * 2.0 ** -24 * mag + 1e-30
    err = np.abs(t_gpu.astype(np.float64) - ref)
    assert (err <= bound).all(), f"T error {err.max()} over its fp32 summation bound"


def check_full(d, g):
    ref = oracle.dual_linear(d["x"], d["w_res"], d["l1t"], d["l2t"])
    assert np.array_equal(_np(g["qx"]), ref["qx_packed"]), "Q_X bytes"
    assert np.array_equal(_np(g["sx"]), ref["sx"]), "s_X"
    assert np.array_equal(_np(g["qw"]), to_panels(ref["qw_packed"])), "Q_W bytes"
    assert np.array_equal(_np(g["sw"]), ref["sw"]), "s_W"
    if g["acc"] is not None:
        assert np.array_equal(_np(g["acc"]).astype(np.int64), ref["acc"]), "int32 accumulator"
    check_t(_np(g["t"]), d)
    yo = ref["y"]
    y = _np(g["y"]).astype(np.float64)
    assert np.isfinite(y).all()
    err = np.abs(y - yo).max() if yo.size else 0.0
    scale = np.abs(yo).max() if yo.size else 0.0
    assert err <= Y_TOL * scale + 1e-30, f"max|Y - Y_or| = {err} > {Y_TOL} * {scale}"
    return err, scale


# ------------------------------------------------------------------ hand-worked layer

def test_e6_hand_worked_layer_padded():
    """The hand-worked whole layer, zero-padded to m = 128 and n = 16 (padding changes no value)."""
    with open(os.path.join(GOLDEN, "e6_layer.json")) as f:
        g = json.load(f)
    x = np.zeros((2, 128), np.float16)
    x[:, :4] = np.array(g["x"])
    w = np.zeros((16, 128), np.float32)
    w[:3, :4] = np.array(g["w_res"])
    l1t = np.zeros((16, 128), np.float16)
    l1t[:1, :4] = np.array(g["l1t"])
    l2t = np.zeros((16, 16), np.float16)
    l2t[:3, :1] = np.array(g["l2t"])
    d = {"x": x, "w_res": w, "l1t": l1t, "l2t": l2t}
    out = run_gpu(d)
    qx = oracle.unpack_codes(_np(out["qx"]))
    assert qx[:, :4].tolist() == g["qx"] and (qx[:, 4:] == 0).all()
    assert _np(out["qx"])[:, :2].tolist() == g["qx_packed"]
    assert _np(out["sx"]).astype(np.float64).tolist() == g["sx"]
    qw = oracle.unpack_codes(from_panels(_np(out["qw"])))
    assert qw[:3, :4].tolist() == g["qw"] and (qw[3:] == 0).all()
    assert _np(out["sw"])[:3].astype(np.float64).tolist() == g["sw"]
    assert _np(out["acc"])[:, :3].tolist() == g["acc"]
    assert _np(out["t"])[:, :1].astype(np.float64).tolist() == g["t"]
    y = _np(out["y"]).astype(np.float64)
    assert np.abs(y[:, :3] - np.array(g["y"])).max() <= Y_TOL * np.abs(np.array(g["y"])).max()
    assert (y[:, 3:] == 0).all()


# ------------------------------------------------------------------ configurations, full compare

@pytest.mark.parametrize("name", ["tiny", "o_proj_decode"])
def test_config_full(name):
    _say(f"config {name}")
    d = layers.layer(name)
    err, scale = check_full(d, run_gpu(d))
    _say(f"  max|Y-Y_or| = {err:.3g}, max|Y_or| = {scale:.3g}")


# ragged and edge shapes: tokens not a multiple of any tile, n not a multiple of the
# channel tile, m with a half stage, r not a multiple of 32, rank 0, largest rank
RAGGED = [
    (1, 128, 16, 16), (17, 384, 48, 32), (33, 512, 80, 48), (130, 640, 144, 16),
    (5, 256, 272, 0), (64, 1024, 128, 128), (200, 256, 272, 256), (2, 4096, 32, 32),
    (129, 1152, 208, 64), (16, 256, 256, 240),
    # the many-token kernel from b = 65, while the activation launch keeps its few-token
    # form up to b = 128
    (65, 384, 176, 32), (128, 512, 144, 48),
    # few-token launch shapes whose CTAs own more output tiles than waves
    (32, 1024, 8192, 64), (64, 512, 8192, 32), (16, 512, 16384, 16), (27, 512, 8208, 48),
    # wide few-token grids with a partial last channel tile; 16-tile CTAs (8x2 and 4x4
    # blocks of 16), whose main loop is software-pipelined: 64 K pieces for 8 waves, and
    # 2 pieces for 8 waves (most waves get none)
    (27, 384, 24592, 32), (27, 8192, 24592, 16), (64, 256, 12304, 48),
    # 4x4-block CTAs whose waves read their K slices of Q_X from LDS (a full slice of
    # four pieces a wave; a ragged token count and a partial last channel tile)
    (64, 4096, 14336, 64), (49, 2048, 12304, 32),
    # the other tilings that read Q_X from LDS, each with ragged tokens and uneven pieces
    # per wave: 1x2 and 1x4 blocks of eight waves, 2x4, 2x2 of four waves, 8x2 at m = 8192
    (20, 1536, 1040, 32), (40, 3072, 2000, 48), (57, 2560, 6160, 16), (31, 4096, 9008, 64),
    (50, 1152, 12304, 32), (29, 8192, 24592, 32),
    # rows past 16384 elements (the quantizer's two-pass path, few and many tokens) and
    # few-token slices of 128 chunks staged through LDS
    (3, 32768, 48, 32), (16, 16512, 64, 16), (130, 20480, 80, 16), (16, 8192, 96, 32),
    # many tokens on grids of at least 4 x 256 tiles (two-stage ring), ragged edges
    (1000, 128, 16400, 48), (300, 128, 272, 48),
]


@pytest.mark.parametrize("b,m,n,r", RAGGED)
def test_ragged_shapes(b, m, n, r):
    _say(f"shape b={b} m={m} n={n} r={r}")
    d = synth.make_random(b, m, n, r, seed=b * 7 + r)
    check_full(d, run_gpu(d))


def _random_shapes(count, seed=2026, max_macs=6e8):
    """Seeded shapes across the launch rules: b in each token range of the few-token
    tilings and beyond, m and n anywhere on their grids, r any multiple of 16 up to 128."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        lo, hi = [(1, 17), (17, 33), (33, 65), (65, 300)][int(rng.integers(0, 4))]
        b, m = int(rng.integers(lo, hi)), 128 * int(rng.integers(1, 40))
        n, r = 16 * int(rng.integers(1, 1600)), 16 * int(rng.integers(0, 9))
        if b * m * n <= max_macs:
            out.append((b, m, n, r))
    return out


@pytest.mark.parametrize("b,m,n,r", _random_shapes(12))
def test_seeded_random_shapes(b, m, n, r):
    _say(f"random shape b={b} m={m} n={n} r={r}")
    d = synth.make_random(b, m, n, r, seed=b + m + n + r)
    check_full(d, run_gpu(d))


def test_zero_rows_and_zero_residual():
    """An all-zero token row (s_X = 0) and W_res = 0 (pure low-rank, s_W = 0)."""
    d = synth.make_random(24, 512, 96, 32, seed=11)
    d["x"][3] = 0
    d["x"][17] = 0
    check_full(d, run_gpu(d))
    d["w_res"][:] = 0
    g = run_gpu(d)
    assert (_np(g["sw"]) == 0).all() and (_np(g["qw"]) == 0).all()
    check_full(d, g)


def test_rank_zero_plain_w4a4():
    d = synth.make_random(40, 768, 112, 0, seed=12)
    g = run_gpu(d)
    check_full(d, g)


def test_largest_m():
    """m = 131072, the largest K the int32 accumulator is allowed."""
    d = synth.make_random(3, 131072, 16, 16, seed=13)
    check_full(d, run_gpu(d))


def test_repeat_runs_bitwise_equal():
    d = synth.make_layer("o_proj_decode")
    a = run_gpu(d, debug_acc=False)
    b = run_gpu(d, debug_acc=False)
    for k in ("qx", "sx", "t", "y"):
        assert torch.equal(a[k], b[k]), k


def test_workspace_shared_across_shapes():
    """Calls of different shapes share one workspace: many-token calls with K slices
    (partial sums in the workspace) interleaved with few-token calls."""
    for b, m, n, r in [(129, 1152, 208, 64), (3, 8192, 16, 16), (300, 2048, 64, 32), (17, 4096, 64, 48)]:
        _say(f"shape b={b} m={m} n={n} r={r}")
        d = synth.make_random(b, m, n, r, seed=b + m)
        check_full(d, run_gpu(d))


def test_workspace_too_small_is_rejected():
    """The many-token quantizers keep T's K-slice partial sums in the workspace."""
    dev = _dev()
    L = twq.lib()
    b, m, r = 2048, 4096, 32
    x = torch.zeros(b, m, dtype=torch.float16, device=dev)
    l1t = torch.zeros(r, m, dtype=torch.float16, device=dev)
    qx = torch.empty(b, m, dtype=torch.uint8, device=dev)
    sx = torch.empty(b, dtype=torch.float32, device=dev)
    t = torch.empty(b, r, dtype=torch.float32, device=dev)
    need = L.twq_quantize_act_workspace_bytes(b, m, r)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    import ctypes
    p = lambda z: ctypes.c_void_p(z.data_ptr())
    assert L.twq_quantize_act_a8(p(x), b, m, p(qx), p(sx), p(l1t), r, p(t), p(ws), need - 16, None) == 6
    assert L.twq_quantize_act(p(x), b, m, p(qx), p(sx), p(l1t), r, p(t), p(ws), need - 16, None) == 6


# ------------------------------------------------------------------ full-size configurations, sampled

BIG = ["gate_up_prefill", "down_prefill", "70b_gate_up_decode", "70b_gate_up_prefill"]


@pytest.mark.parametrize("name", BIG)
def test_config_full_size_sampled(name):
    """Full-size shapes in the launch configuration the benchmark uses: every code and
    scale compared whole, the accumulator and Y at 384 sampled positions."""
    _say(f"config {name}: generating inputs")
    d = layers.layer(name)
    b, m = d["x"].shape
    n = d["w_res"].shape[0]
    _say(f"config {name}: GPU b={b} m={m} n={n} r={d['l1t'].shape[0]}")
    g = run_gpu(d, debug_acc=False)
    qx_ref, qxp_ref, sx_ref = oracle.quantize_act(d["x"])
    assert np.array_equal(_np(g["qx"]), qxp_ref) and np.array_equal(_np(g["sx"]), sx_ref)
    _, qwp_ref, sw_ref = oracle.quantize_weight(d["w_res"])
    assert np.array_equal(_np(g["qw"]), to_panels(qwp_ref)) and np.array_equal(_np(g["sw"]), sw_ref)
    rng = synth.rng_for(100 + b)
    rows = rng.integers(0, b, 384)
    cols = rng.integers(0, n, 384)
    # corners, and the position of the largest |Y| on the GPU so the samples see the scale
    top = int(torch.argmax(g["y"].abs().float()).item())
    rows[:5] = [0, 0, b - 1, b - 1, top // n]
    cols[:5] = [0, n - 1, 0, n - 1, top % n]
    acc_ref, y_ref = oracle.dual_linear_sampled(d["x"], d["w_res"], d["l1t"], d["l2t"], rows, cols)
    acc = twq.debug_residual_acc(g["qx"], g["qw"])
    ri = torch.from_numpy(rows).to(acc.device)
    ci = torch.from_numpy(cols).to(acc.device)
    assert np.array_equal(acc[ri, ci].cpu().numpy().astype(np.int64), acc_ref)
    y = g["y"][ri, ci].cpu().numpy().astype(np.float64)
    # max|Y_or| over the samples is at most the true one, so this bound is the stricter
    scale = np.abs(y_ref).max()
    err = np.abs(y - y_ref).max()
    assert err <= Y_TOL * scale, (err, scale)
    _say(f"  sampled max|Y-Y_or| = {err:.3g}, max|Y_or| over samples = {scale:.3g}")
