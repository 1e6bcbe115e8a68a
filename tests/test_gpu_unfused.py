"""The unfused comparator of bench.py --compare (residual result through HBM, then T L2
and the add as separate platform launches) against the oracle: the kernel-fusion gain
it measures is only meaningful if both sides compute the same layer."""
import sys

import numpy as np
import pytest
import torch

import bench
import oracle
import synth
import w4a4_rank_gemm_amd as twq

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3


@pytest.mark.parametrize("b,m,n,r", [(16, 4096, 4096, 32), (200, 1024, 528, 48), (32, 2048, 1024, 128)])
def test_unfused_comparator_matches_oracle(b, m, n, r):
    print(f"unfused b={b} m={m} n={n} r={r}", flush=True)
    sys.stdout.flush()
    d = synth.make_random(b, m, n, r, seed=70 + b)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(d["x"]).to(dev)
    qw, sw = twq.pack_weight(torch.from_numpy(d["w_res"]).to(dev))
    l1t = torch.from_numpy(d["l1t"]).to(dev)
    l2t = torch.from_numpy(d["l2t"]).to(dev)
    qx = torch.empty((b, m // 2), dtype=torch.uint8, device=dev)
    sx = torch.empty((b,), dtype=torch.float32, device=dev)
    t = torch.empty((b, r), dtype=torch.float32, device=dev)
    y = torch.empty((b, n), dtype=torch.float16, device=dev)
    L = twq.lib()
    ws, wsb = twq._workspace(dev, L.twq_quantize_act_workspace_bytes(b, m, r))
    bench.unfused_layer(twq, x, qx, sx, t, qw, sw, l1t, l2t, y, ws, wsb,
                        twq.ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    y_fused = twq.linear(x, qw, sw, l1t, l2t)
    torch.cuda.synchronize()
    ref = oracle.dual_linear(d["x"], d["w_res"], d["l1t"], d["l2t"])
    assert np.array_equal(qx.cpu().numpy(), ref["qx_packed"]) and np.array_equal(sx.cpu().numpy(), ref["sx"])
    yo = ref["y"]
    for name, yy in (("unfused", y), ("fused", y_fused)):
        err = np.abs(yy.cpu().numpy().astype(np.float64) - yo).max()
        assert err <= Y_TOL * np.abs(yo).max(), (name, err, np.abs(yo).max())
