"""twq_linear_noalloc (the one-call layer on the library's own scratch array) against
twq_linear (a caller workspace) and the oracle.

Two calls in a row on one GPU, the second smaller than the first: the second reads a
scratch array the first has filled with other values, and must not depend on them.
Y must equal twq_linear's bit for bit (the same kernels on the same values) and lie
within 2e-3 * max|Y_oracle| of the oracle.
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


def _layer(d, dev):
    x = torch.from_numpy(d["x"]).to(dev)
    qw, sw = twq.pack_weight(torch.from_numpy(d["w_res"]).to(dev))
    r = d["l1t"].shape[0]
    l1t = torch.from_numpy(d["l1t"]).to(dev) if r else None
    l2t = torch.from_numpy(d["l2t"]).to(dev) if r else None
    return x, qw, sw, l1t, l2t


# (b, m, n, r): a many-token call first (the largest scratch), then few-token calls
# (T's partial sums added in the fused epilogue; r = 0) that read what it left
SEQUENCE = [(300, 2048, 1024, 64), (16, 4096, 4096, 32), (5, 1024, 528, 16), (16, 512, 256, 0)]


def test_noalloc_matches_linear_on_calls_in_a_row():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    dev = torch.device("cuda:0")
    for k, (b, m, n, r) in enumerate(SEQUENCE):
        _say(f"twq_linear_noalloc call {k}: b={b} m={m} n={n} r={r}")
        d = synth.make_random(b, m, n, r, seed=500 + k)
        x, qw, sw, l1t, l2t = _layer(d, dev)
        y_out = torch.empty((b, n), dtype=torch.float16, device=dev)
        y0 = twq.linear_noalloc(x, qw, sw, l1t, l2t, out=y_out)
        y1 = twq.linear(x, qw, sw, l1t, l2t)
        torch.cuda.synchronize()
        assert y0.data_ptr() == y_out.data_ptr()
        a0, a1 = y0.cpu().numpy(), y1.cpu().numpy()
        assert np.array_equal(a0, a1), f"call {k}: twq_linear_noalloc differs from twq_linear"
        ref = oracle.dual_linear(d["x"], d["w_res"], d["l1t"], d["l2t"])["y"]
        err = np.abs(a0.astype(np.float64) - ref).max()
        assert err <= Y_TOL * np.abs(ref).max(), (k, err, np.abs(ref).max())


def test_noalloc_repeat_bitwise_and_oversize_refused():
    dev = torch.device("cuda:0")
    d = synth.make_random(16, 4096, 1024, 32, seed=77)
    x, qw, sw, l1t, l2t = _layer(d, dev)
    _say("twq_linear_noalloc repeat b=16 m=4096 n=1024 r=32")
    ys = [twq.linear_noalloc(x, qw, sw, l1t, l2t).cpu() for _ in range(3)]
    assert all(torch.equal(ys[0], y) for y in ys[1:])
    # a shape whose scratch exceeds the array is refused before any launch
    L = twq.lib()
    b, m, n, r = 65536, 8192, 28672, 128
    assert L.twq_linear_workspace_bytes(b, m, n, r) > L.twq_linear_noalloc_max_bytes()
    p = x.data_ptr()
    st = L.twq_linear_noalloc(p, qw.data_ptr(), sw.data_ptr(), l1t.data_ptr(), l2t.data_ptr(), r, p, b, m, n,
                              None)
    assert st == 6  # TWQ_ERR_WORKSPACE
