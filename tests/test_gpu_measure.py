"""The measurement exports against the one-call layers they time.

bench.py prices the fused launch of a one-call layer (twq_linear and its group-wise,
W4A8 and int4-low-rank forms) by timing twq_debug_linear_main (and its _grouped_main,
_a8_main, _lr4_main forms) alone, on the workspace an earlier call of the same shape
filled. That is a measurement of the right kernel only if the export runs that very
launch: here its Y must equal the one-call layer's bit for bit, over a Y buffer that
was overwritten in between, at decode shapes (T whole, or T's K-slice sums added in the
epilogue) and prefill shapes.
"""
import sys

import pytest
import torch

import w4a4_rank_gemm_amd as twq

pytestmark = pytest.mark.gpu

# (b, m, n, r): o_proj-like decode (T's slices in the epilogue), a decode shape whose
# CTAs read T whole, a 70B-width decode shape, and two prefill shapes (ragged tokens)
SHAPES = [(16, 4096, 4096, 32), (32, 8192, 2048, 128), (32, 8192, 28672, 128), (300, 1024, 2064, 32),
          (1000, 2048, 4096, 64)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(b, m, n, r, seed):
    # no oracle here: seeded normal operands drawn on the GPU (the 70B-width weight is
    # 0.9 GB in fp32), scaled as the synthetic layers are
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn((b, m), generator=g, device=dev).half()
    w = torch.randn((n, m), generator=g, device=dev) * 0.02
    l1t = (torch.randn((r, m), generator=g, device=dev) * (1.0 / m ** 0.5)).half()
    l2t = (torch.randn((n, r), generator=g, device=dev) * 0.05).half()
    return dev, x, w, l1t, l2t


def _both(one_call, main, y_shape, dev, ws_bytes):
    """Y of the one-call layer, then Y of its export on the same workspace (Y poisoned in between)."""
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    y = torch.empty(y_shape, dtype=torch.float16, device=dev)
    one_call(y, ws)
    torch.cuda.synchronize()
    y1 = y.clone()
    y.fill_(float("nan"))
    main(y, ws)
    torch.cuda.synchronize()
    return y1, y


@pytest.mark.parametrize("b,m,n,r", SHAPES)
@pytest.mark.parametrize("variant", ["per_token", "grouped", "a8"])
def test_linear_main_export(b, m, n, r, variant):
    _say(f"measurement export {variant} b={b} m={m} n={n} r={r}")
    dev, x, w, l1t, l2t = _inputs(b, m, n, r, seed=b + m + r)
    L, P, S = twq.lib(), twq._ptr, twq._stream(dev)
    if variant == "grouped":
        qw, sw = twq.pack_weight_grouped(w)
        g = twq.GROUP
        wsb = L.twq_linear_grouped_workspace_bytes(b, m, n, r, g)

        def one(y, ws):
            twq._check(L.twq_linear_grouped(P(x), P(qw), P(sw), P(l1t), P(l2t), r, P(y), b, m, n, g, P(ws), wsb, S),
                       "twq_linear_grouped")

        def main(y, ws):
            twq._check(L.twq_debug_linear_grouped_main(P(x), P(qw), P(sw), P(l1t), P(l2t), r, P(y), b, m, n, g, P(ws),
                                                       wsb, S), "twq_debug_linear_grouped_main")
    else:
        qw, sw = twq.pack_weight(w)
        a8 = variant == "a8"
        wsb = (L.twq_linear_a8_workspace_bytes if a8 else L.twq_linear_workspace_bytes)(b, m, n, r)
        lin = L.twq_linear_a8 if a8 else L.twq_linear
        dbg = L.twq_debug_linear_a8_main if a8 else L.twq_debug_linear_main

        def one(y, ws):
            twq._check(lin(P(x), P(qw), P(sw), P(l1t), P(l2t), r, P(y), b, m, n, P(ws), wsb, S), "one-call layer")

        def main(y, ws):
            twq._check(dbg(P(x), P(qw), P(sw), P(l1t), P(l2t), r, P(y), b, m, n, P(ws), wsb, S), "export")
    y1, y2 = _both(one, main, (b, n), dev, wsb)
    assert torch.equal(y1, y2), "the export's Y differs from the one-call layer's"


@pytest.mark.parametrize("b,m,n,r", SHAPES)
def test_linear_lr4_main_export(b, m, n, r):
    _say(f"measurement export lr4 b={b} m={m} n={n} r={r}")
    dev, x, w, l1t, l2t = _inputs(b, m, n, r, seed=3 * b + r)
    L, P, S = twq.lib(), twq._ptr, twq._stream(dev)
    qw, sw = twq.pack_weight(w)
    lp = twq.pack_lowrank_int4(l1t, l2t)
    wsb = L.twq_linear_lr4_workspace_bytes(b, m, n, r)

    def one(y, ws):
        twq._check(L.twq_linear_lr4(P(x), P(qw), P(sw), P(lp["ql1"]), P(lp["c"]), P(lp["ql2"]), r, P(y), b, m, n,
                                    P(ws), wsb, S), "twq_linear_lr4")

    def main(y, ws):
        twq._check(L.twq_debug_linear_lr4_main(P(x), P(qw), P(sw), P(lp["ql1"]), P(lp["c"]), P(lp["ql2"]), r, P(y),
                                               b, m, n, P(ws), wsb, S), "twq_debug_linear_lr4_main")
    y1, y2 = _both(one, main, (b, n), dev, wsb)
    assert torch.equal(y1, y2), "the export's Y differs from twq_linear_lr4's"
