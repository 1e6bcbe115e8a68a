"""The one-call layers captured into a HIP graph (as bench.py times them) and replayed.

torch's graph capture records the C-ABI launches made on its capture stream. Each
replay must give the eager result bit for bit: the outputs are poisoned with NaN and
unrelated eager work runs between replays, and every replay is checked. Nothing in
libtwq records a memset, so this also guards against one slipping in.
"""
import sys

import pytest
import torch

import w4a4_rank_gemm_amd as twq

pytestmark = pytest.mark.gpu

# decode with T's slice sums in the epilogue, decode with T reduced first, prefill
SHAPES = [(16, 4096, 4096, 32), (32, 8192, 2048, 128), (300, 1024, 2064, 32)]
CALLS = 3  # calls per graph, each on its own input


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _layer(b, m, n, r, seed):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed)
    xs = [torch.randn((b, m), generator=g, device=dev).half() for _ in range(CALLS)]
    w = torch.randn((n, m), generator=g, device=dev) * 0.02
    l1t = (torch.randn((r, m), generator=g, device=dev) * (1.0 / m ** 0.5)).half()
    l2t = (torch.randn((n, r), generator=g, device=dev) * 0.05).half()
    return dev, xs, w, l1t, l2t


def _check_replays(fn, outs, dev):
    """fn() issues CALLS layer calls writing outs; eager once, then captured and replayed."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream(dev)  # default priority
    side.wait_stream(torch.cuda.current_stream(dev))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        fn()
    torch.cuda.synchronize()
    junk = torch.randn((512, 512), device=dev)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.tanh(junk @ junk.T) + 0.5  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"replay {rep}, call {i}: differs from the eager result"


@pytest.mark.parametrize("b,m,n,r", SHAPES)
@pytest.mark.parametrize("variant", ["per_token", "grouped", "a8", "lr4", "noalloc"])
def test_graph_replay(b, m, n, r, variant):
    _say(f"graph replay {variant} b={b} m={m} n={n} r={r}")
    dev, xs, w, l1t, l2t = _layer(b, m, n, r, seed=7 * b + r)
    ys = [torch.empty((b, n), dtype=torch.float16, device=dev) for _ in range(CALLS)]
    if variant == "grouped":
        qw, sw = twq.pack_weight_grouped(w)

        def fn():
            for x, y in zip(xs, ys):
                twq.linear_grouped(x, qw, sw, l1t, l2t, out=y)
    elif variant == "a8":
        qw, sw = twq.pack_weight(w)

        def fn():
            for x, y in zip(xs, ys):
                twq.linear_a8(x, qw, sw, l1t, l2t, out=y)
    elif variant == "lr4":
        qw, sw = twq.pack_weight(w)
        lp = twq.pack_lowrank_int4(l1t, l2t)

        def fn():
            for x, y in zip(xs, ys):
                twq.linear_lr4(x, qw, sw, lp, out=y)
    elif variant == "noalloc":
        qw, sw = twq.pack_weight(w)

        def fn():
            for x, y in zip(xs, ys):
                twq.linear_noalloc(x, qw, sw, l1t, l2t, out=y)
    else:
        qw, sw = twq.pack_weight(w)

        def fn():
            for x, y in zip(xs, ys):
                twq.linear(x, qw, sw, l1t, l2t, out=y)
    _check_replays(fn, ys, dev)
