#!/usr/bin/env python3
"""Benchmark of the fused W4A4 + low-rank linear on one MI355X.

One step = one call of the layer on one batch: twq_linear (per-token quantization
+ T = X L1, then the residual int4 GEMM with the low-rank epilogue), weights
pre-packed and resident in HBM. The default workload is the largest layer that
fits one GPU, the 70B-size MLP gate/up layer at prefill (b=8192, m=8192,
n=28672, r=128). Inputs are synthetic (seeded,
with the shapes and value distributions of the layer configurations), and the
steps rotate over enough copies of the weights that the caches (4 MB L2 per
XCD, 256 MB Infinity Cache) cannot hold the working set.

Prints one JSON line. `value` is effective TOPS = (2bmn + 2br(m+n)) / time per
step. The `roofline` object prices the dominant kernel -- the fused main-loop
launch exactly as the timed call runs it, timed alone through the measurement
export twq_debug_linear_main -- against HBM bandwidth (few tokens) or the int8
matrix-core peak (many tokens).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 matrix cores, TOP/s
ROTATE_BYTES = 512 << 20     # working set that defeats L2 + Infinity Cache reuse
METRIC_NAME = "fused W4A4+low-rank linear: \u00b5s/call, effective TOPS, % int8-MFMA/HBM roofline"


def layer_ops(b, m, n, r):
    """Useful operations of one layer call: the int8 GEMM plus the two low-rank products."""
    return 2 * b * m * n + 2 * b * r * (m + n)


def call_bytes(b, m, n, r):
    """Compulsory HBM bytes of one whole call: X fp16, Q_W, s_W, L1 and L2 fp16, Y fp16."""
    return 2 * b * m + m * n // 2 + 4 * n + 2 * r * (m + n) + 2 * b * n


def dual_linear_bytes(b, m, n, r):
    """Algorithmic bytes of one twq_dual_linear launch: it reads Q_X, s_X, Q_W, s_W, T and
    L2, and writes Y, each once."""
    return b * m // 2 + 4 * b + m * n // 2 + 4 * n + 4 * b * r + 2 * n * r + 2 * b * n


def call_bytes_grouped(b, m, n, r, g):
    """Compulsory HBM bytes of one group-wise call: as call_bytes, with one s_W per group."""
    return 2 * b * m + m * n // 2 + 4 * n * (m // g) + 2 * r * (m + n) + 2 * b * n


def dual_linear_grouped_bytes(b, m, n, r, g):
    """Algorithmic bytes of one twq_dual_linear_grouped launch: Q_X, the m/g scales per
    token and per channel, Q_W, T and L2 read once, Y written once."""
    return b * m // 2 + 4 * b * (m // g) + m * n // 2 + 4 * n * (m // g) + 4 * b * r + 2 * n * r + 2 * b * n


def dual_linear_a8_bytes(b, m, n, r):
    """Algorithmic bytes of one twq_dual_linear_a8 launch: as dual_linear_bytes with one
    byte per activation code."""
    return b * m + 4 * b + m * n // 2 + 4 * n + 4 * b * r + 2 * n * r + 2 * b * n


def call_bytes_lr4(b, m, n, r):
    """Compulsory HBM bytes of one call with the int4 low-rank branch: X fp16, Q_W, s_W,
    Q_L1 and Q_L2 (4-bit), c, Y fp16."""
    return 2 * b * m + m * n // 2 + 4 * n + r * (m + n) // 2 + 4 * r + 2 * b * n


def dual_linear_lr4_bytes(b, m, n, r):
    """Algorithmic bytes of one twq_dual_linear_lr4 launch: Q_X, s_X, Q_W, s_W, Q_H, s_H and
    Q_L2 read once, Y written once."""
    return b * m // 2 + 4 * b + m * n // 2 + 4 * n + b * r // 2 + 4 * b + n * r // 2 + 2 * b * n


KERNEL_SOURCES = ("w4a4_rank_gemm_amd/csrc/dual_linear.hip", "w4a4_rank_gemm_amd/csrc/twq_device.h",
                  "w4a4_rank_gemm_amd/csrc/twq_kernels.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dual_linear_traffic.json")


def kernel_source_hash():
    """sha256 over the sources of the fused kernel: the HBM traffic measured with
    rocprofv3 counters is reported only while the kernel is the one that was measured."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per twq_dual_linear launch from the committed counter summary, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    entry = rec.get("workloads", {}).get(workload)
    return None if entry is None else entry.get("traffic_bytes")


def cpu_model():
    """The host CPU's model name (the first "model name" of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def rocm_version():
    """The ROCm release of the image (/opt/rocm/.info/version), or None."""
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                return f.read().strip()
        except OSError:
            continue
    return None


def host_env(torch):
    """Where the numbers were taken: GPU name, ROCm and HIP versions, torch, host CPU."""
    try:
        gpu = torch.cuda.get_device_name(0)
        props = torch.cuda.get_device_properties(0)
        arch = getattr(props, "gcnArchName", None)
        units = props.multi_processor_count
    except Exception:  # noqa: BLE001 - informative only
        gpu, arch, units = None, None, None
    return {"gpu": gpu, "gpu_arch": arch, "compute_units": units, "rocm": rocm_version(),
            "hip": getattr(torch.version, "hip", None),
            "torch": torch.__version__, "host_cpu": cpu_model(), "host_threads": os.cpu_count()}


def lowrank_storage_ratio(m, n, r):
    """fp16 low-rank storage r(m+n) * 2 bytes over the 4-bit residual m n / 2 bytes."""
    return 2 * r * (m + n) / (m * n / 2)


# The oracle's work per call is linear in the tokens (rows are independent), so shapes
# whose whole call would take the host much longer than the budget are timed on their
# first rows and scaled to the batch: at most this many multiply-adds of the residual
# product per timed call (about 7 s on 16 host threads).
CPU_MACS_PER_CALL = 3e11


def _cpu_rows(b, m, n):
    return int(min(b, max(16, CPU_MACS_PER_CALL // (m * n))))


def _cpu_sample(calls, rows, b, m, n, r, el, what):
    part = "whole calls" if rows == b else f"calls on the first {rows} of {b} tokens, scaled to the whole batch,"
    return (f"{calls} {what}{part} of the same workload (b={b}, m={m}, n={n}, r={r}) in {el:.1f} s; "
            "weights quantized once outside the timing")


def _cpu_baseline_grouped(d, g, budget_s=12.0):
    """The group-wise oracle on the host, weights pre-quantized, on the first rows of the
    batch (the per-group integer sums of every row would not fit in memory at full size);
    the rate scales with the rows it covered."""
    import numpy as np

    import oracle
    x, w, l1t, l2t = d["x"], d["w_res"], d["l1t"], d["l2t"]
    b, m = x.shape
    n, r = w.shape[0], l1t.shape[0]
    rows = int(min(b, max(1, (256 << 20) // (n * (m // g) * 8))))
    xs = np.ascontiguousarray(x[:rows])
    qw, _, sw = oracle.quantize_weight_grouped(w, g)  # offline packing, not timed
    calls = 0
    t0 = time.perf_counter()
    while True:
        qx, _, sx = oracle.quantize_act_grouped(xs, g)
        accg = oracle.residual_acc_grouped(qx, qw, g)
        y = np.einsum("ig,jg,ijg->ij", sx.astype(np.float64), sw.astype(np.float64), accg)
        if r:
            y += oracle.lowrank_out(oracle.lowrank_t(xs, l1t), l2t)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 1000:
            break
    sec = el / calls * b / rows
    return {"value": layer_ops(b, m, n, r) / sec / 1e12, "unit": "TOPS", "cores": oracle.max_threads(),
            "kind": "oracle", "ms_per_call": sec * 1e3,
            "sample": f"{calls} calls on the first {rows} of {b} tokens (b={b}, m={m}, n={n}, r={r}, "
                      f"groups of {g}) in {el:.1f} s, scaled to the whole batch; weights quantized once "
                      "outside the timing"}


def _cpu_baseline_a8(d, budget_s=12.0):
    """The W4A8 oracle on the host: per-call work with weights pre-quantized."""
    import numpy as np

    import oracle
    x, w, l1t, l2t = d["x"], d["w_res"], d["l1t"], d["l2t"]
    b, m = x.shape
    n, r = w.shape[0], l1t.shape[0]
    qw, _, sw = oracle.quantize_weight(w)  # offline packing, not timed
    rows = _cpu_rows(b, m, n)
    xs = np.ascontiguousarray(x[:rows])
    calls = 0
    t0 = time.perf_counter()
    while True:
        qx, sx = oracle.quantize_act_a8(xs)
        acc = oracle.residual_acc(qx, qw)
        y = sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] * acc
        if r:
            y += oracle.lowrank_out(oracle.lowrank_t(xs, l1t), l2t)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 1000:
            break
    sec = el / calls * b / rows
    return {"value": layer_ops(b, m, n, r) / sec / 1e12, "unit": "TOPS", "cores": oracle.max_threads(),
            "kind": "oracle", "ms_per_call": sec * 1e3,
            "sample": _cpu_sample(calls, rows, b, m, n, r, el, "W4A8 ")}


def _cpu_baseline(d, budget_s=12.0, lr4=False):
    """The oracle (plain C, OpenMP) on the host: per-call work with weights pre-quantized."""
    import numpy as np

    import oracle
    x, w, l1t, l2t = d["x"], d["w_res"], d["l1t"], d["l2t"]
    b, m = x.shape
    n, r = w.shape[0], l1t.shape[0]
    qw, _, sw = oracle.quantize_weight(w)  # offline packing, not timed
    lq = oracle.quantize_lowrank(l1t, l2t) if (lr4 and r) else None
    rows = _cpu_rows(b, m, n)
    x = np.ascontiguousarray(x[:rows])
    calls = 0
    t0 = time.perf_counter()
    while True:
        qx, _, sx = oracle.quantize_act(x)
        acc = oracle.residual_acc(qx, qw)
        y = sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] * acc
        if r and lr4:
            rq = oracle.lowrank_requant(qx, sx, lq["ql1"], lq["c"])
            y += rq["sh"].astype(np.float64)[:, None] * oracle.residual_acc(rq["qh"], lq["ql2"])
        elif r:
            y += oracle.lowrank_out(oracle.lowrank_t(x, l1t), l2t)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 1000:
            break
    sec = el / calls * b / rows
    return {"value": layer_ops(b, m, n, r) / sec / 1e12, "unit": "TOPS", "cores": oracle.max_threads(),
            "kind": "oracle", "ms_per_call": sec * 1e3,
            "sample": _cpu_sample(calls, rows, b, m, n, r, el, "")}


def _graph_time(fn, steps, warmup, stream):
    """GPU time per step (us) of `fn(i)` for i in range(steps), captured into a HIP graph on
    `stream` and replayed once after an untimed replay of `warmup` steps."""
    import torch
    gw, g = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn(0)  # lazy initialisation outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(gw, stream=stream):
            for i in range(warmup):
                fn(i)
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                fn(i)
        gw.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
    return e0.elapsed_time(e1) / steps * 1e3


def unfused_layer(twq, x, qx, sx, t, qw, sw, l1t, l2t, y, ws, wsb, stream):
    """The unfused comparator of the fused layer (the pages' kernel-fusion baseline, page 2
    section A.4): the same quantizer and residual kernel, but the residual result is
    written to HBM as Y_res (twq_dual_linear with r = 0), then T L2 is a separate fp16
    GEMM and Y_res + T L2 a separate add (platform library launches). Writes y in place.
    All tensors on one GPU; qx, sx, t are scratch of the quantizer's output shapes."""
    import torch
    L = twq.lib()
    P = lambda z: None if z is None else twq.ctypes.c_void_p(z.data_ptr())
    b, m = x.shape
    n = qw.shape[0]
    r = 0 if l1t is None else l1t.shape[0]
    twq._check(L.twq_quantize_act(P(x), b, m, P(qx), P(sx), P(l1t), r, P(t), P(ws), wsb, stream), "twq_quantize_act")
    twq._check(L.twq_dual_linear(P(qx), P(sx), P(qw), P(sw), None, None, 0, P(y), b, m, n, stream), "twq_dual_linear")
    if r:
        y.add_(torch.nn.functional.linear(t.half(), l2t))


COMPARE_CONFIGS = ("o_proj_decode", "70b_gate_up_decode", "gate_up_prefill", "70b_gate_up_prefill")
SWEEP_RANKS = (0, 32, 64, 128, 256)


def compare(args):
    """Context for the fused layer, one JSON line per measurement (weights rotated as in
    the main benchmark, HIP graphs):
      fused      twq_linear (quantize + T, then the fused main loop and epilogue);
      unfused    the same pieces with the partial result spilled: twq_quantize_act (Q_X,
                 s_X, T), the residual-only fused kernel writing Y_res to HBM, then T L2
                 and Y_res + T L2 as two more launches (fp16 GEMM and add from the
                 platform library);
      residual   twq_linear with r = 0 (plain W4A4);
      fp16       the dense fp16 layer Y = X W^T on the platform GEMM (hipBLASLt);
    and a sweep of the rank r over SWEEP_RANKS on each shape (fused layer only; random
    factors, which do not change the time)."""
    import torch

    import synth
    import w4a4_rank_gemm_amd as twq
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)  # default priority
    L = twq.lib()
    P = lambda t: None if t is None else twq.ctypes.c_void_p(t.data_ptr())
    hs = lambda: twq.ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    names = args.compare_configs.split(",") if args.compare_configs else COMPARE_CONFIGS
    for name in names:
        cfg = synth.CONFIGS[name]
        b, m, n, r = cfg.b, cfg.m, cfg.n, cfg.r
        gen = torch.Generator(device=dev).manual_seed(cfg.index)
        x0 = (torch.randn((b, m), generator=gen, device=dev) * 2).half()
        w0 = torch.randn((n, m), generator=gen, device=dev) * 0.02
        qw0, sw0 = twq.pack_weight(w0)
        w16_0 = w0.half()
        del w0
        copies = max(1, math.ceil(ROTATE_BYTES / call_bytes(b, m, n, max(SWEEP_RANKS))))
        copies16 = max(1, math.ceil(ROTATE_BYTES / (2 * m * n)))
        sets = [{"x": x0.clone(), "qw": qw0.clone(), "sw": sw0.clone(),
                 "qx": torch.empty((b, m // 2), dtype=torch.uint8, device=dev),
                 "sx": torch.empty((b,), dtype=torch.float32, device=dev),
                 "y": torch.empty((b, n), dtype=torch.float16, device=dev)} for _ in range(copies)]
        w16 = [w16_0.clone() for _ in range(copies16)]
        del w16_0

        def lowrank(rk):
            for s_ in sets:
                s_["l1t"] = (torch.randn((rk, m), generator=gen, device=dev) * 0.02).half() if rk else None
                s_["l2t"] = (torch.randn((n, rk), generator=gen, device=dev) * 0.02).half() if rk else None
                s_["t"] = torch.empty((b, rk), dtype=torch.float32, device=dev) if rk else None

        ws, wsb = twq._workspace(dev, max(L.twq_linear_workspace_bytes(b, m, n, max(SWEEP_RANKS)),
                                          L.twq_quantize_act_workspace_bytes(b, m, max(SWEEP_RANKS))))

        def fused(rk):
            def f(i):
                s_ = sets[i % copies]
                twq._check(L.twq_linear(P(s_["x"]), P(s_["qw"]), P(s_["sw"]), P(s_["l1t"]), P(s_["l2t"]), rk,
                                        P(s_["y"]), b, m, n, P(ws), wsb, hs()), "twq_linear")
            return f

        def unfused(i):
            s_ = sets[i % copies]
            unfused_layer(twq, s_["x"], s_["qx"], s_["sx"], s_["t"], s_["qw"], s_["sw"], s_["l1t"], s_["l2t"], s_["y"],
                          ws, wsb, hs())

        def fp16(i):
            sets[i % copies]["y"].copy_(torch.nn.functional.linear(sets[i % copies]["x"], w16[i % copies16]))

        def emit(variant, us, rk=r):
            print(json.dumps({"compare": name, "variant": variant, "b": b, "m": m, "n": n, "r": rk,
                              "us_per_call": round(us, 3), "effective_tops": round(layer_ops(b, m, n, rk) / us / 1e6, 2)}),
                  flush=True)

        lowrank(r)
        emit("fused", _graph_time(fused(r), args.steps, args.warmup, stream))
        emit("unfused", _graph_time(unfused, args.steps, args.warmup, stream))
        emit("residual", _graph_time(fused(0), args.steps, args.warmup, stream), 0)
        emit("fp16", _graph_time(fp16, args.steps, args.warmup, stream), 0)
        for rk in SWEEP_RANKS:
            lowrank(rk)
            emit("fused_rank_sweep", _graph_time(fused(rk), args.steps, args.warmup, stream), rk)
        del sets, w16
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="70b_gate_up_prefill")
    ap.add_argument("--path", choices=("linear", "split"), default="linear",
                    help="linear: one twq_linear call per step; split: twq_quantize_act + twq_dual_linear")
    ap.add_argument("--lowrank", choices=("fp16", "int4"), default="fp16",
                    help="fp16: the fp16 low-rank branch; int4: 4-bit L1, L2 and H (twq_linear_lr4, or "
                         "twq_quantize_act_lr4 + twq_dual_linear_lr4 with --path split)")
    ap.add_argument("--group", type=int, choices=(0, 128), default=0,
                    help="128: group-wise scales (twq_*_grouped entry points, groups of 128 along K)")
    ap.add_argument("--act-bits", type=int, choices=(4, 8), default=4,
                    help="8: W4A8 (twq_*_a8 entry points, 8-bit per-token activation codes)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate over (0: auto)")
    ap.add_argument("--eager", action="store_true", help="launch from Python instead of a HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before timing, copy 256 MiB device-to-device 4 times (a kernel of known "
                         "traffic for scaling hardware counters)")
    ap.add_argument("--compare", action="store_true",
                    help="instead of the benchmark line: fused vs unfused vs residual-only vs dense fp16, "
                         "and a rank sweep, one JSON line each")
    ap.add_argument("--compare-configs", default="", help="comma-separated workloads for --compare")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the layer is benchmarked on one "
                                   "MI355X; run with --gpus 1"}))
        sys.exit(2)
    if args.compare:
        return compare(args)

    import numpy as np
    import torch

    import synth
    import w4a4_rank_gemm_amd as twq

    cfg = synth.CONFIGS[args.config]
    b, m, n, r = cfg.b, cfg.m, cfg.n, cfg.r
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# generating {args.config}: b={b} m={m} n={n} r={r}", file=sys.stderr, flush=True)
    d = synth.make_layer(cfg)

    lr4 = args.lowrank == "int4"
    grp = args.group
    a8 = args.act_bits == 8
    if lr4 and grp:
        ap.error("--group applies to the fp16 low-rank branch only")
    if a8 and (lr4 or grp):
        ap.error("--act-bits 8 takes per-token scales and the fp16 low-rank branch")
    per_copy = (call_bytes_lr4(b, m, n, r) if lr4 else call_bytes_grouped(b, m, n, r, grp) if grp
                else call_bytes(b, m, n, r))
    copies = args.copies or max(1, math.ceil(ROTATE_BYTES / per_copy))
    x0 = torch.from_numpy(d["x"]).to(dev)
    w0 = torch.from_numpy(d["w_res"]).to(dev)
    l10 = torch.from_numpy(d["l1t"]).to(dev) if r else None
    l20 = torch.from_numpy(d["l2t"]).to(dev) if r else None
    qw0, sw0 = twq.pack_weight_grouped(w0, grp) if grp else twq.pack_weight(w0)
    del w0
    lp0 = twq.pack_lowrank_int4(l10, l20) if (lr4 and r) else None
    sets = []
    for c in range(copies):
        s_ = {
            "x": x0.clone(), "qw": qw0.clone(), "sw": sw0.clone(),
            "l1t": l10.clone() if (r and not lr4) else None, "l2t": l20.clone() if (r and not lr4) else None,
            "qx": torch.empty((b, m) if a8 else (b, m // 2), dtype=torch.uint8, device=dev),
            "sx": torch.empty((m // grp, b) if grp else (b,), dtype=torch.float32, device=dev),
            "t": torch.empty((b, r), dtype=torch.float32, device=dev) if (r and not lr4) else None,
            "y": torch.empty((b, n), dtype=torch.float16, device=dev),
        }
        if lr4:
            s_.update({"ql1": lp0["ql1"].clone() if r else None, "c": lp0["c"].clone() if r else None,
                       "ql2": lp0["ql2"].clone() if r else None,
                       "qh": torch.empty((b, r // 2), dtype=torch.uint8, device=dev) if r else None,
                       "sh": torch.empty((b,), dtype=torch.float32, device=dev) if r else None})
        sets.append(s_)
    del lp0
    L = twq.lib()
    ws, wsb = twq._workspace(dev, max(L.twq_quantize_act_workspace_bytes(b, m, r),
                                      L.twq_linear_lr4_workspace_bytes(b, m, n, r) if lr4
                                      else L.twq_linear_grouped_workspace_bytes(b, m, n, r, grp) if grp
                                      else L.twq_linear_a8_workspace_bytes(b, m, n, r) if a8
                                      else L.twq_linear_workspace_bytes(b, m, n, r)))
    P = lambda t: None if t is None else twq.ctypes.c_void_p(t.data_ptr())

    def layer(s, stream):
        if lr4:
            twq._check(L.twq_linear_lr4(P(s["x"]), P(s["qw"]), P(s["sw"]), P(s["ql1"]), P(s["c"]), P(s["ql2"]), r,
                                        P(s["y"]), b, m, n, P(ws), wsb, stream), "twq_linear_lr4")
            return
        if a8:
            twq._check(L.twq_linear_a8(P(s["x"]), P(s["qw"]), P(s["sw"]), P(s["l1t"]), P(s["l2t"]), r, P(s["y"]),
                                       b, m, n, P(ws), wsb, stream), "twq_linear_a8")
            return
        if grp:
            twq._check(L.twq_linear_grouped(P(s["x"]), P(s["qw"]), P(s["sw"]), P(s["l1t"]), P(s["l2t"]), r,
                                            P(s["y"]), b, m, n, grp, P(ws), wsb, stream), "twq_linear_grouped")
            return
        twq._check(L.twq_linear(P(s["x"]), P(s["qw"]), P(s["sw"]), P(s["l1t"]), P(s["l2t"]), r, P(s["y"]),
                                b, m, n, P(ws), wsb, stream), "twq_linear")

    def quant(s, stream):
        if a8:
            twq._check(L.twq_quantize_act_a8(P(s["x"]), b, m, P(s["qx"]), P(s["sx"]), P(s["l1t"]), r, P(s["t"]),
                                             P(ws), wsb, stream), "twq_quantize_act_a8")
            return
        if grp:
            twq._check(L.twq_quantize_act_grouped(P(s["x"]), b, m, grp, P(s["qx"]), P(s["sx"]), P(s["l1t"]), r,
                                                  P(s["t"]), P(ws), wsb, stream), "twq_quantize_act_grouped")
            return
        if lr4:
            twq._check(L.twq_quantize_act_lr4(P(s["x"]), b, m, P(s["ql1"]), P(s["c"]), r, P(s["qx"]), P(s["sx"]),
                                              P(s["qh"]), P(s["sh"]), stream), "twq_quantize_act_lr4")
            return
        twq._check(L.twq_quantize_act(P(s["x"]), b, m, P(s["qx"]), P(s["sx"]), P(s["l1t"]), r,
                                      P(s["t"]), P(ws), wsb, stream), "twq_quantize_act")

    def dual(s, stream):
        if a8:
            twq._check(L.twq_dual_linear_a8(P(s["qx"]), P(s["sx"]), P(s["qw"]), P(s["sw"]), P(s["t"]), P(s["l2t"]),
                                            r, P(s["y"]), b, m, n, stream), "twq_dual_linear_a8")
            return
        if lr4:
            twq._check(L.twq_dual_linear_lr4(P(s["qx"]), P(s["sx"]), P(s["qw"]), P(s["sw"]), P(s["qh"]),
                                             P(s["sh"]), P(s["ql2"]), r, P(s["y"]), b, m, n, stream),
                       "twq_dual_linear_lr4")
            return
        if grp:
            twq._check(L.twq_dual_linear_grouped(P(s["qx"]), P(s["sx"]), P(s["qw"]), P(s["sw"]), P(s["t"]),
                                                 P(s["l2t"]), r, P(s["y"]), b, m, n, grp, stream),
                       "twq_dual_linear_grouped")
            return
        twq._check(L.twq_dual_linear(P(s["qx"]), P(s["sx"]), P(s["qw"]), P(s["sw"]), P(s["t"]), P(s["l2t"]), r,
                                     P(s["y"]), b, m, n, stream), "twq_dual_linear")

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.Stream(dev)  # default priority

    def hs():
        return twq.ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def layer_main(s, stream):
        # the fused launch of the one-call layer alone, on the Q_X, s_X and T (or T's
        # partial sums) that an earlier call of the same shape left in the workspace
        if lr4:
            twq._check(L.twq_debug_linear_lr4_main(P(s["x"]), P(s["qw"]), P(s["sw"]), P(s["ql1"]), P(s["c"]),
                                                   P(s["ql2"]), r, P(s["y"]), b, m, n, P(ws), wsb, stream),
                       "twq_debug_linear_lr4_main")
        elif a8:
            twq._check(L.twq_debug_linear_a8_main(P(s["x"]), P(s["qw"]), P(s["sw"]), P(s["l1t"]), P(s["l2t"]), r,
                                                  P(s["y"]), b, m, n, P(ws), wsb, stream), "twq_debug_linear_a8_main")
        elif grp:
            twq._check(L.twq_debug_linear_grouped_main(P(s["x"]), P(s["qw"]), P(s["sw"]), P(s["l1t"]), P(s["l2t"]),
                                                       r, P(s["y"]), b, m, n, grp, P(ws), wsb, stream),
                       "twq_debug_linear_grouped_main")
        else:
            twq._check(L.twq_debug_linear_main(P(s["x"]), P(s["qw"]), P(s["sw"]), P(s["l1t"]), P(s["l2t"]), r,
                                               P(s["y"]), b, m, n, P(ws), wsb, stream), "twq_debug_linear_main")

    one_call = args.path == "linear"

    def steps_fn(k, with_quant=True, offset=0):
        # with_quant=False: the main-loop kernel alone, exactly as the timed step
        # launches it (the one-call layer's fused launch, or twq_dual_linear of the
        # split path), for its launch duration
        def run():
            st = hs()
            for i in range(k):
                s = sets[(i + offset) % copies]
                if not with_quant:
                    if one_call:
                        layer_main(s, st)
                    else:
                        dual(s, st)
                elif one_call:
                    layer(s, st)
                else:
                    quant(s, st)
                    dual(s, st)
        return run

    def timed(fn_or_graph, is_graph):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        if is_graph:
            fn_or_graph.replay()
        else:
            fn_or_graph()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1)  # ms

    with torch.cuda.stream(stream):
        # one eager call first (lazy initialisation, workspace), then the warmup steps;
        # Q_X, s_X and T of every copy are filled once for the kernel-only timing
        steps_fn(1)()
        for s_ in sets:
            quant(s_, hs())
        torch.cuda.synchronize()
        if args.eager:
            steps_fn(args.warmup)()
            ms = timed(steps_fn(args.steps), False)
            ms_dual = timed(steps_fn(args.steps, with_quant=False), False)
        else:
            gw = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gw, stream=stream):
                steps_fn(args.warmup)()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                steps_fn(args.steps)()
            gd = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gd, stream=stream):
                steps_fn(args.steps, with_quant=False)()
            gw.replay()
            torch.cuda.synchronize()
            ms = timed(g, True)
            gd.replay()  # untimed pass of the kernel-only graph
            ms_dual = timed(gd, True)
        torch.cuda.synchronize()

    ms_step = ms / args.steps
    us_dual = ms_dual / args.steps * 1e3
    ops = layer_ops(b, m, n, r)
    tops = ops / (ms_step * 1e-3) / 1e12
    decode = b <= 64
    kbytes = (dual_linear_lr4_bytes(b, m, n, r) if lr4 else dual_linear_grouped_bytes(b, m, n, r, grp) if grp
              else dual_linear_a8_bytes(b, m, n, r) if a8 else dual_linear_bytes(b, m, n, r))
    cbytes = per_copy
    traffic = None if (lr4 or grp or a8) else measured_traffic(args.config)
    if decode:
        ach = kbytes / (us_dual * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        ach = 2 * b * m * n / (us_dual * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "frac": round(ach / PEAK_INT8_TOPS, 4), "traffic": traffic}
    sfx = "_grouped" if grp else "_a8" if a8 else ""
    if lr4:
        sfx = "_lr4"
    roof["kernel"] = f"fused launch of twq_linear{sfx}" if one_call else f"twq_dual_linear{sfx}"
    roof["kernel_us"] = round(us_dual, 3)
    roof["algorithmic_bytes"] = kbytes
    roof["algorithmic_int8_ops"] = 2 * b * m * n

    if args.path == "linear":
        entry_points = f"twq_linear{sfx}"
    else:
        entry_points = f"twq_quantize_act{sfx}+twq_dual_linear{sfx}"
    out = {
        "metric": METRIC_NAME,
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "us_per_call": round(ms_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int4 codes on i8 MFMA (int32 acc), int4 low-rank on i8 MFMA" if lr4 else
                  "int4 weight x int8 activation codes on i8 MFMA (int32 acc) + fp16 low-rank (fp32 acc)" if a8 else
                  "int4 codes on i8 MFMA (int32 acc) + fp16 low-rank (fp32 acc)"),
        "data": "synthetic",
        "config": {"workload": f"{args.config}: b={b} m={m} n={n} r={r}", "b": b, "m": m, "n": n, "r": r,
                   "weight_copies_rotated": copies, "launch": "eager" if args.eager else "hip_graph",
                   "lowrank": args.lowrank, "group": grp or "per token / per channel", "act_bits": args.act_bits,
                   "entry_points": entry_points,
                   "call_bytes": cbytes,
                   "hbm_frac_whole_call": round(cbytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "int8_mfma_frac_whole_call": round(2 * b * m * n / (ms_step * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                   "seed": {"seed_sequence": synth.SEED_BASE, "spawn_key": cfg.index, "generator": "PCG64",
                            "synth_version": synth.GEN_VERSION}},
        "env": host_env(torch),
        "roofline": roof,
    }
    if not args.no_cpu:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = (_cpu_baseline_grouped(d, grp) if grp else _cpu_baseline_a8(d) if a8
                               else _cpu_baseline(d, lr4=lr4))
        out["cpu_baseline"]["host"] = cpu_model()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
