"""Host logic of bench.py: the one-GPU refusal, the byte and operation counts the roofline
divides by (checked on the o_proj decode shape, tensor by tensor), and the CPU-oracle
sample size."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def test_dual_linear_bytes_on_the_o_proj_shape():
    # b=16 tokens, m=n=4096, r=32: Q_X 16*4096/2, s_X 16*4, Q_W 4096*4096/2, s_W 4096*4,
    # T 16*32*4, L2^T 4096*32*2, Y 16*4096*2
    parts = [32768, 64, 8388608, 16384, 2048, 262144, 131072]
    assert bench.dual_linear_bytes(16, 4096, 4096, 32) == sum(parts) == 8833088
    # W4A8 reads one byte per activation code instead of half a byte
    assert bench.dual_linear_a8_bytes(16, 4096, 4096, 32) == sum(parts) + 32768
    # group-wise: one scale per 128 elements of each token row and output channel
    assert bench.dual_linear_grouped_bytes(16, 4096, 4096, 32, 128) == sum(parts) + 64 * 31 + 16384 * 31


def test_layer_ops():
    assert bench.layer_ops(16, 4096, 4096, 32) == 2 * 16 * 4096 * 4096 + 2 * 16 * 32 * 8192
    assert bench.layer_ops(8, 128, 16, 0) == 2 * 8 * 128 * 16


def test_cpu_sample_covers_whole_calls_unless_they_are_very_large():
    assert bench._cpu_rows(16, 4096, 4096) == 16
    assert bench._cpu_rows(4096, 14336, 4096) == 4096
    rows = bench._cpu_rows(8192, 8192, 28672)  # the 70B prefill call: about 1.9e12 multiply-adds
    assert 16 <= rows < 8192 and rows * 8192 * 28672 <= bench.CPU_MACS_PER_CALL
    assert "first 1277 of 8192 tokens" in bench._cpu_sample(2, rows, 8192, 8192, 28672, 128, 14.0, "")
