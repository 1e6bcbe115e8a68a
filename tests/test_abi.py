"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol include/twq.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import w4a4_rank_gemm_amd as twq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "twq.h")

OK, NULL, SHAPE, ALIGN, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3, 4, 6
A = ctypes.c_void_p(4096)       # an aligned, never-dereferenced address
MIS = ctypes.c_void_p(4096 + 8)  # misaligned


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(twq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = twq.lib()
    declared = _declared()
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(twq.EXPORTS)


def test_status_strings_and_version():
    L = twq.lib()
    assert L.twq_status_string(0) == b"ok"
    assert L.twq_status_string(2) == b"unsupported shape"
    assert L.twq_status_string(99) == b"unknown status"
    assert L.twq_version() >= 100


@pytest.mark.parametrize("b,m,r", [(1, 100, 0), (1, 0, 0), (1, 256, 8), (1, 256, 272), (-1, 256, 0),
                                   (1, 131072 + 128, 0)])
def test_quantize_act_rejects_shapes(b, m, r):
    st = twq.lib().twq_quantize_act(A, b, m, A, A, A, r, A, A, 1 << 30, None)
    assert st == SHAPE


def test_quantize_act_rejects_null_and_alignment():
    L = twq.lib()
    assert L.twq_quantize_act(None, 4, 256, A, A, None, 0, None, None, 0, None) == NULL
    assert L.twq_quantize_act(A, 4, 256, A, A, None, 32, A, None, 0, None) == NULL
    assert L.twq_quantize_act(MIS, 4, 256, A, A, None, 0, None, None, 0, None) == ALIGN
    assert L.twq_quantize_act(A, 4, 256, A, A, MIS, 32, A, A, 1 << 30, None) == ALIGN


def test_quantize_act_workspace():
    L = twq.lib()
    need = L.twq_quantize_act_workspace_bytes(2048, 4096, 32)  # many tokens: K-slice partial sums
    assert need > 0 and need % (2048 * 32 * 4) == 0
    assert L.twq_quantize_act_workspace_bytes(2048, 4096, 0) == 0
    assert L.twq_quantize_act_workspace_bytes(16, 4096, 32) % (16 * 32 * 4) == 0  # few tokens: K slices
    assert L.twq_quantize_act_workspace_bytes(16, 4096, 0) == 0
    assert L.twq_quantize_act_workspace_bytes(16, 100, 32) == 0  # invalid shape
    assert L.twq_quantize_act(A, 2048, 4096, A, A, A, 32, A, None, 0, None) == WORKSPACE
    assert L.twq_quantize_act_a8(A, 2048, 4096, A, A, A, 32, A, None, 0, None) == WORKSPACE
    assert L.twq_quantize_act_grouped(A, 2048, 4096, 128, A, A, A, 32, A, A, need - 1, None) == WORKSPACE
    assert L.twq_quantize_act(A, 16, 4096, A, A, A, 32, A, None, 0, None) == WORKSPACE  # few tokens


def test_empty_calls_are_no_ops():
    L = twq.lib()
    assert L.twq_quantize_act(None, 0, 256, None, None, None, 0, None, None, 0, None) == OK
    assert L.twq_pack_weight(None, 0, 256, None, None, None) == OK
    assert L.twq_dual_linear(None, None, None, None, None, None, 0, None, 0, 256, 64, None) == OK
    assert L.twq_dual_linear(None, None, None, None, None, None, 0, None, 8, 256, 0, None) == OK
    assert L.twq_debug_residual_acc(None, None, None, 0, 256, 16, None) == OK


@pytest.mark.parametrize("b,m,n,r", [(4, 256, 24, 0), (4, 200, 32, 0), (4, 256, 32, 48 + 8),
                                     (1 << 25, 256, 32, 0), (4, 256, -16, 0)])
def test_dual_linear_rejects_shapes(b, m, n, r):
    assert twq.lib().twq_dual_linear(A, A, A, A, A, A, r, A, b, m, n, None) == SHAPE


def test_dual_linear_rejects_null_and_alignment():
    L = twq.lib()
    assert L.twq_dual_linear(A, A, A, A, None, None, 32, A, 4, 256, 32, None) == NULL
    assert L.twq_dual_linear(A, None, A, A, None, None, 0, A, 4, 256, 32, None) == NULL
    assert L.twq_dual_linear(A, A, A, A, None, None, 0, MIS, 4, 256, 32, None) == ALIGN
    assert L.twq_pack_weight(A, 32, 256, MIS, A, None) == ALIGN
    assert L.twq_pack_weight(A, 24, 256, A, A, None) == SHAPE
    assert L.twq_debug_residual_acc(A, None, A, 4, 256, 32, None) == NULL


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    x = torch.zeros(4, 256, dtype=torch.float16)
    with pytest.raises(ValueError):
        twq.quantize_act(x)


def test_lowrank_int4_validation():
    L = twq.lib()
    # ranks must be a multiple of 32 for the int4 low-rank variant
    assert L.twq_pack_lowrank_int4(A, A, 16, 256, 32, A, A, A, A, A, None) == SHAPE
    assert L.twq_quantize_act_lr4(A, 4, 256, A, A, 48, A, A, A, A, None) == SHAPE
    assert L.twq_quantize_act_lr4(A, 4, 256, A, A, 0, A, A, A, A, None) == SHAPE
    assert L.twq_quantize_act_lr4(A, 4, 256, A, A, 288, A, A, A, A, None) == SHAPE
    assert L.twq_linear_lr4(A, A, A, A, A, A, 48, A, 4, 256, 32, A, 1 << 30, None) == SHAPE
    assert L.twq_dual_linear_lr4(A, A, A, A, A, A, A, 16, A, 4, 256, 32, None) == SHAPE
    assert L.twq_pack_lowrank_int4(None, A, 32, 256, 32, A, A, A, A, A, None) == NULL
    assert L.twq_quantize_act_lr4(A, 4, 256, None, A, 32, A, A, A, A, None) == NULL
    assert L.twq_quantize_act_lr4(A, 4, 256, A, A, 32, A, A, None, A, None) == NULL
    assert L.twq_debug_lr4_h(A, 4, 256, A, A, 32, None, A, A, A, A, None) == NULL
    assert L.twq_quantize_act_lr4(A, 4, 256, A, MIS, 32, A, A, A, A, None) == ALIGN
    assert L.twq_linear_lr4(A, A, A, A, A, None, 32, A, 4, 256, 32, A, 1 << 30, None) == NULL
    need = L.twq_linear_lr4_workspace_bytes(4, 256, 32, 32)
    assert need >= 4 * 128 + 4 * 4 + 4 * 16 + 4 * 4
    assert L.twq_linear_lr4(A, A, A, A, A, A, 32, A, 4, 256, 32, A, need - 1, None) == WORKSPACE
    assert L.twq_linear_lr4(A, A, A, A, A, A, 32, A, 4, 256, 32, None, need, None) == WORKSPACE
    assert L.twq_dual_linear_lr4(A, A, A, A, None, A, A, 32, A, 4, 256, 32, None) == NULL
    assert L.twq_dual_linear_lr4(A, A, A, A, A, A, MIS, 32, A, 4, 256, 32, None) == ALIGN
    # empty calls
    assert L.twq_pack_lowrank_int4(None, None, 0, 256, 32, None, None, None, None, None, None) == OK
    assert L.twq_quantize_act_lr4(None, 0, 256, None, None, 32, None, None, None, None, None) == OK
    assert L.twq_linear_lr4(None, None, None, None, None, None, 32, None, 0, 256, 32, None, 0, None) == OK
    assert L.twq_dual_linear_lr4(None, None, None, None, None, None, None, 32, None, 0, 256, 32, None) == OK


def test_linear_validation():
    L = twq.lib()
    need = L.twq_linear_workspace_bytes(16, 4096, 4096, 32)
    assert need >= 16 * 4096 // 2 + 16 * 4
    assert L.twq_linear_workspace_bytes(16, 100, 4096, 32) == 0
    assert L.twq_linear(A, A, A, A, A, 32, A, 16, 4096, 4096, A, need - 1, None) == WORKSPACE
    assert L.twq_linear(A, A, A, A, A, 32, A, 16, 4096, 4096, None, need, None) == WORKSPACE
    assert L.twq_linear(A, A, A, None, A, 32, A, 16, 4096, 4096, A, need, None) == NULL
    assert L.twq_linear(MIS, A, A, A, A, 32, A, 16, 4096, 4096, A, need, None) == ALIGN
    assert L.twq_linear(A, A, A, A, A, 24, A, 16, 4096, 4096, A, need, None) == SHAPE
    assert L.twq_linear(A, A, A, A, A, 32, A, 16, 4096, 40, A, need, None) == SHAPE
    assert L.twq_linear(None, None, None, None, None, 32, None, 0, 4096, 4096, None, 0, None) == OK


def test_grouped_validation():
    """Group-wise entry points: only g = 128 is supported; the other checks are those of the
    per-token entry points, and a grouped layer needs room for m/128 scales per token."""
    L = twq.lib()
    for g in (64, 256, 0, -128):
        assert L.twq_quantize_act_grouped(A, 16, 4096, g, A, A, None, 0, None, None, 0, None) == UNSUPPORTED
        assert L.twq_pack_weight_grouped(A, 64, 4096, g, A, A, None) == UNSUPPORTED
        assert L.twq_dual_linear_grouped(A, A, A, A, None, None, 0, A, 16, 4096, 64, g, None) == UNSUPPORTED
        assert L.twq_linear_grouped_workspace_bytes(16, 4096, 64, 0, g) == 0
    assert L.twq_quantize_act_grouped(A, 16, 4000, 128, A, A, None, 0, None, None, 0, None) == SHAPE
    assert L.twq_quantize_act_grouped(None, 16, 4096, 128, A, A, None, 0, None, None, 0, None) == NULL
    assert L.twq_pack_weight_grouped(A, 40, 4096, 128, A, A, None) == SHAPE
    assert L.twq_pack_weight_grouped(A, 64, 4096, 128, MIS, A, None) == ALIGN
    assert L.twq_dual_linear_grouped(A, A, A, A, None, None, 32, A, 16, 4096, 64, 128, None) == NULL
    assert L.twq_dual_linear_grouped(A, A, A, A, None, None, 0, A, 0, 4096, 64, 128, None) == OK
    per_token = L.twq_linear_workspace_bytes(16, 4096, 4096, 32)
    grouped = L.twq_linear_grouped_workspace_bytes(16, 4096, 4096, 32, 128)
    assert grouped >= per_token + 16 * 4 * (4096 // 128 - 1) - 255
    assert L.twq_linear_grouped(A, A, A, A, A, 32, A, 16, 4096, 4096, 128, A, grouped - 1, None) == WORKSPACE
    assert L.twq_linear_grouped(None, None, None, None, None, 32, None, 0, 4096, 4096, 128, None, 0, None) == OK


def test_a8_validation():
    L = twq.lib()
    assert L.twq_quantize_act_a8(A, 16, 4000, A, A, None, 0, None, None, 0, None) == SHAPE
    assert L.twq_quantize_act_a8(None, 16, 4096, A, A, None, 0, None, None, 0, None) == NULL
    assert L.twq_quantize_act_a8(A, 0, 4096, None, None, None, 0, None, None, 0, None) == OK
    assert L.twq_dual_linear_a8(A, A, A, A, None, None, 32, A, 16, 4096, 64, None) == NULL
    assert L.twq_dual_linear_a8(A, A, MIS, A, None, None, 0, A, 16, 4096, 64, None) == ALIGN
    assert L.twq_dual_linear_a8(A, A, A, A, None, None, 0, A, 16, 4096, 40, None) == SHAPE
    assert L.twq_debug_residual_acc_a8(A, A, None, 16, 4096, 64, None) == NULL
    need4 = L.twq_linear_workspace_bytes(16, 4096, 4096, 32)
    need8 = L.twq_linear_a8_workspace_bytes(16, 4096, 4096, 32)
    assert need8 >= need4 + 16 * 4096 // 2 - 255  # one byte per activation code instead of half a byte
    assert L.twq_linear_a8(A, A, A, A, A, 32, A, 16, 4096, 4096, A, need8 - 1, None) == WORKSPACE
    assert L.twq_linear_a8(None, None, None, None, None, 32, None, 0, 4096, 4096, None, 0, None) == OK


def test_panel_layout_helpers_follow_the_documented_offsets():
    """tests/panels.py against the offset formula of twq.h, by an explicit loop:
    byte t of channel j at ((j / 16)(m / 128) + t / 64) 1024 + (j % 16) 64 + t % 64."""
    from tests.panels import from_panels, to_panels
    rng = np.random.default_rng(7)
    n, m = 48, 384
    rows = rng.integers(0, 256, (n, m // 2), dtype=np.uint8)
    flat = np.zeros(n * m // 2, np.uint8)
    for j in range(n):
        for t in range(m // 2):
            flat[((j // 16) * (m // 128) + t // 64) * 1024 + (j % 16) * 64 + t % 64] = rows[j, t]
    assert np.array_equal(to_panels(rows).reshape(-1), flat)
    assert np.array_equal(from_panels(to_panels(rows)), rows)


def test_linear_noalloc_limits_and_checks():
    """twq_linear_noalloc: the same argument checks as twq_linear, and a size above its
    fixed scratch array is refused before any HIP call."""
    L = twq.lib()
    cap = L.twq_linear_noalloc_max_bytes()
    assert cap == 64 << 20
    assert L.twq_linear_noalloc(A, A, A, A, A, 32, A, 16, 100, 4096, None) == SHAPE
    assert L.twq_linear_noalloc(None, A, A, A, A, 32, A, 16, 4096, 4096, None) == NULL
    assert L.twq_linear_noalloc(A, A, A, None, A, 32, A, 16, 4096, 4096, None) == NULL
    assert L.twq_linear_noalloc(A, MIS, A, A, A, 32, A, 16, 4096, 4096, None) == ALIGN
    assert L.twq_linear_noalloc(A, A, A, A, A, 32, A, 0, 4096, 4096, None) == OK  # empty call
    # the largest token count whose scratch fits, and the next that does not
    m, n, r = 8192, 28672, 128
    fits = [b for b in (32, 1024, 4096, 8192, 16384, 65536)
            if L.twq_linear_workspace_bytes(b, m, n, r) <= cap]
    big = [b for b in (32, 1024, 4096, 8192, 16384, 65536) if b not in fits]
    assert 8192 in fits and big, (fits, big)
    assert L.twq_linear_noalloc(A, A, A, A, A, r, A, big[0], m, n, None) == WORKSPACE


def test_fold_validation():
    """twq_fold_lowrank rejects bad shapes, missing operands and short workspaces before
    any HIP call (r == 0 needs no workspace)."""
    L = twq.lib()
    need = L.twq_fold_workspace_bytes(512, 384, 32)
    assert need >= (512 * 32 * 2 + 32 * 384 + 3 * 32 * 32) * 8
    assert L.twq_fold_workspace_bytes(512, 384, 0) == 0
    assert L.twq_fold_workspace_bytes(512, 16, 32) == 0  # r > n
    args = lambda r, ws, wsb, u=A: (A, u, A, A, A, A, 512, 384, r, A, A, A, ws, wsb, None)
    assert L.twq_fold_lowrank(*args(32, A, need - 1)) == WORKSPACE
    assert L.twq_fold_lowrank(*args(32, A, need, u=None)) == NULL
    assert L.twq_fold_lowrank(*args(520, A, need)) == SHAPE
    assert L.twq_fold_lowrank(*args(32, MIS, need)) == ALIGN
