"""Rounding ties and near-ties of the activation quantizer (TwinQuant page 1, section 2,
eq. (1)), GPU against the oracle bit for bit.

The GPU quantizer multiplies by fl32(1/s) and falls back to the correctly rounded
division only when the product is within 2^-18 of a half-integer, so rows are built
whose ratios v/s sit exactly on k + 1/2 (s a power of two) or within a few fp16 ulps
of it (any s), on both sides of zero.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a4_rank_gemm_amd as twq

pytestmark = pytest.mark.gpu


def _row(amax: np.float16, m: int, rng) -> np.ndarray:
    s = np.float32(np.float32(amax) / np.float32(7))
    vals = [amax, -amax]
    for k in range(-7, 7):
        h = np.float16((k + 0.5) * float(s))
        for _ in range(3):
            h = np.nextafter(h, np.float16(-np.inf))
        for _ in range(7):  # fp16 neighbours of (k + 1/2) s, three ulps either side
            if abs(float(h)) <= float(amax):
                vals.append(h)
            h = np.nextafter(h, np.float16(np.inf))
    vals = np.array(vals, dtype=np.float16)
    row = (rng.uniform(-1, 1, m) * float(amax)).astype(np.float16)
    row[: len(vals)] = vals
    row[np.abs(row.astype(np.float32)) > np.float32(amax)] = amax
    return row


@pytest.mark.parametrize("m", [512, 4096])
def test_quantizer_ties_match_oracle(m):
    rng = synth.rng_for(4242 + m)
    amaxes = [np.float16(7 * 2.0 ** j) for j in range(-6, 5)]          # s a power of two: exact ties
    amaxes += [np.float16(v) for v in rng.uniform(0.01, 600.0, 245)]   # any s: near-ties
    x = np.stack([_row(a, m, rng) for a in amaxes])
    _, qx_ref, sx_ref = oracle.quantize_act(x)  # (codes, packed codes, scales)
    qx, sx, _ = twq.quantize_act(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(qx.cpu().numpy(), qx_ref)


def test_quantizer_ties_few_tokens():
    """Few tokens take the same quantizer through several CTAs per row."""
    rng = synth.rng_for(77)
    x = np.stack([_row(np.float16(7 * 2.0 ** j), 4096, rng) for j in (-2, 0, 3)])
    _, qx_ref, sx_ref = oracle.quantize_act(x)  # (codes, packed codes, scales)
    qx, sx, _ = twq.quantize_act(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(qx.cpu().numpy(), qx_ref)
