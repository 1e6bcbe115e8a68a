"""The library's packed Q_W layout, written as numpy index arithmetic for the tests.

The oracle packs each channel's codes as one row of m/2 bytes (two codes a byte, low
nibble first). The library stores the same bytes in 16-channel panels: channels
16p..16p+15 form panel p, a panel holds its m/128 pieces one after another, and a
piece holds the 64 bytes (128 codes) of each of the 16 channels in channel order. So
byte q of channel j lies at ((j // 16) * (m / 128) + q // 64) * 1024 + (j % 16) * 64 + q % 64.
"""
import numpy as np


def to_panels(rows: np.ndarray) -> np.ndarray:
    """Row-major packed codes [n][m/2] -> the panel layout (same shape, bytes moved)."""
    n, kb = rows.shape
    return np.ascontiguousarray(rows.reshape(n // 16, 16, kb // 64, 64).transpose(0, 2, 1, 3)).reshape(n, kb)


def from_panels(panels: np.ndarray) -> np.ndarray:
    """The panel layout [n][m/2] -> row-major packed codes."""
    n, kb = panels.shape
    return np.ascontiguousarray(panels.reshape(n // 16, kb // 64, 16, 64).transpose(0, 2, 1, 3)).reshape(n, kb)
