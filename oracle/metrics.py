"""Quality and size metrics (test infrastructure).

The SpectralQuant README lists cosine similarity, MSE and compression ratio as
the metrics of its ``metrics.py`` (Repository Structure) and reports a
per-vector cosine similarity and an analytical compression ratio (Headline
Results).  Reading: cosine is the mean over vectors of cos(x, x~) where x~ is
exactly what the scores see (including the QJL term)."""
from __future__ import annotations

import numpy as np


def cosine(x: np.ndarray, xt: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    xt = np.asarray(xt, np.float64)
    num = (x * xt).sum(axis=1)
    den = np.linalg.norm(x, axis=1) * np.linalg.norm(xt, axis=1)
    return num / np.where(den > 0, den, 1.0)


def rel_mse(x: np.ndarray, xt: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    e = ((x - np.asarray(xt, np.float64)) ** 2).sum(axis=1)
    n = (x * x).sum(axis=1)
    return e / np.where(n > 0, n, 1.0)


def bits_per_coord(widths, m: int, d: int) -> float:
    """Information bits per coordinate of one record: codes + QJL + gamma."""
    return (float(np.sum(widths)) + m + (16 if m > 0 else 0)) / d


def compression_ratio(bits_per_vector: float, d: int, ref_bits: int = 16) -> float:
    """Size of a 16-bit vector over the compressed size."""
    return ref_bits * d / bits_per_vector
