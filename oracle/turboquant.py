"""TurboQuant-style random-rotation baseline (test infrastructure).

Built from the scos-lab "TurboQuant" README's description of its modules
(Project Structure: TurboQuantMSE and TurboQuantProd, a random orthogonal
rotation, a scalar quantiser optimal for the coordinate law of a rotated unit
vector, and a 1-bit QJL inner-product sketch) and its finding that Prod is used
for keys and MSE for values (Key Findings, item 2).  It is prior art, used here
only as the comparison point the SpectralQuant README measures against.

Reading: for d >= 128 a coordinate of a random unit vector is close to
N(0, 1/d), so the scalar codebook is the Gaussian Lloyd-Max codebook scaled by
1/sqrt(d) (its distortion reproduces the README's Algorithm Correctness table).
"""
from __future__ import annotations

import math

import numpy as np

from .record import record_words, field_offsets
from .spectralquant import Calibration, lloyd_max_gaussian


def _codebook(bits: int, d: int):
    c, t = lloyd_max_gaussian(bits)
    return c / math.sqrt(d), t / math.sqrt(d)


def tq_mse_unit(w: np.ndarray, bits: int) -> np.ndarray:
    """Quantise each coordinate of (rotated) unit vectors w [T, d] with the
    ``bits``-bit codebook; returns the reconstruction."""
    d = w.shape[1]
    c, t = _codebook(bits, d)
    return c[np.searchsorted(t, w, side="left")]


def tq_mse_values(x: np.ndarray, rot: np.ndarray, bits: int) -> np.ndarray:
    """TurboQuant-MSE: nu = ||x||, w = Pi x / nu, x~ = nu Pi^T Q_b(w)."""
    x = np.asarray(x, np.float64)
    nu = np.linalg.norm(x, axis=1, keepdims=True)
    w = (x @ rot.T) / np.where(nu > 0, nu, 1.0)
    return nu * (tq_mse_unit(w, bits) @ rot)


def tq_prod_keys(x: np.ndarray, rot: np.ndarray, sketch: np.ndarray, bits: int) -> np.ndarray:
    """TurboQuant-Prod: (bits-1)-bit MSE stage on the rotated unit vector, then
    a 1-bit QJL sketch of the residual over ALL d dims:
    x~ = nu Pi^T ( w^ + sqrt(pi/2)/d * ||rho|| * S^T sign(S rho) )."""
    x = np.asarray(x, np.float64)
    d = x.shape[1]
    nu = np.linalg.norm(x, axis=1, keepdims=True)
    w = (x @ rot.T) / np.where(nu > 0, nu, 1.0)
    wh = tq_mse_unit(w, bits - 1) if bits > 1 else np.zeros_like(w)
    rho = w - wh
    sgn = np.where(rho @ sketch.T >= 0, 1.0, -1.0)
    corr = (math.sqrt(math.pi / 2) / d) * np.linalg.norm(rho, axis=1, keepdims=True) * (sgn @ sketch)
    return nu * ((wh + corr) @ rot)


def tq_calibration(rot: np.ndarray, sketch, bits: int, keys: bool) -> Calibration:
    """The TurboQuant-style scheme written as a calibration of the generic
    (normalised, R8) SpectralQuant pipeline, so the same compress / dequantize
    / scores / attend and record layout run it: rotation Pi = rot (rows), every
    coordinate at width bits - 1 (keys: the MSE stage) or bits (values) with
    the Gaussian Lloyd-Max codebook scaled by 1/sqrt(d), the QJL sketch over
    all d coordinates (keys: m = d rows of ``sketch``), per-vector norm stored.
    Coordinate scale sigma_i = 1/sqrt(d), the law of a rotated unit vector's
    coordinate (it sets the parity band)."""
    rot = np.asarray(rot, np.float64)
    d = rot.shape[0]
    b = bits - 1 if keys else bits
    c, t = _codebook(b, d) if b > 0 else (np.zeros(1), np.zeros(0))
    widths = np.full(d, b, dtype=np.int64)
    m = d if keys else 0
    S = np.asarray(sketch, np.float32).astype(np.float64)[:m, :d] if keys else np.zeros((0, d))
    sigma = np.full(d, 1.0 / math.sqrt(d))
    return Calibration(d, rot.copy(), sigma ** 2, sigma, float(d), d, math.inf, widths,
                       [t.copy() for _ in range(d)], [c.copy() for _ in range(d)], {}, m, S,
                       record_words(widths, m, True), field_offsets(widths), int(widths.sum()), m > 0,
                       True)
