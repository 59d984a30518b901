"""SpectralQuant, step by step, in float64 NumPy (test infrastructure only).

Calibration follows the ``pre_computed_calibration`` fixture of the
spectralquant repository's ``tests/conftest.py`` for the second-moment matrix,
the eigen-order, d_eff and the spectral gap, and the README's "Repository
Structure" (calibration: PCA, d_eff, kappa; spectral rotation; Lloyd-Max with
per-regime codebooks; QJL correction on signal dims only) plus the ossradar.top
summary's core-capability list (water-filled non-uniform bit allocation,
Lloyd-Max codebooks per region) for the rest.

Readings taken where the pages are silent (each repeated at its function):
  R1  eigenvector sign: the entry of largest magnitude is made positive.
  R2  integer reverse water-filling = greedy marginal allocation on
      lambda_i * 4**(-b_i), ties to the lower index, widths capped at max_bits.
  R3  region = (regime, width); regime = signal for the top d_eff eigen-
      coordinates, noise otherwise; one codebook per region, fitted on the
      pooled samples standardised by sigma_i = sqrt(lambda_i).
  R4  Lloyd-Max on samples: start at the sample quantiles (j + 1/2) / L,
      alternate midpoint thresholds / cell means until the partition repeats
      or the iteration cap; an empty cell keeps its level.
  R5  no per-vector norm; sigma_i is folded into per-coordinate tables.
  R6  QJL on keys only: m = qjl_bits * d_eff Gaussian rows over the signal
      residual r; z_j = [ (S r)_j >= 0 ]; gamma = ||r|| stored as IEEE half;
      estimator factor sqrt(pi/2) / m.
  R7  code_i = #{ j : threshold_ij < y_i } (a tie goes to the lower cell, NaN
      gives 0); a zero-width coordinate reconstructs to 0.
  R8  normalised variant (README Repository Structure lists normalised and
      unnormalised result sets; TurboQuant stores a per-vector norm): every
      sample is divided by its norm before calibration, and at compression
      the vector's norm nu is stored (IEEE half) and the unit vector x / nu
      is rotated and quantised; reconstructions, scores and value sums are
      scaled back by the stored nu.  A zero vector keeps nu = 0.
  R9  d_eff by cumulative variance (README Repository Structure: the deff
      sweep compares the participation ratio with a cumulative-variance
      rule, threshold not given): the smallest k whose k leading eigenvalues
      sum to at least a caller-given fraction of the total.
  R10 calibration stability (README paper-section table: a calibration
      coefficient of variation, no definition given): the population
      coefficient of variation (std / mean, numpy's default ddof = 0) of the
      participation ratio and of d_eff across calibrations of one head on
      disjoint, equally sized sample sets.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
from scipy.special import ndtr

from .record import record_words, field_offsets


# --------------------------------------------------------------------------
# Calibration
# --------------------------------------------------------------------------

def second_moment(x: np.ndarray) -> np.ndarray:
    """C = X^T X / n, uncentered (conftest ``pre_computed_calibration``)."""
    x = np.asarray(x, dtype=np.float64)
    return x.T @ x / x.shape[0]


def eigenbasis(c: np.ndarray):
    """Eigenvalues in descending order and the matching unit eigenvectors as
    the ROWS of R (so y = R x), as in the conftest fixture (eigh, then reversed).
    Negative round-off eigenvalues are clamped to 0.  Sign rule R1: the entry
    of largest magnitude in each eigenvector is positive (first such entry on
    an exact tie)."""
    lam, v = np.linalg.eigh(c)
    lam = np.maximum(lam[::-1].copy(), 0.0)
    v = v[:, ::-1].copy()
    for k in range(v.shape[1]):
        j = int(np.argmax(np.abs(v[:, k])))
        if v[j, k] < 0:
            v[:, k] = -v[:, k]
    return lam, v.T.copy()


def participation_ratio(lam: np.ndarray) -> float:
    """(sum lambda)^2 / sum lambda^2 (conftest fixture's d_eff before rounding)."""
    lam = np.asarray(lam, dtype=np.float64)
    s2 = float((lam ** 2).sum())
    return float(lam.sum() ** 2 / s2) if s2 > 0 else 0.0


def effective_dim(lam: np.ndarray) -> int:
    """d_eff = int(round(PR)) as in the conftest fixture (Python round: half to
    even), clamped to [1, d]."""
    d = len(lam)
    return int(min(max(int(round(participation_ratio(lam))), 1), d))


def effective_dim_cumvar(lam: np.ndarray, fraction: float) -> int:
    """d_eff by cumulative variance (reading R9): the smallest k in [1, d]
    with lambda_0 + ... + lambda_{k-1} >= fraction * (lambda_0 + ... +
    lambda_{d-1}), partial sums taken left to right; fraction in (0, 1]."""
    if not 0.0 < fraction <= 1.0:
        raise ValueError("fraction must be in (0, 1]")
    lam = np.asarray(lam, dtype=np.float64)
    csum = np.cumsum(lam)                  # sequential partial sums
    total = csum[-1]
    for k in range(1, len(lam) + 1):
        if csum[k - 1] >= fraction * total:
            return k
    return len(lam)


def coefficient_of_variation(values) -> float:
    """Population std / mean (reading R10)."""
    v = np.asarray(values, dtype=np.float64)
    return float(v.std() / v.mean())


def calibration_stability(samples: np.ndarray, n_splits: int, deff_cumvar: float = 0.0,
                          normalize: bool = False) -> dict:
    """Reading R10: split the calibration samples [n, d] into n_splits
    contiguous, disjoint, equal parts (a remainder is dropped), take each
    part's spectrum (second moment, eigenvalues) and report the participation
    ratio and d_eff of every part with their coefficients of variation."""
    x = np.asarray(samples, dtype=np.float64)
    if normalize:
        x, _ = _unit_rows(x)
    per = x.shape[0] // n_splits
    if per < 2:
        raise ValueError("each split needs at least 2 samples")
    prs, deffs = [], []
    for k in range(n_splits):
        lam, _ = eigenbasis(second_moment(x[k * per:(k + 1) * per]))
        prs.append(participation_ratio(lam))
        deffs.append(effective_dim_cumvar(lam, deff_cumvar) if deff_cumvar > 0 else effective_dim(lam))
    return dict(pr=np.array(prs), d_eff=np.array(deffs), pr_cv=coefficient_of_variation(prs),
                deff_cv=coefficient_of_variation(deffs), samples_per_split=per)


def spectral_gap(lam: np.ndarray, d_eff: int) -> float:
    """kappa = lambda[d_eff-1] / lambda[d_eff], infinite when d_eff == d
    (conftest fixture) or when lambda[d_eff] is zero."""
    if d_eff >= len(lam) or lam[d_eff] <= 0:
        return math.inf
    return float(lam[d_eff - 1] / lam[d_eff])


def water_fill(lam: np.ndarray, total_bits: int, max_bits: int = 8) -> np.ndarray:
    """Reverse water-filling of an integer bit budget over eigenvalues (R2).

    Each of ``total_bits`` steps gives one more bit to the coordinate whose
    current distortion proxy lambda_i * 4**(-b_i) is largest (a bit divides a
    Gaussian coordinate's MSE by about 4).  Ties go to the lowest index.  When
    every coordinate is at ``max_bits`` the rest of the budget is unused."""
    lam = np.asarray(lam, dtype=np.float64)
    b = np.zeros(len(lam), dtype=np.int64)
    for _ in range(int(total_bits)):
        score = lam * np.power(4.0, -b.astype(np.float64))
        score[b >= max_bits] = -np.inf
        i = int(np.argmax(score))
        if score[i] == -np.inf:
            break
        b[i] += 1
    return b


def regions(widths: np.ndarray, d_eff: int):
    """Map (regime, width) -> list of coordinates (R3).  Regime 0 = signal
    (i < d_eff), 1 = noise.  Zero-width coordinates belong to no region."""
    out: dict = {}
    for i, b in enumerate(widths):
        if b <= 0:
            continue
        out.setdefault((0 if i < d_eff else 1, int(b)), []).append(i)
    return out


def lloyd_max_samples(u: np.ndarray, levels: int, max_iter: int = 200):
    """Lloyd-Max scalar quantiser fitted to samples (R4).

    Returns (centroids[L], thresholds[L-1], iterations, converged).  Cell j is
    (t_{j-1}, t_j]; thresholds are midpoints of adjacent centroids; centroids
    are cell means.  Start: the sample quantile of order (j + 1/2)/L, i.e.
    sorted[floor((2j+1) N / (2L))].  Stop when the partition repeats (then both
    optimality conditions hold exactly) or after ``max_iter`` updates."""
    u = np.sort(np.asarray(u, dtype=np.float64))
    n = len(u)
    L = int(levels)
    if n == 0:
        c = np.zeros(L)
        return c, (c[:-1] + c[1:]) / 2, 0, True
    c = u[(np.arange(L, dtype=np.int64) * 2 + 1) * n // (2 * L)].copy()
    prefix = np.concatenate([[0.0], np.cumsum(u)])
    prev = None
    updates = 0
    converged = False
    while True:
        t = (c[:-1] + c[1:]) / 2
        k = np.searchsorted(u, t, side="right")          # k_j = #{u <= t_j}
        if prev is not None and np.array_equal(k, prev):
            converged = True                              # c = means of its own partition
            break
        if updates == max_iter:
            break
        edges = np.concatenate([[0], k, [n]])
        cnt = np.diff(edges)
        sums = prefix[edges[1:]] - prefix[edges[:-1]]
        nz = cnt > 0
        c = c.copy()
        c[nz] = sums[nz] / cnt[nz]
        prev = k
        updates += 1
    return c, (c[:-1] + c[1:]) / 2, updates, converged


def _phi(x):
    return np.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def lloyd_max_gaussian(bits: int, tol: float = 1e-14, max_iter: int = 100000):
    """Lloyd-Max quantiser of the standard normal density (Max, 1960).
    Centroid of (a, b]: (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  Returns
    (centroids, thresholds)."""
    L = 2 ** bits
    c = np.linspace(-2.0, 2.0, L) if L > 1 else np.zeros(1)
    for _ in range(max_iter):
        t = (c[:-1] + c[1:]) / 2
        a = np.concatenate([[-np.inf], t])
        b = np.concatenate([t, [np.inf]])
        pa = np.where(np.isinf(a), 0.0, _phi(np.where(np.isinf(a), 0.0, a)))
        pb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
        mass = ndtr(b) - ndtr(a)
        cn = (pa - pb) / mass
        if np.max(np.abs(cn - c)) < tol:
            c = cn
            break
        c = cn
    return c, (c[:-1] + c[1:]) / 2


def gaussian_distortion(centroids: np.ndarray, thresholds: np.ndarray) -> float:
    """E[(Z - Q(Z))^2] for Z ~ N(0,1) and the quantiser (c, t), in closed form:
    per cell (a, b] with mass P:  E[Z^2; cell] - 2 c E[Z; cell] + c^2 P, where
    E[Z^2; cell] = P + a phi(a) - b phi(b) and E[Z; cell] = phi(a) - phi(b)."""
    c = np.asarray(centroids, float)
    a = np.concatenate([[-np.inf], thresholds])
    b = np.concatenate([thresholds, [np.inf]])
    fa = np.where(np.isinf(a), 0.0, _phi(np.where(np.isinf(a), 0.0, a)))
    fb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
    afa = np.where(np.isinf(a), 0.0, np.where(np.isinf(a), 0.0, a) * fa)
    bfb = np.where(np.isinf(b), 0.0, np.where(np.isinf(b), 0.0, b) * fb)
    p = ndtr(b) - ndtr(a)
    # E[Z^2; cell] = P + a phi(a) - b phi(b);  E[Z; cell] = phi(a) - phi(b)
    return float(np.sum(p + afa - bfb - 2 * c * (fa - fb) + c * c * p))


@dataclasses.dataclass
class Calibration:
    """One head's calibration artifact (all float64 except the QJL matrix,
    which is the float32 Gaussian draw it was given)."""
    head_dim: int
    R: np.ndarray              # [d, d] rows = eigenvectors, descending lambda
    lam: np.ndarray            # [d]
    sigma: np.ndarray          # [d] sqrt(lambda)
    pr: float
    d_eff: int
    kappa: float
    widths: np.ndarray         # [d] int
    thresholds: list           # per coordinate: sigma_i * t (len 2^b - 1)
    centroids: list            # per coordinate: sigma_i * c (len 2^b)
    unit_codebooks: dict       # region -> (c, t, iterations, converged, n_samples)
    m: int                     # QJL rows
    S: np.ndarray              # [m, d_eff] float64 copy of the float32 draw
    W: int                     # record words
    offsets: np.ndarray        # [d] bit offset of each code field
    qjl_offset: int            # bit offset of z_0
    has_gamma: bool
    normalized: bool = False   # R8: per-vector norm stored, unit vectors quantised


def _unit_rows(x: np.ndarray):
    """(x / |x| row-wise, |x|); zero rows stay zero."""
    nu = np.sqrt((x * x).sum(axis=1))
    return x / np.where(nu > 0, nu, 1.0)[:, None], nu


def calibrate(samples: np.ndarray, avg_bits: float, qjl_bits: int,
              gauss: Optional[np.ndarray], max_bits: int = 8,
              lloyd_iters: int = 200, normalize: bool = False,
              deff_cumvar: float = 0.0) -> Calibration:
    """Calibrate one head on ``samples`` [n, d] (normalised variant R8: on the
    samples divided by their norms).

    1. C = X^T X / n; eigh; descending; sign rule R1; R = V^T.
    2. d_eff = round(PR) (conftest fixture), or by cumulative variance when
       deff_cumvar > 0 (R9); kappa.
    3. widths by greedy water-filling of round(avg_bits * d) bits (R2).
    4. per region (R3) Lloyd-Max on pooled u = (R x)_i / sigma_i (R4);
       tables scaled back by sigma_i (R5).
    5. QJL matrix S = gauss[:m, :d_eff], m = qjl_bits * d_eff (R6).
    """
    x = np.asarray(samples, dtype=np.float64)
    if normalize:
        x, _ = _unit_rows(x)
    n, d = x.shape
    lam, R = eigenbasis(second_moment(x))
    sigma = np.sqrt(lam)
    pr = participation_ratio(lam)
    d_eff = effective_dim_cumvar(lam, deff_cumvar) if deff_cumvar > 0 else effective_dim(lam)
    kappa = spectral_gap(lam, d_eff)
    widths = water_fill(lam, int(round(avg_bits * d)), max_bits)
    y = x @ R.T                                           # rotated samples
    thresholds = [np.zeros(0) for _ in range(d)]
    centroids = [np.zeros(0) for _ in range(d)]
    books = {}
    for key, coords in sorted(regions(widths, d_eff).items()):
        pooled = [y[:, i] / sigma[i] for i in coords if sigma[i] > 0]
        u = np.concatenate(pooled) if pooled else np.zeros(0)
        c, t, it, conv = lloyd_max_samples(u, 2 ** key[1], lloyd_iters)
        books[key] = (c, t, it, conv, len(u))
        for i in coords:
            thresholds[i] = sigma[i] * t
            centroids[i] = sigma[i] * c
    m = int(qjl_bits) * d_eff if qjl_bits > 0 else 0
    if m > 0:
        S = np.asarray(gauss, dtype=np.float32)[:m, :d_eff].astype(np.float64)
    else:
        S = np.zeros((0, d_eff))
    W = record_words(widths, m, normalize)
    return Calibration(d, R, lam, sigma, pr, d_eff, kappa, widths, thresholds, centroids,
                       books, m, S, W, field_offsets(widths), int(widths.sum()), m > 0, normalize)


# --------------------------------------------------------------------------
# Compression
# --------------------------------------------------------------------------

@dataclasses.dataclass
class CompressResult:
    y: np.ndarray        # [T, d] rotated coordinates (of x / nu when normalised)
    codes: np.ndarray    # [T, d] int
    yhat: np.ndarray     # [T, d] centroid reconstruction (rotated space)
    z: np.ndarray        # [T, m] uint8 QJL bits
    gamma: np.ndarray    # [T] float16 residual norm
    sr: np.ndarray       # [T, m] S r (before the sign)
    rnorm: np.ndarray    # [T] ||r|| in float64
    nu: Optional[np.ndarray] = None   # [T] float16 vector norms (normalised variant)


def rotate(cal: Calibration, x: np.ndarray) -> np.ndarray:
    """y = R x for each row x (spectral rotation)."""
    return np.asarray(x, dtype=np.float64) @ cal.R.T


def quantize(cal: Calibration, y: np.ndarray):
    """Per-coordinate code = #{thresholds below y} (R7) and its centroid."""
    T, d = y.shape
    codes = np.zeros((T, d), dtype=np.int64)
    yhat = np.zeros((T, d))
    for i in range(d):
        if cal.widths[i] == 0:
            continue
        th = cal.thresholds[i]
        col = y[:, i]
        codes[:, i] = np.searchsorted(th, col, side="left")   # #{th < y}
        codes[np.isnan(col), i] = 0
        yhat[:, i] = cal.centroids[i][codes[:, i]]
    return codes, yhat


def compress(cal: Calibration, x: np.ndarray) -> CompressResult:
    """Rotate, quantise, and (keys) the selective QJL of the signal residual
    (normalised variant: of the unit vector x / nu, nu stored as a half)."""
    x = np.asarray(x, dtype=np.float64)
    nu16 = None
    if cal.normalized:
        x, nu = _unit_rows(x)
        nu16 = nu.astype(np.float16)
    y = rotate(cal, x)
    codes, yhat = quantize(cal, y)
    T = y.shape[0]
    if cal.m > 0:
        r = y[:, :cal.d_eff] - yhat[:, :cal.d_eff]
        rn = np.sqrt((r * r).sum(axis=1))
        sr = r @ cal.S.T
        z = (sr >= 0).astype(np.uint8)
        gamma = rn.astype(np.float16)
    else:
        rn = np.zeros(T)
        sr = np.zeros((T, 0))
        z = np.zeros((T, 0), dtype=np.uint8)
        gamma = np.zeros(T, dtype=np.float16)
    return CompressResult(y, codes, yhat, z, gamma, sr, rn, nu16)


def band_mask(cal: Calibration, y: np.ndarray, rel: float = 1e-4) -> np.ndarray:
    """[T, d] True where y_i lies within rel * sigma_i of one of its thresholds
    (the zone where several codes are acceptable)."""
    T, d = y.shape
    out = np.zeros((T, d), dtype=bool)
    for i in range(d):
        th = cal.thresholds[i]
        if len(th) == 0:
            continue
        j = np.clip(np.searchsorted(th, y[:, i]), 1, len(th))
        dist = np.minimum(np.abs(y[:, i] - th[j - 1]),
                          np.abs(y[:, i] - th[np.minimum(j, len(th) - 1)]))
        out[:, i] = dist <= rel * cal.sigma[i]
    return out


def qjl_band_mask(cal: Calibration, res: CompressResult, rel: float = 1e-3) -> np.ndarray:
    """[T, m] True where |(S r)_j| <= rel * ||S_j|| * ||r|| (sign not fixed)."""
    if cal.m == 0:
        return np.zeros((res.y.shape[0], 0), dtype=bool)
    sn = np.sqrt((cal.S ** 2).sum(axis=1))
    return np.abs(res.sr) <= rel * sn[None, :] * res.rnorm[:, None]


# --------------------------------------------------------------------------
# Read side
# --------------------------------------------------------------------------

def _centroid_values(cal: Calibration, codes: np.ndarray) -> np.ndarray:
    T, d = codes.shape
    yhat = np.zeros((T, d))
    for i in range(d):
        if cal.widths[i] > 0:
            yhat[:, i] = cal.centroids[i][codes[:, i]]
    return yhat


def _qjl_term(cal: Calibration, z: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """Rotated-space QJL correction on the signal dims:
    sqrt(pi/2)/m * gamma * S^T (2z - 1)  -> [T, d_eff]."""
    sgn = 2.0 * z.astype(np.float64) - 1.0
    return (math.sqrt(math.pi / 2) / cal.m) * gamma.astype(np.float64)[:, None] * (sgn @ cal.S)


def _nu_scale(cal: Calibration, nu) -> np.ndarray:
    """Per-token factor of the normalised variant (the stored half nu), else 1."""
    if not cal.normalized:
        return None
    return np.asarray(nu, dtype=np.float16).astype(np.float64)


def dequantize(cal: Calibration, codes: np.ndarray, z: np.ndarray, gamma: np.ndarray,
               nu=None) -> np.ndarray:
    """x~ = R^T ( yhat + pad_d( QJL correction ) )   (values: R^T yhat),
    times the stored norm nu in the normalised variant."""
    yh = _centroid_values(cal, codes)
    if cal.m > 0:
        yh[:, :cal.d_eff] += _qjl_term(cal, z, gamma)
    f = _nu_scale(cal, nu)
    if f is not None:
        yh *= f[:, None]
    return yh @ cal.R


def scores_plain(cal: Calibration, q: np.ndarray, codes, z, gamma, nu=None) -> np.ndarray:
    """Route (i): s = <q, x~_t> for queries q [G, d] -> [G, T]."""
    return np.asarray(q, np.float64) @ dequantize(cal, codes, z, gamma, nu).T


def scores_rotated(cal: Calibration, q: np.ndarray, codes, z, gamma, nu=None) -> np.ndarray:
    """Route (ii), the decode-time form: rotate the query once (q~ = R q), then
    s_t = sum_i q~_i C_i[code_ti] + sqrt(pi/2)/m * gamma_t * sum_j w_j (2 z_tj - 1)
    with w = S q~[:d_eff]; times nu_t in the normalised variant.  [G, T]."""
    qt = np.asarray(q, np.float64) @ cal.R.T
    s = qt @ _centroid_values(cal, codes).T
    if cal.m > 0:
        w = qt[:, :cal.d_eff] @ cal.S.T                   # [G, m]
        sgn = 2.0 * z.astype(np.float64) - 1.0            # [T, m]
        s += (math.sqrt(math.pi / 2) / cal.m) * (w @ sgn.T) * gamma.astype(np.float64)[None, :]
    f = _nu_scale(cal, nu)
    if f is not None:
        s *= f[None, :]
    return s


def softmax(s: np.ndarray, scale: float) -> np.ndarray:
    """Row softmax of scale * s, max-subtracted."""
    a = np.asarray(s, np.float64) * scale
    a = a - a.max(axis=-1, keepdims=True)
    e = np.exp(a)
    return e / e.sum(axis=-1, keepdims=True)


def attend(cal_v: Calibration, scores: np.ndarray, scale: float, codes_v, nu_v=None) -> np.ndarray:
    """o = sum_t softmax(scale * s)_t x~v_t, computed as R_v^T sum_t p_t yhat_v,t
    (values carry no QJL term; normalised variant: p_t nu_t).  scores [G, T] -> [G, d]."""
    p = softmax(scores, scale)
    f = _nu_scale(cal_v, nu_v)
    if f is not None:
        p = p * f[None, :]
    return (p @ _centroid_values(cal_v, codes_v)) @ cal_v.R
