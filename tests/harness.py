"""Shared test machinery: build matching calibrations on both sides, compare
GPU outputs with the oracle under the acceptance rules.

Acceptance (the SpectralQuant build's parity bar):
  * codes bit-exact wherever the oracle's rotated coordinate is farther than
    1e-4 * sigma_i from every threshold; inside that band only +-1 flips;
  * QJL bits exact unless |(S r)_j| <= 1e-3 ||S_j|| ||r|| or a signal code flipped;
  * gamma within one half-precision ulp plus the rotation's forward error bound
    sqrt(d_eff) (d + 1) 2^-24 |x| (any value when a signal code flipped);
  * dequantised vectors, scores and attention outputs within 1e-3 relative with a
    floor: |gpu - ref| <= 1e-3 * (|ref| + floor).
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import workloads as wl

BAND = 1e-4
QJL_BAND = 1e-3
RTOL = 1e-3

# A head_dim-64 shape, not one of the pages' five workloads: only here do the
# kernels' 64-wide instances run (the register compress kernel at d = 64, one
# 64-coordinate attend block, the fused decode with NP = 1).  The spectra are
# the Llama-shaped families evaluated at d = 64; 2 layers x 4 KV heads, 16
# query heads (groups of 4), bf16 data, 512-token calibration sets.
HD64 = wl.Config("hd64", 5, 64, 2, 4, 16, (700,), 1, "bf16", 512, (3.0,), 1,
                 "keys128", "values128", 170.0, 3.0)
wl.CONFIGS.setdefault("hd64", HD64)


def calib_inputs(cfg, heads, which, seed=wl.DEFAULT_SEED, n_tokens=None):
    """heads: list of (layer, kv_head).  Returns (samples [H][n][d], gauss or None)."""
    X = np.stack([wl.calibration_set(cfg, l, h, which, seed, n_tokens) for l, h in heads])
    if which == "k" and cfg.qjl_bits > 0:
        G = np.stack([wl.qjl_gaussian(cfg, l, h, "k", seed) for l, h in heads])
    else:
        G = None
    return X.astype(np.float32), G


def calibrate_both(sq, cfg, heads, which, budget, seed=wl.DEFAULT_SEED, n_tokens=None):
    """Library calibration (handle) and oracle calibrations of the same heads;
    asserts the integer parts agree exactly."""
    X, G = calib_inputs(cfg, heads, which, seed, n_tokens)
    qb = cfg.qjl_bits if which == "k" else 0
    cal = sq.sq_calibrate(X, budget, qb, G)
    ors = []
    for k in range(len(heads)):
        oc = oracle.calibrate(X[k], budget, qb, G[k] if G is not None else None)
        inf = cal.info(k)
        ex = cal.export(k)
        assert inf.d_eff == oc.d_eff and inf.m == oc.m and inf.record_words == oc.W
        assert np.array_equal(ex["widths"], oc.widths)
        ors.append(oc)
    return cal, ors


def data_block(cfg, heads, which, T, seed=wl.DEFAULT_SEED):
    return np.stack([wl.kv_block(cfg, l, h, which, T, "data", seed) for l, h in heads])


def words_of(packed_slot: np.ndarray, W: int, T: int) -> np.ndarray:
    """[T, W] record words of one head's slot."""
    Tp = -(-T // 64) * 64
    return (packed_slot[:Tp * W].reshape(Tp // 64, W, 64).transpose(0, 2, 1)
            .reshape(Tp, W)[:T])


def compare_compress(oc, gpu_slot: np.ndarray, x: np.ndarray, T: int):
    """Check one head's GPU records against the oracle.  Returns a dict of
    counts; raises AssertionError on a violation."""
    res = oracle.compress(oc, x)
    band = oracle.band_mask(oc, res.y, BAND)
    qband = oracle.qjl_band_mask(oc, res, QJL_BAND)
    norm = bool(getattr(oc, "normalized", False))
    ref = oracle.pack(oc.widths, oc.m, res.codes, res.z, res.gamma, res.nu if norm else None)
    W = oc.W
    gw = words_of(gpu_slot, W, T).astype(np.uint64)
    rw = words_of(ref, W, T).astype(np.uint64)
    Tp = -(-T // 64) * 64
    # pad tokens must be zero
    pad = (gpu_slot[:Tp * W].reshape(Tp // 64, W, 64).transpose(0, 2, 1).reshape(Tp, W)[T:])
    assert np.all(pad == 0), "pad tokens not zero"
    if norm:
        gc, gz, gg, gn = oracle.unpack(oc.widths, oc.m, gpu_slot, T, norm=True)
    else:
        gc, gz, gg = oracle.unpack(oc.widths, oc.m, gpu_slot, T)
    diff = gc != res.codes
    assert not np.any(diff & ~band), f"{int((diff & ~band).sum())} code mismatches outside the band"
    assert np.all(np.abs(gc - res.codes)[diff] <= 1), "in-band flip larger than one code"
    n_flip = int(diff.sum())
    tok_flip = diff.any(axis=1)
    sig_flip = diff[:, :oc.d_eff].any(axis=1) if oc.m > 0 else np.zeros(T, bool)
    out = dict(tokens=T, coords=int(T * oc.head_dim), band=int(band.sum()), flips=n_flip,
               flip_tokens=int(tok_flip.sum()))
    if oc.m > 0:
        zd = gz != res.z
        bad = zd & ~qband & ~sig_flip[:, None]
        assert not np.any(bad), f"{int(bad.sum())} QJL bit mismatches outside the band"
        gu = gg.view(np.uint16).astype(np.int64)
        ru = res.gamma.view(np.uint16).astype(np.int64)
        # gamma = |r| inherits the rotation's absolute rounding error: each y_i
        # of an fp32 dot product of d exact products is within (d + 1) u |x|
        # (u = 2^-24; the +1 covers the bf16x3 representation of R), so |r|
        # moves by at most sqrt(d_eff) times that, then one fp16 rounding.
        g_ref = res.gamma.astype(np.float64)
        ulp16 = np.exp2(np.floor(np.log2(np.maximum(g_ref, 2.0 ** -14))) - 10)
        xn = np.linalg.norm(np.asarray(x, np.float64), axis=1)
        if norm:
            xn = np.ones_like(xn)  # r lives in the unit vector's space
        tol = ulp16 + math.sqrt(oc.d_eff) * (oc.head_dim + 2) * 2.0 ** -24 * xn
        gbad = (np.abs(gg.astype(np.float64) - g_ref) > tol) & ~sig_flip
        assert not np.any(gbad), f"{int(gbad.sum())} gamma values outside one ulp + rotation error"
        out["qjl_flips"] = int(zd.sum())
        out["gamma_ulp"] = int((gu != ru).sum())
    if norm:
        # the norm: |y| of the fp32 rotation against |x| in float64, one half
        # rounding each: within one half ulp plus the rotation's error
        n_ref = res.nu.astype(np.float64)
        ulpn = np.exp2(np.floor(np.log2(np.maximum(n_ref, 2.0 ** -14))) - 10)
        xn = np.linalg.norm(np.asarray(x, np.float64), axis=1)
        ntol = ulpn + (oc.head_dim + 2) * 2.0 ** -24 * xn
        nbad = np.abs(gn.astype(np.float64) - n_ref) > ntol
        nbad &= ~(np.isnan(n_ref) & np.isnan(gn.astype(np.float64)))
        assert not np.any(nbad), f"{int(nbad.sum())} vector norms outside one ulp + rotation error"
        out["nu_ulp"] = int((gn.view(np.uint16) != res.nu.view(np.uint16)).sum())
    # tokens with no excused difference must match bit for bit (gamma and the norm aside)
    clean = ~tok_flip
    mask = np.full(W, 0xFFFFFFFF, np.uint64)
    if oc.m > 0:
        clean &= ~(gz != res.z).any(axis=1)
        mask[W - 1] &= 0x0000FFFF
    if norm:
        mask[W - 1] &= 0xFFFF0000 if oc.m > 0 else 0x0000FFFF
    assert np.array_equal(gw[clean] & mask, rw[clean] & mask)
    return out, res


def assert_close_floor(gpu, ref, floor, what, rtol=RTOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    lim = rtol * (np.abs(ref) + floor)
    bad = err > lim
    assert not np.any(bad), (f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; "
                             f"worst err/lim {float(np.max(err / lim)):.3g}")
    return float(np.max(err / lim)) if err.size else 0.0


def score_floor(oc, q: np.ndarray, xt: np.ndarray) -> np.ndarray:
    """[G, T] floor ||q~|| ||x~_t|| / sqrt(d)."""
    qn = np.linalg.norm(q, axis=1)
    xn = np.linalg.norm(xt, axis=1)
    return qn[:, None] * xn[None, :] / math.sqrt(oc.head_dim)


def assert_calibration_matches(ex: dict, oc, pr_rtol=1e-10):
    """A libsq calibration export of one head against the oracle's calibration
    of the same samples: integer layout exact; eigenvalues to 1e-12 of the
    largest; eigenvectors of well-separated eigenvalues to 1e-9 (same sign
    rule); codebooks to 1e-6; the QJL rows are the same float32 draws."""
    inf = ex["info"]
    assert inf.d_eff == oc.d_eff and inf.m == oc.m and inf.record_words == oc.W
    assert inf.code_bits == int(oc.widths.sum())
    np.testing.assert_array_equal(ex["widths"], oc.widths)
    assert abs(inf.participation_ratio - oc.pr) <= pr_rtol * oc.pr
    if math.isinf(oc.kappa):
        assert math.isinf(inf.kappa)
    else:
        assert abs(inf.kappa - oc.kappa) <= 1e-8 * oc.kappa
    np.testing.assert_allclose(ex["eigenvalues"], oc.lam, rtol=0, atol=1e-12 * oc.lam[0])
    gaps = np.abs(np.diff(oc.lam))
    sep = np.minimum(np.r_[np.inf, gaps], np.r_[gaps, np.inf])
    good = sep > 1e-3 * oc.lam[0]
    np.testing.assert_allclose(ex["rotation"][good], oc.R[good], atol=1e-9)
    thr = np.concatenate([t for t in oc.thresholds if len(t)] or [np.zeros(0)])
    cen = np.concatenate([c for c in oc.centroids if len(c)] or [np.zeros(0)])
    np.testing.assert_allclose(ex["thresholds"], thr, rtol=1e-6, atol=1e-6 * oc.sigma[0])
    np.testing.assert_allclose(ex["centroids"], cen, rtol=1e-6, atol=1e-6 * oc.sigma[0])
    if oc.m:
        np.testing.assert_array_equal(ex["qjl"], oc.S.astype(np.float32))
