"""Pins of the calibration variants in the oracle: d_eff by cumulative
variance and the calibration-stability coefficient of variation (README
"Repository Structure" deff sweep and paper-section table).  Each expected
value comes from a closed form or a planted spectrum, not from the oracle."""
import math

import numpy as np
import pytest

import oracle


def test_cumvar_flat_spectrum_is_ceil_fraction_times_d():
    for d in (4, 32, 128):
        lam = np.ones(d)
        for f in (0.3, 0.55, 0.9, 0.97):
            want = math.ceil(f * d - 1e-12)
            assert oracle.effective_dim_cumvar(lam, f) == want, (d, f)


def test_cumvar_exact_boundary_counts_as_reached():
    # partial sums hit the threshold exactly: 2 of 4 equal eigenvalues hold 1/2
    assert oracle.effective_dim_cumvar(np.ones(4), 0.5) == 2
    assert oracle.effective_dim_cumvar(np.array([4.0, 2.0, 1.0, 1.0]), 0.75) == 2


def test_cumvar_geometric_closed_form():
    # lambda_i = r^i: sum_{i<k} / sum_{i<d} = (1 - r^k) / (1 - r^d) >= f
    # <=> k >= log(1 - f (1 - r^d)) / log r
    for r, d, f in ((0.8, 64, 0.9), (0.8, 64, 0.95), (0.95, 128, 0.9), (0.5, 32, 0.99)):
        lam = r ** np.arange(d, dtype=np.float64)
        k_real = math.log(1 - f * (1 - r ** d)) / math.log(r)
        assert abs(k_real - round(k_real)) > 1e-6
        assert oracle.effective_dim_cumvar(lam, f) == math.ceil(k_real), (r, d, f)


def test_cumvar_full_fraction_is_the_rank_and_monotone():
    lam = np.array([3.0, 2.0, 1.0, 0.0, 0.0])
    assert oracle.effective_dim_cumvar(lam, 1.0) == 3
    lam = np.exp(-np.arange(64) / 5.0)
    ks = [oracle.effective_dim_cumvar(lam, f) for f in np.linspace(0.05, 1.0, 40)]
    assert all(a <= b for a, b in zip(ks, ks[1:]))
    with pytest.raises(ValueError):
        oracle.effective_dim_cumvar(lam, 0.0)


def _planted(lam, rng):
    """Samples whose second moment is exactly Q diag(lam) Q^T: row i of the
    unrotated set is sqrt(d lam_i) e_i."""
    d = len(lam)
    q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    x = np.diag(np.sqrt(d * lam))
    return x @ q.T


def test_calibrate_uses_the_cumvar_rule_for_d_eff_and_qjl_rows():
    rng = np.random.default_rng(3)
    d = 32
    lam = 0.7 ** np.arange(d)
    x = _planted(lam, rng)
    g = rng.standard_normal((d, d)).astype(np.float32)
    for f in (0.8, 0.9, 0.99):
        k = math.ceil(math.log(1 - f * (1 - 0.7 ** d)) / math.log(0.7))
        cal = oracle.calibrate(x, 3.0, 1, g, deff_cumvar=f)
        assert cal.d_eff == k
        assert cal.m == k and cal.S.shape == (k, k)
        assert cal.kappa == pytest.approx(1 / 0.7, rel=1e-9)
    # the default rule is still the rounded participation ratio
    pr = lam.sum() ** 2 / (lam ** 2).sum()
    assert oracle.calibrate(x, 3.0, 1, g).d_eff == round(pr)


def test_stability_cv_of_two_planted_spectra():
    # split A: e_0..e_3 twice each (isotropic rank 4, PR = 4); split B:
    # e_0..e_7 once (PR = 8); CV of {4, 8} = 2 / 6
    d = 16
    eye = np.eye(d)
    a = np.concatenate([eye[:4], eye[:4]]) * 2.5
    b = eye[:8] * 0.3
    st = oracle.calibration_stability(np.concatenate([a, b, eye[:1]]), 2)  # remainder dropped
    assert st["samples_per_split"] == 8
    np.testing.assert_allclose(st["pr"], [4.0, 8.0], rtol=1e-12)
    np.testing.assert_array_equal(st["d_eff"], [4, 8])
    assert st["pr_cv"] == pytest.approx(1 / 3, rel=1e-12)
    assert st["deff_cv"] == pytest.approx(1 / 3, rel=1e-12)


def test_stability_cv_is_zero_for_identical_and_rescaled_splits():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 16)) * np.linspace(2, 0.1, 16)
    st = oracle.calibration_stability(np.concatenate([x, x, x]), 3)
    assert st["pr_cv"] == 0.0 and st["deff_cv"] == 0.0
    st = oracle.calibration_stability(np.concatenate([x, 4.0 * x]), 2)
    assert st["pr_cv"] < 1e-13
    st = oracle.calibration_stability(np.concatenate([x, 4.0 * x]), 2, normalize=True)
    assert st["pr_cv"] < 1e-13
    assert oracle.coefficient_of_variation([1.0, 3.0]) == 0.5
