"""Pins of the CPU oracle against things other than itself: closed forms,
printed values, brute force and invariants.  CPU only (not marked gpu)."""
import dataclasses
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- rotation

def test_eigenbasis_recovers_planted_basis():
    """C = Q diag(l) Q^T with a known Q and distinct l: eigenvalues come back in
    descending order and R's ROWS are Q's columns (up to the sign rule), so
    y = R x maps Q e_k to e_k."""
    d = 16
    q = wl.random_orthogonal(_rng(1), d)
    lam = np.sort(_rng(2).uniform(0.5, 20.0, d))[::-1]
    c = (q * lam[None, :]) @ q.T
    got_lam, R = oracle.eigenbasis(c)
    np.testing.assert_allclose(got_lam, lam, rtol=1e-12)
    for k in range(d):
        s = np.sign(R[k] @ q[:, k])
        np.testing.assert_allclose(R[k], s * q[:, k], atol=1e-12)
        y = R @ q[:, k]
        np.testing.assert_allclose(np.abs(y), np.eye(d)[k], atol=1e-12)


def test_rotation_invariants_on_sampled_data():
    cfg = wl.CONFIGS["llama8b"]
    x = wl.calibration_set(cfg, 0, 3, "k")
    c = oracle.second_moment(x)
    lam, R = oracle.eigenbasis(c)
    d = len(lam)
    np.testing.assert_allclose(R @ R.T, np.eye(d), atol=1e-12)
    cn = np.linalg.norm(c, 2)
    for i in range(d):
        assert np.linalg.norm(c @ R[i] - lam[i] * R[i]) <= 1e-10 * cn
    assert abs(lam.sum() - np.trace(c)) <= 1e-12 * abs(np.trace(c))
    assert np.all(np.diff(lam) <= 0)
    for i in range(d):                                  # sign rule
        j = np.argmax(np.abs(R[i]))
        assert R[i, j] > 0


def test_second_moment_is_uncentered():
    """A mean offset must show up in C (the fixture's X^T X / n, no centering)."""
    x = np.ones((10, 3)) * 2.0
    np.testing.assert_allclose(oracle.second_moment(x), np.full((3, 3), 4.0))


# ---------------------------------------------------------------- d_eff, kappa

def test_deff_population_special_cases():
    assert oracle.effective_dim(np.ones(32)) == 32            # flat -> d
    assert oracle.effective_dim(np.r_[np.ones(4), np.zeros(28)]) == 4   # isotropic rank 4
    assert oracle.effective_dim(np.r_[1.0, np.zeros(31)]) == 1
    sg = wl.population_spectrum("sharp_gap", 32)
    assert abs(oracle.participation_ratio(sg) - (8 * 50 + 24) ** 2 / (8 * 2500 + 24)) < 1e-12
    assert oracle.effective_dim(sg) == 9
    assert oracle.effective_dim(wl.population_spectrum("keys128", 128)) == 3
    assert abs(oracle.participation_ratio(wl.population_spectrum("values128", 128)) - 48) < 1e-6
    assert oracle.effective_dim(wl.population_spectrum("keys256", 256)) == 9
    assert abs(oracle.participation_ratio(wl.population_spectrum("values256", 256)) - 100) < 1e-6


def test_pr_rounds_half_to_even():
    """lambda = (12, 2, 2, 2, 2): sum 20, sum of squares 160, PR = 2.5 exactly;
    Python's round gives 2 (half to even), as the conftest fixture's int(round(.))."""
    lam = np.array([12.0, 2.0, 2.0, 2.0, 2.0])
    assert oracle.participation_ratio(lam) == 2.5
    assert oracle.effective_dim(lam) == 2


def test_spectral_gap():
    lam = np.array([10.0, 9.0, 1.0, 0.5])
    assert oracle.spectral_gap(lam, 2) == 9.0
    assert math.isinf(oracle.spectral_gap(lam, 4))
    assert math.isinf(oracle.spectral_gap(np.array([1.0, 0.0]), 1))


def test_deff_sampled_flat_matches_wishart_mean():
    """Sample PR of n white vectors in d dims averages d n / (n + d + 1)
    (second moment of a Wishart matrix); the fixture size n=256, d=32 gives 28.35."""
    prs = []
    for s in range(40):
        x = wl.flat_data(256, 32, seed=1000 + s)
        prs.append(oracle.participation_ratio(oracle.eigenbasis(oracle.second_moment(x))[0]))
    assert abs(np.mean(prs) - 32 * 256 / (256 + 33)) < 0.25


def test_deff_isotropic_rank4_is_4_and_fixture_rank4_bounded():
    for s in range(10):
        x = wl.rank_k_isotropic(256, 32, 4, seed=s)
        cal = oracle.calibrate(x, 3.0, 0, None)
        assert cal.d_eff == 4
        x2 = wl.rank4_fixture(256, 32, seed=s)
        pr = oracle.participation_ratio(oracle.eigenbasis(oracle.second_moment(x2))[0])
        assert 1.0 <= pr <= 4.0 + 1e-9


def test_pr_never_exceeds_rank():
    for k in (1, 2, 5, 9):
        x = _rng(k).standard_normal((50, k)) @ _rng(k + 100).standard_normal((k, 20))
        lam = oracle.eigenbasis(oracle.second_moment(x))[0]
        assert oracle.participation_ratio(lam) <= k + 1e-9


# ---------------------------------------------------------------- water-filling

def _brute_force_alloc(lam, B, bmax):
    best, arg = None, None
    for b in itertools.product(range(bmax + 1), repeat=len(lam)):
        if sum(b) != B:
            continue
        v = float(np.sum(lam * 4.0 ** (-np.array(b, float))))
        if best is None or v < best - 1e-15:
            best, arg = v, b
    return best, arg


@pytest.mark.parametrize("seed", range(12))
def test_water_fill_is_brute_force_optimal(seed):
    r = _rng(seed)
    d = int(r.integers(2, 6))
    lam = np.sort(r.lognormal(0, 2, d))[::-1]
    bmax = int(r.integers(2, 5))
    B = int(r.integers(1, min(12, d * bmax) + 1))
    b = oracle.water_fill(lam, B, bmax)
    assert b.sum() == B and b.max() <= bmax
    best, _ = _brute_force_alloc(lam, B, bmax)
    assert float(np.sum(lam * 4.0 ** (-b.astype(float)))) <= best * (1 + 1e-12)


def test_water_fill_monotone_and_near_real_valued_solution():
    lam = wl.population_spectrum("keys128", 128) * 217.0
    b = oracle.water_fill(lam, 384, 8)
    assert b.sum() == 384
    assert np.all(np.diff(b) <= 0)
    # real-valued reverse water-filling without the cap on the uncapped coordinates
    free = b < 8
    budget = 384 - 8 * (~free).sum()
    lo, hi = 1e-12, lam.max()
    for _ in range(200):
        th = math.sqrt(lo * hi)
        tot = np.sum(np.maximum(0, 0.5 * np.log2(lam[free] / th)))
        lo, hi = (th, hi) if tot > budget else (lo, th)
    real = np.maximum(0, 0.5 * np.log2(lam[free] / th))
    assert np.all(np.abs(b[free] - real) <= 1.0 + 1e-9)


def test_water_fill_caps_and_ties():
    b = oracle.water_fill(np.array([1.0, 1.0, 1.0]), 4, 8)
    assert list(b) == [2, 1, 1]                # ties to the lower index
    b = oracle.water_fill(np.array([5.0, 1.0]), 20, 3)
    assert list(b) == [3, 3]                   # capacity reached, rest unused


# ---------------------------------------------------------------- Lloyd-Max

def test_gaussian_lloyd_max_matches_max_1960():
    g = _gold("gaussian_lloyd_max.json")
    for bits in (1, 2, 3):
        c, t = oracle.lloyd_max_gaussian(bits)
        half = c[len(c) // 2:]
        np.testing.assert_allclose(half, g["levels"][str(bits)], atol=6e-5)
        np.testing.assert_allclose(t[len(t) // 2:], g["thresholds"][str(bits)], atol=6e-5)
        np.testing.assert_allclose(c, -c[::-1], atol=1e-12)
    assert abs(oracle.lloyd_max_gaussian(1)[0][1] - math.sqrt(2 / math.pi)) < 1e-12
    for bits in (1, 2, 3, 4):
        c, t = oracle.lloyd_max_gaussian(bits)
        assert abs(oracle.gaussian_distortion(c, t) - g["distortion"][str(bits)]) < 6e-5 * max(1, 10 ** (bits - 2))


def test_gaussian_distortion_closed_form_against_sampling():
    c, t = oracle.lloyd_max_gaussian(2)
    z = _rng(3).standard_normal(400000)
    q = c[np.searchsorted(t, z)]
    emp = np.mean((z - q) ** 2)
    assert abs(emp - oracle.gaussian_distortion(c, t)) < 4 * np.std((z - q) ** 2) / math.sqrt(len(z))


def test_lloyd_samples_conditions_by_direct_masks():
    u = _rng(5).standard_normal(5000) * 1.7 + 0.3
    for L in (2, 4, 8, 32):
        c, t, it, conv = oracle.lloyd_max_samples(u, L, 200)
        assert np.all(np.diff(c) > 0)
        np.testing.assert_array_equal(t, (c[:-1] + c[1:]) / 2)
        if conv:
            edges = np.r_[-np.inf, t, np.inf]
            for j in range(L):
                cell = u[(u > edges[j]) & (u <= edges[j + 1])]
                if len(cell):
                    assert abs(cell.mean() - c[j]) <= 1e-12 * max(1.0, abs(c[j]))


def test_lloyd_samples_converges_to_gaussian_constants():
    u = _rng(6).standard_normal(400000)
    for bits in (1, 2, 3):
        c, t, it, conv = oracle.lloyd_max_samples(u, 2 ** bits, 2000)
        cg, _ = oracle.lloyd_max_gaussian(bits)
        np.testing.assert_allclose(c, cg, atol=0.02)


def test_lloyd_samples_degenerate_inputs():
    c, t, it, conv = oracle.lloyd_max_samples(np.zeros(0), 4)
    assert np.all(c == 0)
    c, t, it, conv = oracle.lloyd_max_samples(np.array([1.0, 2.0]), 8)   # fewer samples than levels
    assert np.all(np.diff(c) >= 0) and conv


# ---------------------------------------------------------------- quantiser

def test_quantize_equals_brute_force_nearest_centroid():
    cfg = wl.CONFIGS["tiny"]
    x = wl.kv_block(cfg, 0, 0, "k", 256, "data")
    cal = oracle.calibrate(x, 3.0, 1, wl.qjl_gaussian(cfg, 0, 0))
    y = oracle.rotate(cal, x)
    codes, yhat = oracle.quantize(cal, y)
    band = oracle.band_mask(cal, y, 1e-9)
    for i in range(cal.head_dim):
        if cal.widths[i] == 0:
            assert np.all(codes[:, i] == 0) and np.all(yhat[:, i] == 0)
            continue
        cen = cal.centroids[i]
        nearest = np.argmin(np.abs(y[:, i][:, None] - cen[None, :]), axis=1)
        ok = ~band[:, i]
        np.testing.assert_array_equal(codes[ok, i], nearest[ok])


def test_quantize_tie_and_nan_rules():
    cal = oracle.calibrate(wl.flat_data(300, 4), 2.0, 0, None)
    th = cal.thresholds[0]
    y = np.zeros((3, 4))
    y[0, 0] = th[1]            # exactly on a threshold -> lower cell
    y[1, 0] = np.nan
    y[2, 0] = np.nextafter(th[1], np.inf)
    codes, _ = oracle.quantize(cal, y)
    assert codes[0, 0] == 1 and codes[1, 0] == 0 and codes[2, 0] == 2


# ---------------------------------------------------------------- QJL

def test_qjl_estimator_unbiased_with_closed_form_variance():
    """Over many independent Gaussian sketches S, the oracle's QJL score term
    averages <q~_s, r> with variance ((pi/2)|q~_s|^2 |r|^2 - <q~_s, r>^2) / m."""
    cfg = wl.CONFIGS["tiny"]
    x = wl.kv_block(cfg, 0, 1, "k", 256, "data")
    base = oracle.calibrate(x, 3.0, 1, wl.qjl_gaussian(cfg, 0, 1))
    xv = x[:1]
    q = _rng(8).standard_normal((1, cfg.head_dim))
    res = oracle.compress(base, xv)
    qt = (q @ base.R.T)[0]
    r = res.y[0, :base.d_eff] - res.yhat[0, :base.d_eff]
    truth = float(qt[:base.d_eff] @ r)
    mse_part = float(qt @ res.yhat[0])
    vals = []
    rng = _rng(9)
    for _ in range(6000):
        cal = dataclasses.replace(base, S=rng.standard_normal((base.m, base.d_eff))
                                  .astype(np.float32).astype(np.float64))
        rr = oracle.compress(cal, xv)
        s = oracle.scores_rotated(cal, q, rr.codes, rr.z, rr.gamma)[0, 0]
        vals.append(s - mse_part)
    vals = np.array(vals)
    # gamma is stored as a half: allow its relative rounding in the mean
    g = float(res.gamma[0]) / float(np.linalg.norm(r))
    var = ((math.pi / 2) * (qt[:base.d_eff] @ qt[:base.d_eff]) * (r @ r) * g * g - (truth * g) ** 2) / base.m
    se = math.sqrt(var / len(vals))
    assert abs(vals.mean() - truth * g) < 4.5 * se
    assert abs(vals.var() / var - 1) < 0.1


# ---------------------------------------------------------------- scores / attend

def _small_setup(cfg_name="llama8b", head=0, T=300):
    cfg = wl.CONFIGS[cfg_name]
    ck = oracle.calibrate(wl.calibration_set(cfg, 0, head, "k"), cfg.budgets[0], cfg.qjl_bits,
                          wl.qjl_gaussian(cfg, 0, head))
    cv = oracle.calibrate(wl.calibration_set(cfg, 0, head, "v"), cfg.budgets[0], 0, None)
    xk = wl.kv_block(cfg, 0, head, "k", T, "data")
    xv = wl.kv_block(cfg, 0, head, "v", T, "data")
    return cfg, ck, cv, xk, xv


def test_score_routes_agree():
    cfg, ck, cv, xk, xv = _small_setup()
    r = oracle.compress(ck, xk)
    q = wl.queries(cfg, 1, 4)[0]
    s1 = oracle.scores_plain(ck, q, r.codes, r.z, r.gamma)
    s2 = oracle.scores_rotated(ck, q, r.codes, r.z, r.gamma)
    assert np.max(np.abs(s1 - s2)) <= 1e-12 * np.max(np.abs(s1))


def test_scores_without_qjl_equal_rotated_query_dot_centroids():
    cfg, ck, cv, xk, xv = _small_setup()
    r = oracle.compress(ck, xk)
    q = wl.queries(cfg, 1, 2)[0]
    zero_g = np.zeros_like(r.gamma)
    s = oracle.scores_rotated(ck, q, r.codes, r.z, zero_g)
    np.testing.assert_allclose(s, (q @ ck.R.T) @ r.yhat.T, rtol=1e-12, atol=1e-9)


def test_attend_invariants():
    cfg, ck, cv, xk, xv = _small_setup()
    rk = oracle.compress(ck, xk)
    rv = oracle.compress(cv, xv)
    q = wl.queries(cfg, 1, 4)[0]
    s = oracle.scores_rotated(ck, q, rk.codes, rk.z, rk.gamma)
    p = oracle.softmax(s, 1 / math.sqrt(cfg.head_dim))
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    xt_v = oracle.dequantize(cv, rv.codes, rv.z, rv.gamma)
    o = oracle.attend(cv, s, 1 / math.sqrt(cfg.head_dim), rv.codes)
    np.testing.assert_allclose(o, p @ xt_v, rtol=1e-11, atol=1e-13)
    s2 = np.zeros_like(s)
    s2[:, 17] = 1e4
    o2 = oracle.attend(cv, s2, 1.0, rv.codes)
    np.testing.assert_allclose(o2, np.repeat(xt_v[17:18], len(s2), 0), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- record layout

def _brute_pack_token(widths, m, codes, z, gamma_bits, W):
    widths, W, m = [int(b) for b in widths], int(W), int(m)
    acc, pos = 0, 0
    for b, c in zip(widths, codes):
        for k in range(b):
            if (int(c) >> k) & 1:
                acc |= 1 << (pos + k)
        pos += b
    for j in range(m):
        if z[j]:
            acc |= 1 << (pos + j)
    if m:
        acc |= int(gamma_bits) << (32 * W - 16)
    return [(acc >> (32 * w)) & 0xFFFFFFFF for w in range(W)]


def test_record_hand_worked_example():
    widths, codes, z = [3, 0, 5, 2, 8, 1], [5, 0, 17, 2, 200, 1], [1, 0]
    # LSB-first: 5@0 | 17@3 | 2@8 | 200@10 | 1@18 | z0=1@19 -> 0x000F228D ; 37 bits -> W = 2
    # gamma 1.5 = half 0x3E00 in the top 16 bits of word 1 -> 0x3E000000
    W = oracle.record_words(widths, 2)
    assert W == 2
    pk = oracle.pack(widths, 2, np.array([codes]), np.array([z], np.uint8), np.array([1.5], np.float16))
    assert pk.shape == (64 * W,)
    assert pk[0] == 0x000F228D and pk[64] == 0x3E000000
    assert np.all(pk[1:64] == 0) and np.all(pk[65:] == 0)


def test_pack_matches_bitwise_construction_and_roundtrips():
    r = _rng(11)
    for trial in range(6):
        d = int(r.integers(1, 40))
        widths = r.integers(0, 9, d)
        m = int(r.integers(0, 12))
        T = int(r.integers(1, 150))
        codes = np.stack([r.integers(0, 2 ** b, T) if b else np.zeros(T, int) for b in widths], 1)
        z = r.integers(0, 2, (T, m)).astype(np.uint8)
        gamma = r.uniform(0, 300, T).astype(np.float16)
        W = int(oracle.record_words(widths, m))
        pk = oracle.pack(widths, m, codes, z, gamma)
        assert len(pk) == -(-T // 64) * 64 * W
        for t in (0, T // 2, T - 1):
            want = _brute_pack_token(list(widths), m, codes[t], z[t], gamma.view(np.uint16)[t], W)
            got = [int(pk[((t // 64) * W + w) * 64 + t % 64]) for w in range(W)]
            assert got == want
        pad = -(-T // 64) * 64
        for t in range(T, pad):
            assert all(pk[((t // 64) * W + w) * 64 + t % 64] == 0 for w in range(W))
        c2, z2, g2 = oracle.unpack(widths, m, pk, T)
        np.testing.assert_array_equal(c2, codes)
        np.testing.assert_array_equal(z2, z)
        if m:
            np.testing.assert_array_equal(g2.view(np.uint16), gamma.view(np.uint16))


def test_record_sizes_of_the_configs():
    cfg, ck, cv, _, _ = _small_setup()
    assert ck.widths.sum() == 384 and cv.widths.sum() == 384
    assert ck.W == -(-(384 + ck.m + 16) // 32) and cv.W == 12


# ---------------------------------------------------------------- baseline + quality

def test_turboquant_distortion_reproduces_printed_table():
    g = _gold("tq_distortion_scoslab.json")
    d = g["d"]
    w = _rng(12).standard_normal((3000, d))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    for bits, emp in zip(g["bits"], g["empirical"]):
        e = ((w - oracle.tq_mse_unit(w, bits)) ** 2).sum(axis=1)
        # printed to 3 decimals; sampling error of the mean is tiny at 3000 x 1536
        assert abs(e.mean() - emp) <= 0.0051 + 3 * e.std() / math.sqrt(len(e))


def test_spectralquant_beats_turboquant_style_cosine_on_same_inputs():
    cfg, ck, cv, xk, xv = _small_setup(T=1000)
    rk = oracle.compress(ck, xk)
    sq = oracle.cosine(xk, oracle.dequantize(ck, rk.codes, rk.z, rk.gamma)).mean()
    rot = wl.tq_rotation(cfg, 0, 0)
    tq = oracle.cosine(xk, oracle.tq_prod_keys(xk, rot, wl.tq_qjl(cfg, 0, 0), 3)).mean()
    assert sq > tq
    assert 0.88 < tq < 0.96          # Gaussian expectation ~0.92 for 2 bits + QJL
    rv = oracle.compress(cv, xv)
    sqv = oracle.cosine(xv, oracle.dequantize(cv, rv.codes, rv.z, rv.gamma)).mean()
    tqv = oracle.cosine(xv, oracle.tq_mse_values(xv, rot, 3)).mean()
    assert sqv > tqv


def test_headline_compression_ratios_reconstruct():
    g = _gold("headline_compression.json")
    sq = oracle.compression_ratio(2.5 * 128 + 24, 128)
    tq = oracle.compression_ratio(3 * 128 + 24, 128)
    assert round(sq, 2) == g["spectralquant"] and round(tq, 2) == g["turboquant"]
    assert round(100 * (sq / tq - 1), 1) == g["improvement_pct"]


def test_sq_distortion_near_gaussian_prediction_with_ample_calibration():
    """With many calibration samples, each coordinate's relative distortion
    approaches the Gaussian Lloyd-Max D(b_i) (Max 1960), so
    E|x - x~|^2 ~= sum_i lambda_i D(b_i) for Gaussian data (values: no QJL)."""
    cfg = wl.CONFIGS["llama8b"]
    a = wl.head_covariance_factor(cfg, 0, 0, "v")
    rng = _rng(13)
    xc = rng.standard_normal((20000, 128)) @ a
    xd = rng.standard_normal((4000, 128)) @ a
    cal = oracle.calibrate(xc, 3.0, 0, None, lloyd_iters=2000)
    r = oracle.compress(cal, xd)
    err = ((r.y - r.yhat) ** 2).sum(axis=1).mean()
    D = {b: oracle.gaussian_distortion(*oracle.lloyd_max_gaussian(b)) if b else 1.0 for b in range(9)}
    pred = sum(cal.lam[i] * D[int(cal.widths[i])] for i in range(128))
    assert abs(err / pred - 1) < 0.05
