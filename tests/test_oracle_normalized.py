"""Pins of the oracle's normalised variant (per-vector norm stored, unit
vectors quantised) and of the TurboQuant-style scheme run through it (CPU
only): the generic pipeline under a TurboQuant calibration must reproduce the
separately pinned tq_prod_keys / tq_mse_values, codes must be the nearest
codebook level (brute force), the variant must be scale invariant, and the
record's norm field must sit where the layout says (brute-force bit writer)."""
import math

import numpy as np

import oracle
import workloads as wl


def _rng(s):
    return np.random.default_rng(s)


def _tq_cal(d, bits, keys, seed=3):
    r = _rng(seed)
    rot = wl.random_orthogonal(r, d)
    sk = r.standard_normal((d, d)).astype(np.float32)
    return oracle.tq_calibration(rot, sk, bits, keys), rot, sk


def test_tq_calibration_codes_are_nearest_levels():
    d = 64
    cal, rot, _ = _tq_cal(d, 3, keys=False)
    x = _rng(5).standard_normal((40, d)) * 7.0
    res = oracle.compress(cal, x)
    w = (x / np.linalg.norm(x, axis=1, keepdims=True)) @ rot.T
    lv = cal.centroids[0]
    want = np.argmin(np.abs(w[..., None] - lv[None, None, :]), axis=-1)
    np.testing.assert_array_equal(res.codes, want)
    np.testing.assert_allclose(res.nu.astype(np.float64), np.linalg.norm(x, axis=1), rtol=2.0 ** -11)


def test_tq_calibration_reproduces_turboquant_prod_and_mse():
    """Keys: (b-1)-bit stage + all-dims QJL; values: b-bit stage; the generic
    reconstruction equals tq_prod_keys / tq_mse_values except for the half
    rounding of the stored nu and gamma (relative 2^-11 each)."""
    d, bits = 128, 3
    x = _rng(7).standard_normal((50, d)) * np.linspace(4.0, 0.3, d)
    for keys in (True, False):
        cal, rot, sk = _tq_cal(d, bits, keys)
        res = oracle.compress(cal, x)
        got = oracle.dequantize(cal, res.codes, res.z, res.gamma, res.nu)
        want = (oracle.tq_prod_keys(x, rot, sk.astype(np.float64), bits) if keys
                else oracle.tq_mse_values(x, rot, bits))
        err = np.linalg.norm(got - want, axis=1)
        assert np.all(err <= 3 * 2.0 ** -11 * np.linalg.norm(want, axis=1) + 1e-12), err.max()
        assert cal.W == oracle.record_words(cal.widths, cal.m, True)


def test_normalized_variant_is_scale_invariant():
    cfg = wl.CONFIGS["llama8b"]
    X = wl.calibration_set(cfg, 0, 1, "k")
    cal = oracle.calibrate(X, 3.0, 1, wl.qjl_gaussian(cfg, 0, 1), normalize=True)
    assert cal.normalized and cal.W == oracle.record_words(cal.widths, cal.m, True)
    x = wl.kv_block(cfg, 0, 1, "k", 200, "data")
    r1 = oracle.compress(cal, x)
    r2 = oracle.compress(cal, 3.75 * x)
    np.testing.assert_array_equal(r1.codes, r2.codes)
    np.testing.assert_array_equal(r1.z, r2.z)
    x1 = oracle.dequantize(cal, r1.codes, r1.z, r1.gamma, r1.nu)
    x2 = oracle.dequantize(cal, r2.codes, r2.z, r2.gamma, r2.nu)
    np.testing.assert_allclose(x2, 3.75 * x1, rtol=2.0 ** -10, atol=1e-9 * np.abs(x2).max())
    # the two score routes agree and attend is the weighted sum of the reconstructions
    q = wl.queries(cfg, 1, 3)[0]
    s1 = oracle.scores_plain(cal, q, r1.codes, r1.z, r1.gamma, r1.nu)
    s2 = oracle.scores_rotated(cal, q, r1.codes, r1.z, r1.gamma, r1.nu)
    assert np.max(np.abs(s1 - s2)) <= 1e-12 * np.max(np.abs(s1))
    cv = oracle.calibrate(wl.calibration_set(cfg, 0, 1, "v"), 3.0, 0, None, normalize=True)
    xv = wl.kv_block(cfg, 0, 1, "v", 200, "data")
    rv = oracle.compress(cv, xv)
    o = oracle.attend(cv, s2, 1 / math.sqrt(128), rv.codes, rv.nu)
    p = oracle.softmax(s2, 1 / math.sqrt(128))
    np.testing.assert_allclose(o, p @ oracle.dequantize(cv, rv.codes, rv.z, rv.gamma, rv.nu),
                               rtol=1e-11, atol=1e-13)


def test_record_norm_field_position():
    """Normalised records: nu as a half in bits [32W-32, 32W-16) with QJL bits
    (gamma above it), in the top 16 bits without; brute-force bit writer."""
    r = _rng(9)
    for m in (0, 3, 9):
        widths = r.integers(0, 9, 20)
        T = 70
        codes = np.stack([r.integers(0, 2 ** b, T) if b else np.zeros(T, int) for b in widths], 1)
        z = r.integers(0, 2, (T, m)).astype(np.uint8)
        gamma = r.uniform(0, 30, T).astype(np.float16)
        nu = r.uniform(0, 300, T).astype(np.float16)
        W = oracle.record_words(widths, m, True)
        assert W == max(1, -(-(int(widths.sum()) + m + (16 if m else 0) + 16) // 32))
        pk = oracle.pack(widths, m, codes, z, gamma, nu)
        for t in (0, 33, T - 1):
            acc, pos = 0, 0
            for b, c in zip(widths, codes[t]):
                acc |= int(c) << pos
                pos += int(b)
            for j in range(m):
                acc |= int(z[t, j]) << (pos + j)
            if m:
                acc |= int(gamma.view(np.uint16)[t]) << (32 * W - 16)
            acc |= int(nu.view(np.uint16)[t]) << (32 * W - (32 if m else 16))
            got = [int(pk[((t // 64) * W + w) * 64 + t % 64]) for w in range(W)]
            assert got == [(acc >> (32 * w)) & 0xFFFFFFFF for w in range(W)]
        c2, z2, g2, n2 = oracle.unpack(widths, m, pk, T, norm=True)
        np.testing.assert_array_equal(c2, codes)
        np.testing.assert_array_equal(n2.view(np.uint16), nu.view(np.uint16))
