"""Host-side tests of libsq (no GPU): every declared symbol is exported, the
host calibration matches the oracle, save/load round-trips, the host unpacker
reads the oracle's record layout, and argument errors are reported."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import oracle
import workloads as wl
import compression_sq_compress_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "sq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sq_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = sq.lib()
    names = _declared_symbols()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(sq.EXPORTS)


def _heads(cfg, which, heads, n_tokens=None):
    X = np.stack([wl.calibration_set(cfg, l, h, which, n_tokens=n_tokens) for l, h in heads])
    G = (np.stack([wl.qjl_gaussian(cfg, l, h) for l, h in heads])
         if which == "k" and cfg.qjl_bits else None)
    return X.astype(np.float32), G


@pytest.mark.parametrize("cfgname,which,heads,budget", [
    ("tiny", "k", [(l, h) for l in range(3) for h in range(4)], 3.0),
    ("tiny", "v", [(l, h) for l in range(3) for h in range(4)], 3.0),
    ("llama8b", "k", [(0, h) for h in range(8)], 3.0),
    ("llama8b", "v", [(0, h) for h in range(8)], 3.0),
    ("qwen14b", "k", [(5, h) for h in range(4)], 2.5),
    ("qwen14b", "v", [(6, h) for h in range(4)], 3.5),
])
def test_calibration_matches_oracle(cfgname, which, heads, budget):
    cfg = wl.CONFIGS[cfgname]
    X, G = _heads(cfg, which, heads)
    qb = cfg.qjl_bits if which == "k" else 0
    cal = sq.sq_calibrate(X, budget, qb, G)
    assert cal.n_heads == len(heads)
    for k in range(len(heads)):
        oc = oracle.calibrate(X[k], budget, qb, G[k] if G is not None else None)
        ex = cal.export(k)
        inf = ex["info"]
        assert inf.d_eff == oc.d_eff and inf.m == oc.m and inf.record_words == oc.W
        assert inf.code_bits == int(oc.widths.sum())
        np.testing.assert_array_equal(ex["widths"], oc.widths)
        assert abs(inf.participation_ratio - oc.pr) <= 1e-10 * oc.pr
        if math.isinf(oc.kappa):
            assert math.isinf(inf.kappa)
        else:
            assert abs(inf.kappa - oc.kappa) <= 1e-8 * oc.kappa
        np.testing.assert_allclose(ex["eigenvalues"], oc.lam, rtol=0, atol=1e-12 * oc.lam[0])
        # eigenvectors of well-separated eigenvalues agree, same sign rule
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


def test_calibration_thread_count_does_not_change_results():
    cfg = wl.CONFIGS["llama8b"]
    X, G = _heads(cfg, "k", [(0, h) for h in range(4)])
    a = sq.sq_calibrate(X, 3.0, 1, G, n_threads=1)
    b = sq.sq_calibrate(X, 3.0, 1, G, n_threads=4)
    for k in range(4):
        ea, eb = a.export(k), b.export(k)
        for key in ("eigenvalues", "rotation", "widths", "thresholds", "centroids", "qjl"):
            np.testing.assert_array_equal(ea[key], eb[key])


def test_degenerate_calibrations_agree_on_integer_parts():
    d = 32
    zero = np.zeros((1, 40, d), np.float32)
    cal = sq.sq_calibrate(zero, 3.0, 0, None)
    oc = oracle.calibrate(zero[0], 3.0, 0, None)
    assert cal.info(0).d_eff == oc.d_eff == 1
    np.testing.assert_array_equal(cal.export(0)["widths"], oc.widths)
    rank_def = wl.flat_data(16, d)[None].astype(np.float32)        # n < d
    cal = sq.sq_calibrate(rank_def, 3.0, 0, None)
    oc = oracle.calibrate(rank_def[0], 3.0, 0, None)
    assert cal.info(0).d_eff == oc.d_eff
    np.testing.assert_array_equal(cal.export(0)["widths"], oc.widths)


def test_save_load_roundtrip(tmp_path):
    cfg = wl.CONFIGS["tiny"]
    X, G = _heads(cfg, "k", [(0, 0), (1, 2)])
    cal = sq.sq_calibrate(X, 3.0, 1, G)
    p = str(tmp_path / "c.sqcal")
    cal.save(p)
    cal2 = sq.Calibration.load(p)
    assert cal2.n_heads == 2
    for k in range(2):
        a, b = cal.export(k), cal2.export(k)
        for key in ("eigenvalues", "rotation", "widths", "thresholds", "centroids", "qjl"):
            np.testing.assert_array_equal(a[key], b[key])
        ia, ib = a["info"], b["info"]
        assert (ia.d_eff, ia.m, ia.record_words, ia.n_thresholds) == (ib.d_eff, ib.m, ib.record_words, ib.n_thresholds)
    assert cal.packed_head_words(100) == cal2.packed_head_words(100) == 128 * max(
        cal.info(0).record_words, cal.info(1).record_words)
    bad = tmp_path / "bad.sqcal"
    bad.write_bytes(b"not a calibration file")
    with pytest.raises(sq.SQError) as e:
        sq.Calibration.load(str(bad))
    assert e.value.status == 6
    trunc = tmp_path / "trunc.sqcal"
    trunc.write_bytes(open(p, "rb").read()[:200])
    with pytest.raises(sq.SQError):
        sq.Calibration.load(str(trunc))


def test_host_unpack_reads_oracle_records():
    cfg = wl.CONFIGS["llama8b"]
    X, G = _heads(cfg, "k", [(0, 1)])
    cal = sq.sq_calibrate(X, 3.0, 1, G)
    oc = oracle.calibrate(X[0], 3.0, 1, G[0])
    x = wl.kv_block(cfg, 0, 1, "k", 333, "data")
    r = oracle.compress(oc, x)
    p = oracle.pack(oc.widths, oc.m, r.codes, r.z, r.gamma)
    codes, z, gamma = sq.sq_unpack(cal, 0, p, 333)
    np.testing.assert_array_equal(codes, r.codes)
    np.testing.assert_array_equal(z, r.z)
    np.testing.assert_array_equal(gamma, r.gamma.astype(np.float32))


def test_error_paths():
    d = 32
    x = wl.flat_data(64, d)[None].astype(np.float32)
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate(np.zeros((1, 10, 48), np.float32), 3.0, 0)
    assert e.value.status == 2
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate(x[:, :1], 3.0, 0)
    assert e.value.status == 3
    bad = x.copy()
    bad[0, 3, 5] = np.nan
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate(bad, 3.0, 0)
    assert e.value.status == 3
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate(x, 9.0, 0)
    assert e.value.status == 1
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate(x, 3.0, 1, None)
    assert e.value.status == 1
    cal = sq.sq_calibrate(x, 3.0, 0)
    with pytest.raises(sq.SQError) as e:
        cal.info(1)
    assert e.value.status == 1
    lib = sq.lib()
    # device calls on a handle that was never uploaded: rejected before any HIP call
    st = lib.sq_compress(cal.handle, 0, 1, 1, 0, None, 1, 64, 0, 0, d, None, 0, 64, None)
    assert st == 7 and b"upload" in lib.sq_last_error()
    st = lib.sq_compress_append(cal.handle, 0, 1, 1, 0, None, 1, 64, 0, 0, d, None, 0, 64, 0, None)
    assert st == 7 and b"sq_compress_append" in lib.sq_last_error()
    st = lib.sq_scores(None, 0, 0, 1, 4, 1, None, 1, None, 0, 0, 64, None, None)
    assert st == 1
    o = sq.CalibOpts()
    assert lib.sq_calib_default_opts(None, 32) == 1
    assert lib.sq_calib_default_opts(C.byref(o), 32) == 0 and o.max_bits == 8
    assert lib.sq_packed_head_words(None, 10) == -1


def test_workspace_size_formula():
    # [batch][q head][chunk][d + 2] fp32; chunks of the largest of 2048, 1024,
    # ..., 128 tokens with batch * q heads * chunks >= 4096, else 64
    assert sq.sq_attend_workspace_bytes(64, 32, 32768, 128) == 64 * 32 * 16 * 130 * 4  # 2048
    assert sq.sq_attend_workspace_bytes(1, 32, 32768, 128) == 32 * 128 * 130 * 4       # 256
    assert sq.sq_attend_workspace_bytes(48, 40, 512, 128) == 48 * 40 * 4 * 130 * 4     # 128
    assert sq.sq_attend_workspace_bytes(1, 32, 2048, 128) == 32 * 32 * 130 * 4         # 64
    assert sq.sq_attend_workspace_bytes(1, 4, 1, 32) == 4 * 1 * 34 * 4
    assert sq.sq_attend_workspace_bytes(1, 4, 0, 32) == 0


def test_stale_library_is_refused(tmp_path):
    """A libsq.so built from other sources than the ones beside it is refused
    at load time (its compiled-in source digest differs), so a test or a
    benchmark can never run an out-of-date binary."""
    import shutil
    import subprocess
    import sys
    sq.lib()  # the in-tree library exists and matches
    pkg = os.path.join(ROOT, "compression_sq_compress_amd")
    dst = tmp_path / "compression_sq_compress_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("_build", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    probe = ("import sys; sys.path.insert(0, %r); import compression_sq_compress_amd as m; "
             "m.lib(); print('loaded')" % str(tmp_path))
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True)
    assert r.returncode == 0 and "loaded" in r.stdout, r.stderr[-2000:]
    with open(dst / "csrc" / "api.cpp", "a") as f:
        f.write("\n// a later edit\n")
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True)
    assert r.returncode != 0 and "StaleLibraryError" in r.stderr, (r.stdout, r.stderr[-2000:])


def test_turboquant_style_calibration_matches_oracle():
    """sq_calibrate_tq (host C++) against oracle.tq_calibration: same widths,
    QJL rows, record length, rotation and sketch; Gaussian Lloyd-Max tables
    (Max, 1960, over sqrt(d)) to float32 rounding."""
    for keys, bits, d in ((True, 3, 128), (False, 3, 128), (True, 4, 32), (False, 2, 256)):
        r = np.random.default_rng(d + bits)
        rot = np.stack([wl.random_orthogonal(r, d) for _ in range(2)]).astype(np.float32)
        sk = r.standard_normal((2, d, d)).astype(np.float32)
        cal = sq.sq_calibrate_tq(rot, bits, keys, sk if keys else None)
        for h in range(2):
            oc = oracle.tq_calibration(rot[h].astype(np.float64), sk[h], bits, keys)
            ex = cal.export(h)
            inf = ex["info"]
            assert inf.normalized == 1 and inf.m == oc.m and inf.record_words == oc.W
            np.testing.assert_array_equal(ex["widths"], oc.widths)
            np.testing.assert_array_equal(ex["rotation"], rot[h].astype(np.float64))
            thr = np.concatenate([t for t in oc.thresholds if len(t)] or [np.zeros(0)])
            cen = np.concatenate([c for c in oc.centroids if len(c)] or [np.zeros(0)])
            np.testing.assert_allclose(ex["thresholds"], thr, rtol=1e-6, atol=1e-9)
            np.testing.assert_allclose(ex["centroids"], cen, rtol=1e-6, atol=1e-9)
            if keys:
                np.testing.assert_array_equal(ex["qjl"], sk[h])


def test_normalized_calibration_matches_oracle():
    cfg = wl.CONFIGS["llama8b"]
    for which in ("k", "v"):
        X, G = _heads(cfg, which, [(0, 2), (0, 5)])
        qb = 1 if which == "k" else 0
        cal = sq.sq_calibrate(X, 3.0, qb, G, normalize=True)
        for k in range(2):
            oc = oracle.calibrate(X[k], 3.0, qb, G[k] if G is not None else None, normalize=True)
            ex = cal.export(k)
            inf = ex["info"]
            assert inf.normalized == 1 and inf.d_eff == oc.d_eff and inf.record_words == oc.W
            np.testing.assert_array_equal(ex["widths"], oc.widths)
            np.testing.assert_allclose(ex["eigenvalues"], oc.lam, rtol=0, atol=1e-12 * oc.lam[0])
            cen = np.concatenate([c for c in oc.centroids if len(c)])
            np.testing.assert_allclose(ex["centroids"], cen, rtol=1e-6, atol=1e-6 * oc.sigma[0])


@pytest.mark.parametrize("which,frac", [("k", 0.9), ("k", 0.5), ("v", 0.95)])
def test_cumvar_calibration_matches_oracle(which, frac):
    from harness import assert_calibration_matches
    cfg = wl.CONFIGS["llama8b"]
    X, G = _heads(cfg, which, [(0, 0), (0, 3)])
    qb = 1 if which == "k" else 0
    cal = sq.sq_calibrate(X, 3.0, qb, G, deff_cumvar=frac)
    for k in range(2):
        oc = oracle.calibrate(X[k], 3.0, qb, G[k] if G is not None else None, deff_cumvar=frac)
        assert_calibration_matches(cal.export(k), oc)


def test_cumvar_option_is_checked_and_saved(tmp_path):
    cfg = wl.CONFIGS["tiny"]
    X, G = _heads(cfg, "k", [(0, 0)])
    for bad in (-0.1, 1.5, float("nan")):
        with pytest.raises(sq.SQError) as e:
            sq.sq_calibrate(X, 3.0, 1, G, deff_cumvar=bad)
        assert e.value.status == 1
    o = sq.sq_calib_default_opts(64)
    assert o.deff_cumvar == 0.0
    cal = sq.sq_calibrate(X, 3.0, 1, G, deff_cumvar=0.99)
    p = str(tmp_path / "cv.sqcal")
    cal.save(p)
    cal2 = sq.Calibration.load(p)
    assert cal2.info(0).d_eff == cal.info(0).d_eff
    np.testing.assert_array_equal(cal2.export(0)["qjl"], cal.export(0)["qjl"])
