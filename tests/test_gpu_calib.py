"""GPU calibration (sq_calibrate_device: fp64 second moment, parallel Jacobi
eigendecomposition and sample rotation on the device, Lloyd-Max on the host)
against the oracle's calibration of the same samples, for both d_eff rules and
the normalised variant, plus the calibration-stability coefficient of
variation over disjoint sample splits."""
import sys
import time

import numpy as np
import pytest

import harness as H
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


@pytest.fixture(scope="module")
def sq(torch_dev):
    import compression_sq_compress_amd as m
    return m


def _case(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cfgname,which,heads,budget,normalize,cumvar", [
    ("tiny", "k", [(0, h) for h in range(4)], 3.0, False, 0.0),
    ("tiny", "v", [(1, h) for h in range(4)], 3.0, False, 0.0),
    ("llama8b", "k", [(0, h) for h in range(8)], 3.0, False, 0.0),
    ("llama8b", "v", [(0, h) for h in range(8)], 3.0, False, 0.0),
    ("qwen14b", "k", [(5, h) for h in range(4)], 2.5, False, 0.9),
    ("qwen14b", "v", [(6, h) for h in range(4)], 3.5, True, 0.0),
    ("llama8b", "k", [(0, 1), (0, 6)], 3.0, True, 0.95),
    ("gemma9b", "k", [(3, 0), (3, 1)], 3.0, False, 0.0),
    ("gemma9b", "v", [(3, 2)], 3.0, False, 0.9),
])
def test_device_calibration_matches_oracle(torch_dev, sq, cfgname, which, heads, budget, normalize,
                                           cumvar):
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    _case(f"calibrate_device {cfgname} {which} heads={len(heads)} norm={normalize} cumvar={cumvar}")
    X, G = H.calib_inputs(cfg, heads, which)
    qb = cfg.qjl_bits if which == "k" else 0
    xd = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).cuda()
    cal = sq.sq_calibrate_device(xd, budget, qb, G, normalize=normalize, deff_cumvar=cumvar)
    host = sq.sq_calibrate(X, budget, qb, G, normalize=normalize, deff_cumvar=cumvar)
    for k in range(len(heads)):
        oc = oracle.calibrate(X[k].astype(np.float64), budget, qb, G[k] if G is not None else None,
                              normalize=normalize, deff_cumvar=cumvar)
        ex = cal.export(k)
        H.assert_calibration_matches(ex, oc)
        assert ex["info"].normalized == int(normalize)
        hx = host.export(k)
        np.testing.assert_array_equal(ex["widths"], hx["widths"])
        assert ex["info"].d_eff == hx["info"].d_eff and ex["info"].record_words == hx["info"].record_words


def test_device_calibration_runs_the_pipeline(torch_dev, sq):
    """A device calibration drives compress + scores exactly like the host one:
    upload both, compress the same block, compare records word for word where
    the two codebooks agree to the float32 bit (else both within the parity
    bands of their own oracle reading)."""
    torch = torch_dev
    cfg = wl.CONFIGS["llama8b"]
    heads = [(0, h) for h in range(8)]
    X, G = H.calib_inputs(cfg, heads, "k")
    _case("calibrate_device llama8b keys -> compress")
    cal = sq.sq_calibrate_device(torch.from_numpy(X).cuda(), 3.0, 1, G).upload()
    T = 700
    x = np.stack([wl.kv_block(cfg, l, h, "k", T, "data") for l, h in heads])[None].astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    words = cal.packed_head_words(T)
    packed = torch.zeros((1, len(heads), words), dtype=torch.int32, device="cuda")
    sq.sq_compress(cal, xd, packed)
    torch.cuda.synchronize()
    pk = packed.cpu().numpy()
    for k, (l, h) in enumerate(heads):
        ex = cal.export(k)
        oc = oracle.calibrate(X[k].astype(np.float64), 3.0, 1, G[k])
        H.compare_compress(oc, pk[0, k], x[0, k].astype(np.float64), T)
        assert ex["info"].d_eff == oc.d_eff


def test_device_calibration_errors(torch_dev, sq):
    torch = torch_dev
    x = torch.randn(2, 100, 64, device="cuda")
    bad = x.clone()
    bad[1, 17, 3] = float("inf")
    _case("calibrate_device errors")
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate_device(bad, 3.0, 0)
    assert e.value.status == 3 and "head 1" in str(e.value)
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate_device(x[:, :1].contiguous(), 3.0, 0)
    assert e.value.status == 3
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate_device(x, 3.0, 1, None)
    assert e.value.status == 1
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate_device(x, 3.0, 0, deff_cumvar=2.0)
    assert e.value.status == 1
    with pytest.raises(sq.SQError) as e:
        sq.sq_calibrate_device(torch.randn(1, 10, 48, device="cuda"), 3.0, 0)
    assert e.value.status == 2


def test_calibration_stability_cv(torch_dev, sq):
    """Four disjoint splits of one head's calibration set calibrated as four
    heads in one device call; the coefficients of variation of the
    participation ratio and of d_eff match the oracle's on the same splits."""
    torch = torch_dev
    cfg = wl.CONFIGS["qwen14b"]
    for which in ("k", "v"):
        x = wl.kv_block(cfg, 7, 3, which, 4 * 1024, "calib").astype(np.float32)
        splits = x.reshape(4, 1024, cfg.head_dim)
        _case(f"stability {which}")
        t0 = time.perf_counter()
        cal = sq.sq_calibrate_device(torch.from_numpy(np.ascontiguousarray(splits)).cuda(), 3.0, 0)
        dt = time.perf_counter() - t0
        pr = np.array([cal.info(k).participation_ratio for k in range(4)])
        de = np.array([cal.info(k).d_eff for k in range(4)])
        ref = oracle.calibration_stability(x.astype(np.float64), 4)
        np.testing.assert_allclose(pr, ref["pr"], rtol=1e-10)
        np.testing.assert_array_equal(de, ref["d_eff"])
        cv = oracle.coefficient_of_variation(pr)
        assert abs(cv - ref["pr_cv"]) <= 1e-8 * max(ref["pr_cv"], 1e-12) + 1e-14
        print(f"[stability] {which}: PR {pr.round(3)} CV {100 * cv:.2f}% d_eff {de} "
              f"({dt * 1e3:.1f} ms for 4 splits)", flush=True)
