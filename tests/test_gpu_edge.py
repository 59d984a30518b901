"""GPU edge cases: empty and one-token inputs, strided and batched inputs,
per-batch calibration heads, extreme bit budgets, degenerate calibrations,
fp32 inputs at every supported head_dim, and argument errors that must be
rejected before anything is enqueued."""
import math
import sys

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


def _dev(torch, a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t.to(dtype) if dtype is not None else t


def test_empty_inputs(torch_dev, sq):
    torch = torch_dev
    cfg = wl.CONFIGS["llama8b"]
    heads = [(0, 0), (0, 1)]
    _case("T=0 compress/scores/dequantize/attend")
    kcal, _ = H.calibrate_both(sq, cfg, heads, "k", 3.0)
    vcal, _ = H.calibrate_both(sq, cfg, heads, "v", 3.0)
    kcal.upload()
    vcal.upload()
    x = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    kp = torch.full((1, 2, 64), -1, dtype=torch.int32, device="cuda")
    sq.sq_compress(kcal, x, kp)
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros((1, 8, 0), dtype=torch.float32, device="cuda")
    sq.sq_scores(kcal, q, kp, 0, s, 2)
    deq = torch.full((1, 2, 1, 128), 5.0, dtype=torch.float32, device="cuda")
    sq.sq_dequantize(kcal, kp, 0, deq)
    out = torch.full((1, 8, 128), 3.0, dtype=torch.float32, device="cuda")
    ws = torch.zeros(1, dtype=torch.float32, device="cuda")
    sq.sq_attend(vcal, s, 1.0, kp, 0, ws, out, 2)
    torch.cuda.synchronize()
    assert torch.all(kp == -1) and torch.all(deq == 5.0)
    assert torch.all(out == 0.0)


def _e2e(torch, sq, cfg, heads, T, budget, dt, x_layout="contiguous", require_attend=True):
    """Compress K and V on the GPU, score and attend; compare with the
    oracle (records by the acceptance rules, scores on matching tokens,
    attend when every record of the head matches; with require_attend at
    least one head must have been compared)."""
    nkv = len(heads)
    G = cfg.q_heads // cfg.kv_heads
    kcal, kors = H.calibrate_both(sq, cfg, heads, "k", budget)
    vcal, vors = H.calibrate_both(sq, cfg, heads, "v", budget)
    kcal.upload()
    vcal.upload()
    xk = H.data_block(cfg, heads, "k", T)
    xv = H.data_block(cfg, heads, "v", T)
    if x_layout == "hf":
        # [B][T][H][d] storage viewed as [B][H][T][d]
        xkd = _dev(torch, np.ascontiguousarray(xk.transpose(1, 0, 2))[None], dt).permute(0, 2, 1, 3)
        xvd = _dev(torch, np.ascontiguousarray(xv.transpose(1, 0, 2))[None], dt).permute(0, 2, 1, 3)
        assert not xkd.is_contiguous()
    else:
        xkd, xvd = _dev(torch, xk[None], dt), _dev(torch, xv[None], dt)
    kp = torch.zeros((1, nkv, kcal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    vp = torch.zeros((1, nkv, vcal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    sq.sq_compress(kcal, xkd, kp)
    sq.sq_compress(vcal, xvd, vp)
    q = wl.queries(cfg, 1, nkv * G)
    qd = _dev(torch, q, dt)
    scores = torch.zeros((1, nkv * G, T), dtype=torch.float32, device="cuda")
    sq.sq_scores(kcal, qd, kp, T, scores, nkv)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    ws = torch.zeros(sq.sq_attend_workspace_bytes(1, nkv * G, T, cfg.head_dim) // 4 + 1,
                     dtype=torch.float32, device="cuda")
    out = torch.zeros((1, nkv * G, cfg.head_dim), dtype=torch.float32, device="cuda")
    sq.sq_attend(vcal, scores, scale, vp, T, ws, out, nkv)
    torch.cuda.synchronize()
    kpn = kp.cpu().numpy().view(np.uint32)[0]
    vpn = vp.cpu().numpy().view(np.uint32)[0]
    s_g = scores.cpu().numpy()[0]
    o_g = out.cpu().numpy()[0]
    flips = 0
    compared = 0
    for k in range(nkv):
        sk, rk = H.compare_compress(kors[k], kpn[k], xk[k], T)
        sv, rv = H.compare_compress(vors[k], vpn[k], xv[k], T)
        flips += sk["flips"] + sv["flips"]
        oc = kors[k]
        gc, gz, _ = oracle.unpack(oc.widths, oc.m, kpn[k], T)
        same = (gc == rk.codes).all(axis=1) & (gz == rk.z).all(axis=1)
        qg = q[0, k * G:(k + 1) * G].astype(np.float64)
        ref = oracle.scores_rotated(oc, qg, rk.codes, rk.z, rk.gamma)
        xt = oracle.dequantize(oc, rk.codes, rk.z, rk.gamma)
        H.assert_close_floor(s_g[k * G:(k + 1) * G][:, same], ref[:, same],
                             H.score_floor(oc, qg, xt)[:, same], f"scores head {k}")
        vc, _, _ = oracle.unpack(vors[k].widths, 0, vpn[k], T)
        if same.all() and np.array_equal(vc, rv.codes):
            oref = oracle.attend(vors[k], ref, scale, rv.codes)
            fl = np.linalg.norm(oref, axis=1, keepdims=True) / math.sqrt(cfg.head_dim)
            H.assert_close_floor(o_g[k * G:(k + 1) * G], oref, fl, f"attend head {k}")
            compared += 1
    print(f"  heads with attend compared: {compared}/{nkv}", flush=True)
    if require_attend:
        assert compared > 0, "no head's attention output was compared"
    return kp, vp, flips


def test_one_token(torch_dev, sq):
    _case("T=1 llama8b e2e")
    _e2e(torch_dev, sq, wl.CONFIGS["llama8b"], [(0, 0), (0, 5)], 1, 3.0, torch_dev.bfloat16)


@pytest.mark.parametrize("T", [63, 65, 129])
def test_ragged_tails(torch_dev, sq, T):
    _case(f"ragged T={T} qwen14b e2e")
    _e2e(torch_dev, sq, wl.CONFIGS["qwen14b"], [(3, 0), (3, 1), (3, 2)], T, 2.5, torch_dev.bfloat16)


def test_strided_input_matches_contiguous(torch_dev, sq):
    """HF-style [B][T][H][d] storage gives the same records as contiguous."""
    torch = torch_dev
    cfg = wl.CONFIGS["llama8b"]
    heads = [(0, h) for h in range(4)]
    _case("strided (HF layout) input llama8b")
    kp_s, vp_s, _ = _e2e(torch, sq, cfg, heads, 300, 3.0, torch.bfloat16, x_layout="hf")
    kp_c, vp_c, _ = _e2e(torch, sq, cfg, heads, 300, 3.0, torch.bfloat16)
    assert torch.equal(kp_s, kp_c) and torch.equal(vp_s, vp_c)


def test_batch_with_shared_and_per_batch_calibration(torch_dev, sq):
    """batch=3 with one calibration for all entries (stride 0) equals three
    single-entry calls; per-layer calibrations addressed through the
    calibration batch stride match the oracle of each layer."""
    torch = torch_dev
    cfg = wl.CONFIGS["qwen14b"]
    T = 200
    _case("batch=3 shared calibration; batch=2 per-layer calibration (stride 8)")
    heads = [(0, h) for h in range(8)]
    cal, _ = H.calibrate_both(sq, cfg, heads, "k", 3.5)
    cal.upload()
    xs = np.stack([np.stack([wl.kv_block(cfg, 0, h, "k", T, "data", batch_index=b) for h in range(8)])
                   for b in range(3)])
    x = _dev(torch, xs, torch.bfloat16)
    slot = cal.packed_head_words(T)
    kp = torch.zeros((3, 8, slot), dtype=torch.int32, device="cuda")
    sq.sq_compress(cal, x, kp)
    for b in range(3):
        one = torch.zeros((1, 8, slot), dtype=torch.int32, device="cuda")
        sq.sq_compress(cal, x[b:b + 1], one)
        torch.cuda.synchronize()
        assert torch.equal(one[0], kp[b])
    # two layers as the batch dimension, calibration head = 8*b + h
    lheads = [(l, h) for l in (10, 11) for h in range(8)]
    lcal, lors = H.calibrate_both(sq, cfg, lheads, "k", 3.5)
    lcal.upload()
    xl = np.stack([H.data_block(cfg, lheads[8 * b:8 * b + 8], "k", T) for b in range(2)])
    lp = torch.zeros((2, 8, lcal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    sq.sq_compress(lcal, _dev(torch, xl, torch.bfloat16), lp, calib_batch_stride=8)
    torch.cuda.synchronize()
    lpn = lp.cpu().numpy().view(np.uint32)
    for b in range(2):
        for h in range(8):
            H.compare_compress(lors[8 * b + h], lpn[b, h], xl[b, h], T)


@pytest.mark.parametrize("budget", [0.125, 0.25])
def test_zero_width_signal_coordinates(torch_dev, sq, budget):
    """Budgets below one bit per coordinate on the tiny workload (d_eff 9)
    leave signal coordinates of width zero: they carry no code but enter the
    QJL residual with their full value, a case the grid quantiser's
    pre-scaled rotation rows handle apart (scale 1, code 0)."""
    cfg = wl.CONFIGS["tiny"]
    heads = [(0, 0), (1, 2)]
    _case(f"zero-width signal coordinates: tiny, budget {budget}")
    X, G = H.calib_inputs(cfg, heads, "k")
    cal = sq.sq_calibrate(X, budget, cfg.qjl_bits, G)
    inf = cal.info(0)
    w = cal.export(0)["widths"]
    assert (w[:inf.d_eff] == 0).any() and inf.m > 0, (w[:inf.d_eff], inf.m)
    _e2e(torch_dev, sq, cfg, heads, 200, budget, torch_dev.float32)


@pytest.mark.parametrize("budget", [0.5, 1.0, 6.0, 8.0])
def test_extreme_budgets(torch_dev, sq, budget):
    """Low budgets leave many zero-width coordinates; 8 bits/coord gives every
    coordinate the maximum width and the longest records.  With 255
    thresholds per coordinate, in-band flips are common at high budgets, so
    the attention output is compared where the records match and, for these
    table placements, unconditionally on oracle records in
    test_gpu_parity.test_attend_table_placements_on_oracle_records."""
    _case(f"budget {budget} llama8b e2e")
    _e2e(torch_dev, sq, wl.CONFIGS["llama8b"], [(0, 2), (0, 6)], 200, budget, torch_dev.bfloat16,
         require_attend=budget < 6)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_fp32_inputs_every_head_dim(torch_dev, sq, d):
    """fp32 K/V and queries on flat-spectrum data at each supported head_dim."""
    torch = torch_dev
    _case(f"fp32 flat d={d}")
    T, nkv, G = 150, 2, 2
    X = np.stack([wl.flat_data(400, d, seed=s) for s in (1, 2)]).astype(np.float32)
    Gm = np.stack([np.random.default_rng(100 + s).standard_normal((d, d)).astype(np.float32)
                   for s in range(nkv)])
    cal = sq.sq_calibrate(X, 3.0, 1, Gm).upload()
    ors = [oracle.calibrate(X[k], 3.0, 1, Gm[k]) for k in range(nkv)]
    for k in range(nkv):
        assert cal.info(k).d_eff == ors[k].d_eff and cal.info(k).record_words == ors[k].W
    x = np.stack([wl.flat_data(T, d, seed=10 + s) for s in range(nkv)]).astype(np.float32)
    kp = torch.zeros((1, nkv, cal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    sq.sq_compress(cal, _dev(torch, x[None]), kp)
    q = np.random.default_rng(5).standard_normal((1, nkv * G, d)).astype(np.float32)
    s = torch.zeros((1, nkv * G, T), dtype=torch.float32, device="cuda")
    sq.sq_scores(cal, _dev(torch, q), kp, T, s, nkv)
    torch.cuda.synchronize()
    kpn = kp.cpu().numpy().view(np.uint32)[0]
    sg = s.cpu().numpy()[0]
    for k in range(nkv):
        st, r = H.compare_compress(ors[k], kpn[k], x[k], T)
        gc, gz, _ = oracle.unpack(ors[k].widths, ors[k].m, kpn[k], T)
        same = (gc == r.codes).all(axis=1) & (gz == r.z).all(axis=1)
        qg = q[0, k * G:(k + 1) * G].astype(np.float64)
        ref = oracle.scores_rotated(ors[k], qg, r.codes, r.z, r.gamma)
        xt = oracle.dequantize(ors[k], r.codes, r.z, r.gamma)
        H.assert_close_floor(sg[k * G:(k + 1) * G][:, same], ref[:, same],
                             H.score_floor(ors[k], qg, xt)[:, same], f"fp32 d={d} head {k}")


@pytest.mark.parametrize("name,dt", [("llama8b", "bf16"), ("llama8b", "f32"), ("gemma9b", "bf16")])
def test_nan_inputs(torch_dev, sq, name, dt):
    """NaN entries of either sign in K and V (reading R7: a NaN coordinate
    codes as 0).  One NaN entry makes the whole rotated token NaN on both
    sides, so those tokens must carry all-zero codes and QJL bits and a NaN
    gamma; the other tokens follow the usual acceptance rules."""
    torch = torch_dev
    cfg = wl.CONFIGS[name]
    heads = [(0, 0)]
    T = 100
    _case(f"NaN inputs {dt} {name} T={T}")
    nan_tok = [3, 70, 99]
    for which in ("k", "v"):
        cal, ors = H.calibrate_both(sq, cfg, heads, which, 3.0)
        cal.upload()
        x = H.data_block(cfg, heads, which, T)[0].astype(np.float32)
        if dt == "bf16":
            xd = _dev(torch, x[None, None], torch.bfloat16)
            bits = xd.view(torch.int16)
            bits[0, 0, 3, 7] = 0x7FC0           # +NaN
            bits[0, 0, 70, 0] = -64             # 0xFFC0: -NaN
            bits[0, 0, 99, :] = -127            # 0xFF81: -NaN, signalling payload
        else:
            xd = _dev(torch, x[None, None])
            bits = xd.view(torch.int32)
            bits[0, 0, 3, 7] = 0x7FC00000
            bits[0, 0, 70, 0] = -4194304        # 0xFFC00000
            bits[0, 0, 99, :] = -8388607        # 0xFF800001
        x[nan_tok] = np.nan
        kp = torch.full((1, 1, cal.packed_head_words(T)), -1, dtype=torch.int32, device="cuda")
        sq.sq_compress(cal, xd, kp)
        torch.cuda.synchronize()
        got = kp.cpu().numpy().view(np.uint32)[0, 0]
        oc = ors[0]
        H.compare_compress(oc, got, x, T)
        gc, gz, gg = oracle.unpack(oc.widths, oc.m, got, T)
        assert np.all(gc[nan_tok] == 0), f"{which}: NaN tokens must code as 0"
        if oc.m > 0:
            assert np.all(gz[nan_tok] == 0), "NaN tokens must have all QJL bits clear"
            assert np.all(np.isnan(gg[nan_tok].astype(np.float32))), "NaN tokens must have a NaN gamma"


@pytest.mark.parametrize("d", [32, 64])
def test_bf16_inputs_small_head_dims(torch_dev, sq, d):
    """bf16 keys at head_dim 32 and 64 (the register-quantising compress kernel
    with 2 and 4 waves), several tiles and a ragged tail."""
    torch = torch_dev
    _case(f"bf16 flat d={d}")
    T, nkv = 300, 2
    X = np.stack([wl.flat_data(400, d, seed=s) for s in (3, 4)]).astype(np.float32)
    Gm = np.stack([np.random.default_rng(200 + s).standard_normal((d, d)).astype(np.float32)
                   for s in range(nkv)])
    cal = sq.sq_calibrate(X, 3.0, 1, Gm).upload()
    ors = [oracle.calibrate(X[k], 3.0, 1, Gm[k]) for k in range(nkv)]
    xd = _dev(torch, np.stack([wl.flat_data(T, d, seed=20 + s) for s in range(nkv)])[None], torch.bfloat16)
    x = xd.float().cpu().numpy()[0]  # the bf16-rounded values the kernel sees
    kp = torch.zeros((1, nkv, cal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    sq.sq_compress(cal, xd, kp)
    torch.cuda.synchronize()
    kpn = kp.cpu().numpy().view(np.uint32)[0]
    for k in range(nkv):
        assert cal.info(k).record_words == ors[k].W
        H.compare_compress(ors[k], kpn[k], x[k], T)


def test_degenerate_zero_calibration(torch_dev, sq):
    """All-zero calibration data: every threshold and centroid is 0 and the
    basis is arbitrary, so only what is unique is compared: zero vectors give
    all-zero codes, gamma 0 and every QJL bit set."""
    torch = torch_dev
    d, T = 64, 70
    _case("zero calibration d=64")
    X = np.zeros((1, 50, d), np.float32)
    Gm = np.random.default_rng(3).standard_normal((1, d, d)).astype(np.float32)
    cal = sq.sq_calibrate(X, 3.0, 1, Gm).upload()
    oc = oracle.calibrate(X[0], 3.0, 1, Gm[0])
    assert cal.info(0).d_eff == oc.d_eff == 1 and cal.info(0).record_words == oc.W
    x = torch.zeros((1, 1, T, d), dtype=torch.bfloat16, device="cuda")
    kp = torch.full((1, 1, cal.packed_head_words(T)), -1, dtype=torch.int32, device="cuda")
    sq.sq_compress(cal, x, kp)
    torch.cuda.synchronize()
    r = oracle.compress(oc, np.zeros((T, d)))
    ref = oracle.pack(oc.widths, oc.m, r.codes, r.z, r.gamma)
    got = kp.cpu().numpy().view(np.uint32)[0, 0]
    assert np.array_equal(got[:ref.size], ref)
    assert np.all(r.codes == 0) and np.all(r.z == 1) and np.all(r.gamma == 0)


def test_argument_errors_enqueue_nothing(torch_dev, sq):
    torch = torch_dev
    cfg = wl.CONFIGS["llama8b"]
    heads = [(0, 0), (0, 1)]
    _case("argument errors")
    cal, _ = H.calibrate_both(sq, cfg, heads, "k", 3.0)
    cal.upload()
    T = 100
    x = torch.zeros((1, 2, T, 128), dtype=torch.bfloat16, device="cuda")
    small = torch.full((1, 2, cal.packed_head_words(T) - 64), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(sq.SQError) as e:
        sq.sq_compress(cal, x, small)
    assert e.value.status == 1
    bad_x = torch.zeros((1, 2, T, 130), dtype=torch.bfloat16, device="cuda")[..., 1:129]
    kp = torch.full((1, 2, cal.packed_head_words(T)), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(sq.SQError):
        sq.sq_compress(cal, bad_x, kp)
    q = torch.zeros((1, 7, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros((1, 7, T), dtype=torch.float32, device="cuda")
    with pytest.raises(sq.SQError) as e:
        sq.sq_scores(cal, q, kp, T, s, 2)
    assert e.value.status == 1
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros((1, 8, T), dtype=torch.float32, device="cuda")
    out = torch.zeros((1, 8, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(4, dtype=torch.float32, device="cuda")
    with pytest.raises(sq.SQError) as e:
        sq.sq_attend(cal, s, 1.0, kp, T, ws, out, 2)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.all(kp == -1) and torch.all(small == -1)
