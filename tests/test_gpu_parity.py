"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Each test prints its case before touching the GPU.  Sizes are those the
oracle finishes in seconds while still spanning several 64-token tiles and a
ragged tail; the full-size decode configuration is covered by sampled checks in
test_gpu_fullsize.py.
"""
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


def _to_dev(torch, arr, dtype):
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to("cuda")
    return t.to(dtype)


def _compress_gpu(torch, sq, cal, x_np, dtype, T):
    """x_np [B][H][T][d] -> packed uint32 numpy [B][H][slot]."""
    x = _to_dev(torch, x_np, dtype)
    B, Hh = x.shape[0], x.shape[1]
    slot = cal.packed_head_words(T)
    packed = torch.full((B, Hh, slot), -1, dtype=torch.int32, device="cuda")
    sq.sq_compress(cal, x, packed)
    torch.cuda.synchronize()
    return packed.cpu().numpy().view(np.uint32)


CASES = [
    # name, config, heads, T, budget
    ("tiny", "tiny", [(l, h) for l in range(3) for h in range(4)], 256, 3.0),
    ("llama8b", "llama8b", [(0, h) for h in range(8)], 2048, 3.0),
    ("llama8b-ragged", "llama8b", [(0, h) for h in range(2)], 1000, 3.0),
    ("qwen14b-2.5b", "qwen14b", [(l, h) for l in (0, 47) for h in range(8)], 512, 2.5),
    ("qwen14b-3.5b", "qwen14b", [(l, h) for l in (1,) for h in range(8)], 1024, 3.5),
    ("gemma9b", "gemma9b", [(l, h) for l in (0,) for h in range(4)], 700, 3.0),
    ("hd64", "hd64", [(l, h) for l in range(2) for h in range(4)], 700, 3.0),
]


@pytest.mark.parametrize("name,cfgname,heads,T,budget", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("which", ["k", "v"])
@pytest.mark.parametrize("quantiser", ["grid", "tree"])
def test_compress_matches_oracle(torch_dev, sq, name, cfgname, heads, T, budget, which, quantiser,
                                 monkeypatch):
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    monkeypatch.setenv("SQ_QUANTISER", quantiser)
    _case(f"compress {name} {which} T={T} budget={budget} quantiser={quantiser}")
    cal, ors = H.calibrate_both(sq, cfg, heads, which, budget, n_tokens=T)
    cal.upload()
    x = H.data_block(cfg, heads, which, T)                 # [H][T][d]
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    packed = _compress_gpu(torch, sq, cal, x[None], dt, T)[0]
    tot = dict(coords=0, band=0, flips=0)
    for k in range(len(heads)):
        stats, _ = H.compare_compress(ors[k], packed[k], x[k], T)
        for key in tot:
            tot[key] += stats[key]
    print(f"  coords={tot['coords']} in-band={tot['band']} flips={tot['flips']} "
          f"flip-rate={tot['flips'] / tot['coords']:.2e}", flush=True)
    # compare_compress allows a flip only inside the band; a flip needs the two
    # sides' rotated values to straddle a threshold, i.e. to lie within the
    # fp32 rounding of the rotation (~1e-6 sigma), far inside the 1e-4 sigma
    # band, so flips are a small fraction of the in-band coordinates
    assert tot["flips"] <= max(3, tot["band"] // 5), tot


@pytest.mark.parametrize("name,cfgname,heads,T,budget", CASES, ids=[c[0] for c in CASES])
def test_scores_attend_dequant_on_oracle_records(torch_dev, sq, name, cfgname, heads, T, budget):
    """sq_scores / sq_attend / sq_dequantize fed with ORACLE-packed records and
    oracle scores, compared with the oracle on the same inputs, on every
    workload.  The Gemma-shaped keys (head_dim 256) need two passes of the
    scores kernel (the second adds into the scores) and their values the
    attend kernel with four 64-coordinate blocks per wave; both are asserted
    from the launch plan."""
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    _case(f"read-side {name} T={T}")
    nkv = len(heads)
    G = cfg.q_heads // cfg.kv_heads
    kcal, kors = H.calibrate_both(sq, cfg, heads, "k", budget, n_tokens=T)
    vcal, vors = H.calibrate_both(sq, cfg, heads, "v", budget, n_tokens=T)
    kcal.upload()
    vcal.upload()
    plan = sq.sq_plan_decode(kcal, vcal, 1, nkv * G, nkv, T)
    print(f"  plan: score passes {plan.score_passes} (quads {plan.score_quads}, groups "
          f"{plan.score_wave_groups}); attend placement {plan.attend_placement}, waves "
          f"{plan.attend_waves}, blocks {plan.attend_blocks}, chunks {plan.attend_chunks}", flush=True)
    if cfg.head_dim == 256:
        assert plan.score_passes >= 2 and plan.attend_blocks == 4
    if cfg.head_dim == 64:
        assert plan.attend_blocks == 1
    xk = H.data_block(cfg, heads, "k", T)
    xv = H.data_block(cfg, heads, "v", T)
    slot_k = kcal.packed_head_words(T)
    slot_v = vcal.packed_head_words(T)
    kp = np.zeros((1, nkv, slot_k), np.uint32)
    vp = np.zeros((1, nkv, slot_v), np.uint32)
    rk, rv = [], []
    for k in range(nkv):
        r = oracle.compress(kors[k], xk[k])
        p = oracle.pack(kors[k].widths, kors[k].m, r.codes, r.z, r.gamma)
        kp[0, k, :len(p)] = p
        rk.append(r)
        r = oracle.compress(vors[k], xv[k])
        p = oracle.pack(vors[k].widths, vors[k].m, r.codes, r.z, r.gamma)
        vp[0, k, :len(p)] = p
        rv.append(r)
    q = wl.queries(cfg, 1, nkv * G)                       # [1][Hq][d]
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    qd = _to_dev(torch, q, dt)
    kpd = torch.from_numpy(kp.view(np.int32)).cuda()
    vpd = torch.from_numpy(vp.view(np.int32)).cuda()
    scores = torch.zeros((1, nkv * G, T), dtype=torch.float32, device="cuda")
    sq.sq_scores(kcal, qd, kpd, T, scores, nkv)
    # dequantize (keys, with QJL) on oracle records
    deq = torch.zeros((1, nkv, T, cfg.head_dim), dtype=torch.float32, device="cuda")
    sq.sq_dequantize(kcal, kpd, T, deq)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()[0]
    deq_gpu = deq.cpu().numpy()[0]
    worst = 0.0
    oscores = np.zeros((nkv * G, T))
    for k in range(nkv):
        oc, r = kors[k], rk[k]
        xt = oracle.dequantize(oc, r.codes, r.z, r.gamma)
        H.assert_close_floor(deq_gpu[k], xt, np.linalg.norm(xt, axis=1)[:, None] / math.sqrt(cfg.head_dim),
                             f"dequantize head {k}")
        qg = q[0, k * G:(k + 1) * G].astype(np.float64)
        ref = oracle.scores_rotated(oc, qg, r.codes, r.z, r.gamma)
        oscores[k * G:(k + 1) * G] = ref
        worst = max(worst, H.assert_close_floor(s_gpu[k * G:(k + 1) * G], ref,
                                                H.score_floor(oc, qg, xt), f"scores head {k}"))
    print(f"  scores worst err/tol = {worst:.3g}", flush=True)
    # attend on oracle scores (float32 copy) and oracle value records
    scale = 1.0 / math.sqrt(cfg.head_dim)
    s32 = oscores.astype(np.float32)
    sd = torch.from_numpy(s32[None].copy()).cuda()
    ws = torch.zeros(sq.sq_attend_workspace_bytes(1, nkv * G, T, cfg.head_dim) // 4 + 1,
                     dtype=torch.float32, device="cuda")
    out = torch.zeros((1, nkv * G, cfg.head_dim), dtype=torch.float32, device="cuda")
    sq.sq_attend(vcal, sd, scale, vpd, T, ws, out, nkv)
    torch.cuda.synchronize()
    o_gpu = out.cpu().numpy()[0]
    for k in range(nkv):
        ref = oracle.attend(vors[k], s32[k * G:(k + 1) * G].astype(np.float64), scale, rv[k].codes)
        floor = np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(cfg.head_dim)
        H.assert_close_floor(o_gpu[k * G:(k + 1) * G], ref, floor, f"attend head {k}")


@pytest.mark.parametrize("qjl_bits", [2, 4, 6])
def test_scores_qjl_sketch_lengths(torch_dev, sq, qjl_bits):
    """Scores and compress with longer QJL sketches on the Llama-shaped keys
    (d_eff 3): m = 6 and 12 take the scores kernel's sign-pattern tables (one
    chunk, then two chunks of 8 and 4 bits), m = 18 its per-row loop; records
    compressed on the GPU are checked against the oracle's, scores on oracle
    records against the oracle."""
    torch = torch_dev
    cfg = wl.CONFIGS["llama8b"]
    heads, T, G = [(0, 0), (0, 5)], 700, cfg.q_heads // cfg.kv_heads
    _case(f"qjl sketch: qjl_bits={qjl_bits} T={T}")
    X = np.stack([wl.calibration_set(cfg, l, h, "k") for l, h in heads]).astype(np.float32)
    Gs = np.stack([wl.qjl_gaussian(cfg, l, h, "k", qjl_bits=qjl_bits) for l, h in heads])
    kcal = sq.sq_calibrate(X, 3.0, qjl_bits, Gs)
    ors = [oracle.calibrate(X[k], 3.0, qjl_bits, Gs[k]) for k in range(len(heads))]
    for k, oc in enumerate(ors):
        assert kcal.info(k).m == oc.m == qjl_bits * oc.d_eff
    print(f"  m = {[oc.m for oc in ors]}", flush=True)
    kcal.upload()
    xk = H.data_block(cfg, heads, "k", T)
    packed = _compress_gpu(torch, sq, kcal, xk[None], torch.bfloat16, T)[0]
    for k in range(len(heads)):
        H.compare_compress(ors[k], packed[k], xk[k], T)
    nkv = len(heads)
    kp = np.zeros((1, nkv, kcal.packed_head_words(T)), np.uint32)
    rk = []
    for k in range(nkv):
        r = oracle.compress(ors[k], xk[k])
        p = oracle.pack(ors[k].widths, ors[k].m, r.codes, r.z, r.gamma)
        kp[0, k, :len(p)] = p
        rk.append(r)
    q = wl.queries(cfg, 1, nkv * G)
    qd = _to_dev(torch, q, torch.bfloat16)
    kpd = torch.from_numpy(kp.view(np.int32)).cuda()
    scores = torch.zeros((1, nkv * G, T), dtype=torch.float32, device="cuda")
    sq.sq_scores(kcal, qd, kpd, T, scores, nkv)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()[0]
    worst = 0.0
    for k in range(nkv):
        oc, r = ors[k], rk[k]
        xt = oracle.dequantize(oc, r.codes, r.z, r.gamma)
        qg = q[0, k * G:(k + 1) * G].astype(np.float64)
        ref = oracle.scores_rotated(oc, qg, r.codes, r.z, r.gamma)
        worst = max(worst, H.assert_close_floor(s_gpu[k * G:(k + 1) * G], ref,
                                                H.score_floor(oc, qg, xt), f"scores head {k}"))
    print(f"  scores worst err/tol = {worst:.3g}", flush=True)


@pytest.mark.parametrize("name,cfgname,heads,T,budget", CASES, ids=[c[0] for c in CASES])
def test_end_to_end(torch_dev, sq, name, cfgname, heads, T, budget):
    """GPU compress -> GPU scores -> GPU attend against the all-oracle pipeline;
    tokens whose key codes flipped inside the band are excluded from the score
    comparison (and counted); the attention output of a head is compared when
    none of its key or value records differs from the oracle's (a flip changes
    the exact result), and at head_dim <= 128 at least one head must be
    compared (the Gemma-shaped keys' nine 8-bit coordinates make an in-band
    flip likely in every head).  The attend kernel itself is compared on every
    head and workload against oracle inputs in
    test_scores_attend_dequant_on_oracle_records."""
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    _case(f"end-to-end {name} T={T}")
    nkv = len(heads)
    G = cfg.q_heads // cfg.kv_heads
    kcal, kors = H.calibrate_both(sq, cfg, heads, "k", budget, n_tokens=T)
    vcal, vors = H.calibrate_both(sq, cfg, heads, "v", budget, n_tokens=T)
    kcal.upload()
    vcal.upload()
    xk = H.data_block(cfg, heads, "k", T)
    xv = H.data_block(cfg, heads, "v", T)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    xkd = _to_dev(torch, xk[None], dt)
    xvd = _to_dev(torch, xv[None], dt)
    kp = torch.zeros((1, nkv, kcal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    vp = torch.zeros((1, nkv, vcal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    sq.sq_compress(kcal, xkd, kp)
    sq.sq_compress(vcal, xvd, vp)
    q = wl.queries(cfg, 1, nkv * G)
    qd = _to_dev(torch, q, dt)
    scores = torch.zeros((1, nkv * G, T), dtype=torch.float32, device="cuda")
    sq.sq_scores(kcal, qd, kp, T, scores, nkv)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    ws = torch.zeros(sq.sq_attend_workspace_bytes(1, nkv * G, T, cfg.head_dim) // 4 + 1,
                     dtype=torch.float32, device="cuda")
    out = torch.zeros((1, nkv * G, cfg.head_dim), dtype=torch.float32, device="cuda")
    sq.sq_attend(vcal, scores, scale, vp, T, ws, out, nkv)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()[0]
    o_gpu = out.cpu().numpy()[0]
    kp_np = kp.cpu().numpy().view(np.uint32)[0]
    vp_np = vp.cpu().numpy().view(np.uint32)[0]
    excluded = 0
    compared = 0
    for k in range(nkv):
        oc = kors[k]
        r = oracle.compress(oc, xk[k])
        gc, gz, gg = oracle.unpack(oc.widths, oc.m, kp_np[k], T)
        same = (gc == r.codes).all(axis=1) & (gz == r.z).all(axis=1)
        excluded += int((~same).sum())
        qg = q[0, k * G:(k + 1) * G].astype(np.float64)
        ref = oracle.scores_rotated(oc, qg, r.codes, r.z, r.gamma)
        xt = oracle.dequantize(oc, r.codes, r.z, r.gamma)
        fl = H.score_floor(oc, qg, xt)
        H.assert_close_floor(s_gpu[k * G:(k + 1) * G][:, same], ref[:, same], fl[:, same],
                             f"e2e scores head {k}")
        rvv = oracle.compress(vors[k], xv[k])
        vc, _, _ = oracle.unpack(vors[k].widths, 0, vp_np[k], T)
        if same.all() and np.array_equal(vc, rvv.codes):
            oref = oracle.attend(vors[k], ref, scale, rvv.codes)
            floor = np.linalg.norm(oref, axis=1, keepdims=True) / math.sqrt(cfg.head_dim)
            H.assert_close_floor(o_gpu[k * G:(k + 1) * G], oref, floor, f"e2e attend head {k}")
            compared += 1
    print(f"  tokens excluded for in-band key flips: {excluded}; heads with attend compared: "
          f"{compared}/{nkv}", flush=True)
    if cfg.head_dim <= 128:
        assert compared > 0


def test_compress_is_deterministic(torch_dev, sq):
    torch = torch_dev
    cfg = wl.CONFIGS["llama8b"]
    heads = [(0, 0), (0, 1)]
    _case("determinism llama8b k")
    cal, _ = H.calibrate_both(sq, cfg, heads, "k", 3.0)
    cal.upload()
    x = H.data_block(cfg, heads, "k", 640)
    a = _compress_gpu(torch, sq, cal, x[None], torch.bfloat16, 640)
    b = _compress_gpu(torch, sq, cal, x[None], torch.bfloat16, 640)
    assert np.array_equal(a, b)


# Value calibrations whose widths reach 7 or 8 bits: the attend kernel's
# centroid tables then no longer fit one column per lane; they are packed in
# LDS (a few wide coordinates) or read from device memory (many).
PLACEMENTS = [
    # name, config, stream calibrated as values, budget, max_bits, expected placement
    ("values-8b", "llama8b", "v", 8.0, 8, 2),
    ("values-6b", "llama8b", "v", 6.0, 8, None),
    ("keyspectrum-3b", "llama8b", "k", 3.0, 8, 1),
    ("keyspectrum-3b-max7", "llama8b", "k", 3.0, 7, 1),
]


@pytest.mark.parametrize("name,cfgname,which,budget,max_bits,want", PLACEMENTS,
                         ids=[c[0] for c in PLACEMENTS])
def test_attend_table_placements_on_oracle_records(torch_dev, sq, name, cfgname, which, budget,
                                                   max_bits, want):
    """sq_attend on oracle-packed value records and oracle scores, compared
    with oracle.attend unconditionally, for calibrations whose widths reach 7
    and 8 bits (packed and device-memory centroid tables)."""
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    heads = [(0, 2), (0, 6)]
    T, nkv, G = 700, 2, cfg.q_heads // cfg.kv_heads
    _case(f"attend placement {name} budget={budget} max_bits={max_bits}")
    X = np.stack([wl.calibration_set(cfg, l, h, which) for l, h in heads]).astype(np.float32)
    vcal = sq.sq_calibrate(X, budget, 0, None, max_bits=max_bits).upload()
    vors = [oracle.calibrate(X[k], budget, 0, None, max_bits=max_bits) for k in range(nkv)]
    for k in range(nkv):
        assert np.array_equal(vcal.export(k)["widths"], vors[k].widths)
    plan = sq.sq_plan_decode(None, vcal, 1, nkv * G, nkv, T)
    mw = max(int(v.widths.max()) for v in vors)
    print(f"  max width {mw}; attend placement {plan.attend_placement}, waves {plan.attend_waves}",
          flush=True)
    assert mw >= 7 and plan.attend_placement != 0
    if want is not None:
        assert plan.attend_placement == want
    x = np.stack([wl.kv_block(cfg, l, h, which, T, "data") for l, h in heads])
    slot = vcal.packed_head_words(T)
    vp = np.zeros((1, nkv, slot), np.uint32)
    rv = []
    for k in range(nkv):
        r = oracle.compress(vors[k], x[k])
        p = oracle.pack(vors[k].widths, 0, r.codes, r.z, r.gamma)
        vp[0, k, :len(p)] = p
        rv.append(r)
    s = (np.random.default_rng(17).standard_normal((nkv * G, T)) * 12.0).astype(np.float32)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    ws = torch.zeros(sq.sq_attend_workspace_bytes(1, nkv * G, T, cfg.head_dim) // 4 + 1,
                     dtype=torch.float32, device="cuda")
    out = torch.zeros((1, nkv * G, cfg.head_dim), dtype=torch.float32, device="cuda")
    sq.sq_attend(vcal, torch.from_numpy(s[None].copy()).cuda(), scale,
                 torch.from_numpy(vp.view(np.int32)).cuda(), T, ws, out, nkv)
    torch.cuda.synchronize()
    o_gpu = out.cpu().numpy()[0]
    for k in range(nkv):
        ref = oracle.attend(vors[k], s[k * G:(k + 1) * G].astype(np.float64), scale, rv[k].codes)
        floor = np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(cfg.head_dim)
        H.assert_close_floor(o_gpu[k * G:(k + 1) * G], ref, floor, f"attend {name} head {k}")


@pytest.mark.parametrize("G", [1, 2, 4])
def test_attend_head_dim_256_column_tables(torch_dev, sq, G):
    """head_dim 256 values with widths of at most 6 bits take the column-table
    attend kernel with four 64-coordinate blocks per wave (the lane's four
    fields in one 64-bit window of record rows); compared on oracle records
    and random scores."""
    torch = torch_dev
    d, T, nkv = 256, 900, 2
    _case(f"attend d=256 column tables G={G} T={T}")
    X = np.stack([wl.flat_data(600, d, seed=50 + k) * np.linspace(3.0, 0.5, d) for k in range(nkv)])
    X = X.astype(np.float32)
    vcal = sq.sq_calibrate(X, 3.0, 0, None).upload()
    vors = [oracle.calibrate(X[k], 3.0, 0, None) for k in range(nkv)]
    for k in range(nkv):
        assert np.array_equal(vcal.export(k)["widths"], vors[k].widths)
    plan = sq.sq_plan_decode(None, vcal, 1, nkv * G, nkv, T)
    print(f"  max width {max(int(v.widths.max()) for v in vors)}; placement {plan.attend_placement}, "
          f"waves {plan.attend_waves}, blocks {plan.attend_blocks}", flush=True)
    assert plan.attend_placement == 0 and plan.attend_blocks == 4
    x = np.stack([wl.flat_data(T, d, seed=70 + k) * np.linspace(3.0, 0.5, d) for k in range(nkv)])
    x = wl.round_bf16(x)
    vp = np.zeros((1, nkv, vcal.packed_head_words(T)), np.uint32)
    rv = []
    for k in range(nkv):
        r = oracle.compress(vors[k], x[k])
        p = oracle.pack(vors[k].widths, 0, r.codes, r.z, r.gamma)
        vp[0, k, :len(p)] = p
        rv.append(r)
    s = (np.random.default_rng(19 + G).standard_normal((nkv * G, T)) * 16.0).astype(np.float32)
    scale = 1.0 / math.sqrt(d)
    ws = torch.zeros(sq.sq_attend_workspace_bytes(1, nkv * G, T, d) // 4 + 1, dtype=torch.float32,
                     device="cuda")
    out = torch.zeros((1, nkv * G, d), dtype=torch.float32, device="cuda")
    sq.sq_attend(vcal, torch.from_numpy(s[None].copy()).cuda(), scale,
                 torch.from_numpy(vp.view(np.int32)).cuda(), T, ws, out, nkv)
    torch.cuda.synchronize()
    o_gpu = out.cpu().numpy()[0]
    for k in range(nkv):
        ref = oracle.attend(vors[k], s[k * G:(k + 1) * G].astype(np.float64), scale, rv[k].codes)
        floor = np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(d)
        H.assert_close_floor(o_gpu[k * G:(k + 1) * G], ref, floor, f"attend d=256 G={G} head {k}")
