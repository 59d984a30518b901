"""GPU parity of the normalised calibrations (per-vector norm stored): the
TurboQuant-style baseline (random rotation, Gaussian Lloyd-Max codebook, QJL
over all dims for keys) and the normalised SpectralQuant variant, through the
same compress / scores / attend / dequantize / decode calls, against the
oracle's normalised pipeline on the same inputs."""
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


def _tq_handles(sq, cfg, heads, bits):
    d = cfg.head_dim
    rot = np.stack([wl.tq_rotation(cfg, l, h) for l, h in heads]).astype(np.float32)
    sk = np.stack([wl.tq_qjl(cfg, l, h) for l, h in heads]).astype(np.float32)
    kcal = sq.sq_calibrate_tq(rot, bits, True, sk).upload()
    vcal = sq.sq_calibrate_tq(rot, bits, False).upload()
    kors = [oracle.tq_calibration(rot[k].astype(np.float64), sk[k], bits, True) for k in range(len(heads))]
    vors = [oracle.tq_calibration(rot[k].astype(np.float64), None, bits, False) for k in range(len(heads))]
    return kcal, vcal, kors, vors


def _norm_handles(sq, cfg, heads, budget):
    Xk, Gk = H.calib_inputs(cfg, heads, "k")
    Xv, _ = H.calib_inputs(cfg, heads, "v")
    kcal = sq.sq_calibrate(Xk, budget, 1, Gk, normalize=True).upload()
    vcal = sq.sq_calibrate(Xv, budget, 0, None, normalize=True).upload()
    kors = [oracle.calibrate(Xk[k], budget, 1, Gk[k], normalize=True) for k in range(len(heads))]
    vors = [oracle.calibrate(Xv[k], budget, 0, None, normalize=True) for k in range(len(heads))]
    for k in range(len(heads)):
        assert np.array_equal(kcal.export(k)["widths"], kors[k].widths)
        assert np.array_equal(vcal.export(k)["widths"], vors[k].widths)
    return kcal, vcal, kors, vors


CASES = [
    # scheme, config, heads, T, bits / budget
    ("tq", "llama8b", [(0, h) for h in range(4)], 700, 3),
    ("tq", "qwen14b", [(5, h) for h in range(2)], 300, 4),
    ("tq", "gemma9b", [(0, 1), (0, 6)], 400, 3),
    ("tq", "tiny", [(0, 0), (2, 3)], 256, 3),
    ("norm", "llama8b", [(0, h) for h in range(4)], 700, 3.0),
    ("norm", "gemma9b", [(0, 2), (0, 5)], 400, 3.0),
    ("norm", "hd64", [(0, 1), (1, 2)], 300, 3.0),
]
IDS = [f"{c[0]}-{c[1]}" for c in CASES]


def _handles(sq, scheme, cfg, heads, b):
    return _tq_handles(sq, cfg, heads, b) if scheme == "tq" else _norm_handles(sq, cfg, heads, b)


@pytest.mark.parametrize("scheme,cfgname,heads,T,b", CASES, ids=IDS)
def test_normalized_compress_matches_oracle(torch_dev, sq, scheme, cfgname, heads, T, b):
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    _case(f"compress {scheme} {cfgname} T={T} b={b}")
    kcal, vcal, kors, vors = _handles(sq, scheme, cfg, heads, b)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    for which, cal, ors in (("k", kcal, kors), ("v", vcal, vors)):
        x = H.data_block(cfg, heads, which, T)
        xd = torch.from_numpy(x[None]).cuda().to(dt)
        packed = torch.full((1, len(heads), cal.packed_head_words(T)), -1, dtype=torch.int32, device="cuda")
        sq.sq_compress(cal, xd, packed)
        torch.cuda.synchronize()
        pk = packed.cpu().numpy().view(np.uint32)[0]
        tot = dict(band=0, flips=0, nu_ulp=0)
        for k in range(len(heads)):
            st, _ = H.compare_compress(ors[k], pk[k], x[k], T)
            for key in tot:
                tot[key] += st.get(key, 0)
        print(f"  {which}: in-band={tot['band']} flips={tot['flips']} nu-ulp={tot['nu_ulp']}", flush=True)
        assert tot["flips"] <= max(3, tot["band"] // 5)


def test_normalized_compress_bf16_head_dim_32(torch_dev, sq):
    """Normalised SpectralQuant heads of head_dim 32 with bf16 input: the grid
    kernel's normalised instance with two waves, whose per-token norm sums
    the partials of those two waves only.  The input is rounded to bf16 first
    and the oracle quantises the same rounded vectors; 300 tokens leave a
    ragged last tile."""
    torch = torch_dev
    cfg = wl.CONFIGS["tiny"]
    heads = [(0, 0), (1, 2), (2, 3)]
    T = 300
    _case(f"compress norm tiny bf16 T={T}")
    kcal, vcal, kors, vors = _norm_handles(sq, cfg, heads, 3.0)
    for which, cal, ors in (("k", kcal, kors), ("v", vcal, vors)):
        xd = torch.from_numpy(H.data_block(cfg, heads, which, T)[None]).cuda().to(torch.bfloat16)
        x = xd.float().cpu().numpy()[0].astype(np.float64)
        packed = torch.full((1, len(heads), cal.packed_head_words(T)), -1, dtype=torch.int32, device="cuda")
        sq.sq_compress(cal, xd, packed)
        torch.cuda.synchronize()
        pk = packed.cpu().numpy().view(np.uint32)[0]
        tot = dict(band=0, flips=0, nu_ulp=0)
        for k in range(len(heads)):
            st, _ = H.compare_compress(ors[k], pk[k], x[k], T)
            for key in tot:
                tot[key] += st.get(key, 0)
        print(f"  {which}: in-band={tot['band']} flips={tot['flips']} nu-ulp={tot['nu_ulp']}", flush=True)
        assert tot["flips"] <= max(3, tot["band"] // 5)


@pytest.mark.parametrize("scheme,cfgname,heads,T,b", CASES, ids=IDS)
def test_normalized_read_side_on_oracle_records(torch_dev, sq, scheme, cfgname, heads, T, b):
    """sq_scores, sq_attend, sq_dequantize (and sq_decode where it applies: QJL
    over at most 16 bits) on oracle-packed normalised records."""
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    nkv, G, d = len(heads), cfg.q_heads // cfg.kv_heads, cfg.head_dim
    _case(f"read side {scheme} {cfgname} T={T} b={b}")
    kcal, vcal, kors, vors = _handles(sq, scheme, cfg, heads, b)
    xk = H.data_block(cfg, heads, "k", T)
    xv = H.data_block(cfg, heads, "v", T)
    kp = np.zeros((1, nkv, kcal.packed_head_words(T)), np.uint32)
    vp = np.zeros((1, nkv, vcal.packed_head_words(T)), np.uint32)
    rk, rv = [], []
    for k in range(nkv):
        r = oracle.compress(kors[k], xk[k])
        p = oracle.pack(kors[k].widths, kors[k].m, r.codes, r.z, r.gamma, r.nu)
        kp[0, k, :len(p)] = p
        rk.append(r)
        r = oracle.compress(vors[k], xv[k])
        p = oracle.pack(vors[k].widths, 0, r.codes, r.z, r.gamma, r.nu)
        vp[0, k, :len(p)] = p
        rv.append(r)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    qd = torch.from_numpy(wl.queries(cfg, 1, nkv * G)).cuda().to(dt)
    q = qd.float().cpu().numpy().astype(np.float64)[0]
    kpd = torch.from_numpy(kp.view(np.int32)).cuda()
    vpd = torch.from_numpy(vp.view(np.int32)).cuda()
    scores = torch.zeros((1, nkv * G, T), dtype=torch.float32, device="cuda")
    sq.sq_scores(kcal, qd, kpd, T, scores, nkv)
    deq = torch.zeros((1, nkv, T, d), dtype=torch.float32, device="cuda")
    sq.sq_dequantize(kcal, kpd, T, deq)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()[0]
    deq_gpu = deq.cpu().numpy()[0]
    oscores = np.zeros((nkv * G, T))
    for k in range(nkv):
        oc, r = kors[k], rk[k]
        xt = oracle.dequantize(oc, r.codes, r.z, r.gamma, r.nu)
        H.assert_close_floor(deq_gpu[k], xt, np.linalg.norm(xt, axis=1)[:, None] / math.sqrt(d), f"dequantize {k}")
        qg = q[k * G:(k + 1) * G]
        ref = oracle.scores_rotated(oc, qg, r.codes, r.z, r.gamma, r.nu)
        oscores[k * G:(k + 1) * G] = ref
        H.assert_close_floor(s_gpu[k * G:(k + 1) * G], ref, H.score_floor(oc, qg, xt), f"scores {k}")
    scale = 1.0 / math.sqrt(d)
    s32 = oscores.astype(np.float32)
    ws = torch.zeros(sq.sq_attend_workspace_bytes(1, nkv * G, T, d) // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.zeros((1, nkv * G, d), dtype=torch.float32, device="cuda")
    sq.sq_attend(vcal, torch.from_numpy(s32[None].copy()).cuda(), scale, vpd, T, ws, out, nkv)
    torch.cuda.synchronize()
    o_gpu = out.cpu().numpy()[0]
    for k in range(nkv):
        ref = oracle.attend(vors[k], s32[k * G:(k + 1) * G].astype(np.float64), scale, rv[k].codes, rv[k].nu)
        H.assert_close_floor(o_gpu[k * G:(k + 1) * G], ref,
                             np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(d), f"attend {k}")
    # the fused step: keys whose QJL bits fit two words (m <= 16)
    fused = all(oc.m <= 16 for oc in kors)
    out2 = torch.zeros_like(out)
    if not fused:
        with pytest.raises(sq.SQError) as e:
            sq.sq_decode(kcal, vcal, qd, kpd, vpd, T, scale, ws, out2, nkv)
        assert e.value.status == 2
        print("  sq_decode: refused (QJL over more than 16 bits), as documented", flush=True)
        return
    sq.sq_decode(kcal, vcal, qd, kpd, vpd, T, scale, ws, out2, nkv)
    torch.cuda.synchronize()
    o2 = out2.cpu().numpy()[0]
    for k in range(nkv):
        ref = oracle.attend(vors[k], oscores[k * G:(k + 1) * G], scale, rv[k].codes, rv[k].nu)
        H.assert_close_floor(o2[k * G:(k + 1) * G], ref,
                             np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(d), f"decode {k}")
