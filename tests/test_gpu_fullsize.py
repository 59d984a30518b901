"""GPU parity at the full decode size, in the launch configuration the
benchmark times: 64 sequences x 8 KV heads x 32768 tokens, hd128, bf16,
3 bits, keys with 1 QJL bit per signal dimension, 32 query heads.

The whole batch goes through sq_compress / sq_scores / sq_attend; sampled
(sequence, KV head) slots are then checked against the oracle over all their
32768 tokens: records under the code/QJL/gamma acceptance rules, scores on
the tokens whose key record matches the oracle's, and the attention output
for a slot whose scores and value records were replaced by the oracle's own.
"""
import math
import sys

import numpy as np
import pytest

import harness as H
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

SLOTS = [(0, 0), (37, 5), (63, 7)]


def _case(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def full(request):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import compression_sq_compress_amd as sq
    cfg = wl.CONFIGS["decode"]
    B, T, Hkv, Hq, d = cfg.batch, cfg.tokens[0], cfg.kv_heads, cfg.q_heads, cfg.head_dim
    _case(f"full-size decode setup B={B} T={T} Hkv={Hkv} Hq={Hq} d={d}")
    Xk = np.stack([wl.calibration_set(cfg, 0, h, "k") for h in range(Hkv)]).astype(np.float32)
    Gk = np.stack([wl.qjl_gaussian(cfg, 0, h) for h in range(Hkv)])
    Xv = np.stack([wl.calibration_set(cfg, 0, h, "v") for h in range(Hkv)]).astype(np.float32)
    kcal = sq.sq_calibrate(Xk, 3.0, 1, Gk).upload()
    vcal = sq.sq_calibrate(Xv, 3.0, 0, None).upload()
    kors = [oracle.calibrate(Xk[h], 3.0, 1, Gk[h]) for h in range(Hkv)]
    vors = [oracle.calibrate(Xv[h], 3.0, 0, None) for h in range(Hkv)]
    K = wl.decode_kv_on_device(cfg, "k")
    V = wl.decode_kv_on_device(cfg, "v")
    q = wl.queries(cfg, B, Hq)
    qd = torch.from_numpy(q).cuda().to(torch.bfloat16)
    q_used = qd.float().cpu().numpy().astype(np.float64)      # the bf16 values the GPU sees
    kp = torch.full((B, Hkv, kcal.packed_head_words(T)), -1, dtype=torch.int32, device="cuda")
    vp = torch.full((B, Hkv, vcal.packed_head_words(T)), -1, dtype=torch.int32, device="cuda")
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(sq.sq_attend_workspace_bytes(B, Hq, T, d) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    sq.sq_compress(kcal, K, kp)
    sq.sq_compress(vcal, V, vp)
    sq.sq_scores(kcal, qd, kp, T, scores, Hkv)
    sq.sq_attend(vcal, scores, 1.0 / math.sqrt(d), vp, T, ws, out, Hkv)
    torch.cuda.synchronize()
    return dict(torch=torch, sq=sq, cfg=cfg, kcal=kcal, vcal=vcal, kors=kors, vors=vors, K=K, V=V,
                q=q_used, qd=qd, kp=kp, vp=vp, scores=scores, ws=ws, out=out, B=B, T=T, Hkv=Hkv,
                Hq=Hq, d=d)


@pytest.mark.parametrize("slot", SLOTS, ids=[f"b{b}h{h}" for b, h in SLOTS])
def test_fullsize_compress_and_scores(full, slot):
    b, h = slot
    f = full
    T, G = f["T"], f["Hq"] // f["Hkv"]
    _case(f"full-size compress+scores slot b={b} h={h}")
    xk = f["K"][b, h].float().cpu().numpy()
    xv = f["V"][b, h].float().cpu().numpy()
    kslot = f["kp"][b, h].cpu().numpy().view(np.uint32)
    vslot = f["vp"][b, h].cpu().numpy().view(np.uint32)
    sk, rk = H.compare_compress(f["kors"][h], kslot, xk, T)
    sv, _ = H.compare_compress(f["vors"][h], vslot, xv, T)
    print(f"  keys: in-band={sk['band']} flips={sk['flips']} qjl_flips={sk['qjl_flips']}; "
          f"values: in-band={sv['band']} flips={sv['flips']}", flush=True)
    # slot words beyond the padded token range are untouched (sentinel -1)
    Tp = -(-T // 64) * 64
    assert np.all(kslot[Tp * f["kors"][h].W:] == 0xFFFFFFFF) or Tp * f["kors"][h].W == kslot.size
    oc = f["kors"][h]
    gc, gz, _ = oracle.unpack(oc.widths, oc.m, kslot, T)
    same = (gc == rk.codes).all(axis=1) & (gz == rk.z).all(axis=1)
    qg = f["q"][b, h * G:(h + 1) * G]
    ref = oracle.scores_rotated(oc, qg, rk.codes, rk.z, rk.gamma)
    xt = oracle.dequantize(oc, rk.codes, rk.z, rk.gamma)
    fl = H.score_floor(oc, qg, xt)
    s_gpu = f["scores"][b, h * G:(h + 1) * G].cpu().numpy()
    worst = H.assert_close_floor(s_gpu[:, same], ref[:, same], fl[:, same], f"scores b={b} h={h}")
    print(f"  scores: {int(same.sum())}/{T} tokens compared, worst err/tol {worst:.3g}", flush=True)
    assert same.sum() >= T - max(8, sk["flip_tokens"] + 8)


def test_fullsize_attend_on_oracle_inputs(full):
    """Replace one slot's scores and value records with the oracle's, run
    sq_attend over the whole batch, compare that slot's outputs."""
    f = full
    torch = f["torch"]
    b, h = 21, 3
    T, G, d = f["T"], f["Hq"] // f["Hkv"], f["d"]
    _case(f"full-size attend slot b={b} h={h}")
    cfg = f["cfg"]
    xk = f["K"][b, h].float().cpu().numpy()
    xv = f["V"][b, h].float().cpu().numpy()
    rk = oracle.compress(f["kors"][h], xk)
    rv = oracle.compress(f["vors"][h], xv)
    qg = f["q"][b, h * G:(h + 1) * G]
    s_ref = oracle.scores_rotated(f["kors"][h], qg, rk.codes, rk.z, rk.gamma).astype(np.float32)
    vrec = oracle.pack(f["vors"][h].widths, 0, rv.codes, rv.z, rv.gamma)
    scores = f["scores"].clone()
    vp = f["vp"].clone()
    scores[b, h * G:(h + 1) * G] = torch.from_numpy(s_ref).cuda()
    vp[b, h, :vrec.size] = torch.from_numpy(vrec.view(np.int32)).cuda()
    out = torch.empty_like(f["out"])
    scale = 1.0 / math.sqrt(d)
    f["sq"].sq_attend(f["vcal"], scores, scale, vp, T, f["ws"], out, f["Hkv"])
    torch.cuda.synchronize()
    o = out[b, h * G:(h + 1) * G].cpu().numpy()
    ref = oracle.attend(f["vors"][h], s_ref.astype(np.float64), scale, rv.codes)
    floor = np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(d)
    worst = H.assert_close_floor(o, ref, floor, "full-size attend")
    print(f"  attend worst err/tol {worst:.3g}", flush=True)
    allout = out.cpu().numpy()
    assert np.all(np.isfinite(allout))
    # every other slot is unchanged by the substitution
    mask = np.ones(allout.shape[:2], bool)
    mask[b, h * G:(h + 1) * G] = False
    assert np.array_equal(allout[mask], f["out"].cpu().numpy()[mask])


def test_fullsize_attend_outputs_are_convex_combinations(full):
    """Property at any size: the output of every (sequence, query head), rotated
    back into the value eigenbasis, lies inside the per-coordinate range of the
    centroids (a softmax-weighted mean of centroids)."""
    f = full
    _case("full-size attend range property")
    out = f["out"].cpu().numpy().astype(np.float64)
    G = f["Hq"] // f["Hkv"]
    for h in range(f["Hkv"]):
        oc = f["vors"][h]
        y = out[:, h * G:(h + 1) * G] @ oc.R.T          # rotated outputs [B][G][d]
        lo = np.array([c.min() if len(c) else 0.0 for c in oc.centroids])
        hi = np.array([c.max() if len(c) else 0.0 for c in oc.centroids])
        slack = 1e-3 * (np.abs(lo) + np.abs(hi)) + 1e-3 * oc.sigma[0]
        assert np.all(y >= lo - slack) and np.all(y <= hi + slack), f"head {h}"


def test_fullsize_decode_on_oracle_inputs(full):
    """sq_decode over the whole decode batch, in the launch configuration the
    benchmark times, with one slot's key and value records replaced by the
    oracle's; that slot's outputs against oracle.attend on oracle scores."""
    f = full
    torch = f["torch"]
    b, h = 45, 6
    T, G, d = f["T"], f["Hq"] // f["Hkv"], f["d"]
    _case(f"full-size sq_decode slot b={b} h={h}")
    xk = f["K"][b, h].float().cpu().numpy()
    xv = f["V"][b, h].float().cpu().numpy()
    rk = oracle.compress(f["kors"][h], xk)
    rv = oracle.compress(f["vors"][h], xv)
    krec = oracle.pack(f["kors"][h].widths, f["kors"][h].m, rk.codes, rk.z, rk.gamma)
    vrec = oracle.pack(f["vors"][h].widths, 0, rv.codes, rv.z, rv.gamma)
    kp = f["kp"].clone()
    vp = f["vp"].clone()
    kp[b, h, :krec.size] = torch.from_numpy(krec.view(np.int32)).cuda()
    vp[b, h, :vrec.size] = torch.from_numpy(vrec.view(np.int32)).cuda()
    out = torch.empty_like(f["out"])
    scale = 1.0 / math.sqrt(d)
    f["sq"].sq_decode(f["kcal"], f["vcal"], f["qd"], kp, vp, T, scale, f["ws"], out, f["Hkv"])
    torch.cuda.synchronize()
    o = out[b, h * G:(h + 1) * G].cpu().numpy()
    qg = f["q"][b, h * G:(h + 1) * G]
    s = oracle.scores_rotated(f["kors"][h], qg, rk.codes, rk.z, rk.gamma)
    ref = oracle.attend(f["vors"][h], s, scale, rv.codes)
    floor = np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(d)
    worst = H.assert_close_floor(o, ref, floor, "full-size decode")
    print(f"  decode worst err/tol {worst:.3g}", flush=True)
    allout = out.cpu().numpy()
    assert np.all(np.isfinite(allout))
    # the other slots against the split path on the same records, to the parity tolerance
    ref_all = f["out"].cpu().numpy()
    mask = np.ones(allout.shape[:2], bool)
    mask[b, h * G:(h + 1) * G] = False
    fl = np.linalg.norm(ref_all[mask], axis=1, keepdims=True) / math.sqrt(d)
    H.assert_close_floor(allout[mask], ref_all[mask], fl, "full-size decode vs scores + attend")
