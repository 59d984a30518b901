"""GPU parity of sq_decode, the fused decode step (scores, online softmax and
value sum in one pass, no score tensor): against the oracle on oracle-packed
key and value records for every workload (query groups of 2, 4, 5 and 8
heads, head_dim 32/128/256, ragged tails), plus empty and one-token inputs and
argument errors.  The full decode size is covered in test_gpu_fullsize.py."""
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


CASES = [
    # name, config, heads, T, budget
    ("tiny", "tiny", [(l, h) for l in range(3) for h in range(4)], 256, 3.0),
    ("llama8b", "llama8b", [(0, h) for h in range(8)], 2048, 3.0),
    ("llama8b-ragged", "llama8b", [(0, h) for h in range(2)], 1000, 3.0),
    ("llama8b-one-token", "llama8b", [(0, 3), (0, 4)], 1, 3.0),
    ("qwen14b-2.5b", "qwen14b", [(l, h) for l in (0, 47) for h in range(8)], 512, 2.5),
    ("qwen14b-3.5b", "qwen14b", [(l, h) for l in (1,) for h in range(8)], 1024, 3.5),
    ("gemma9b", "gemma9b", [(l, h) for l in (0,) for h in range(4)], 700, 3.0),
    ("hd64", "hd64", [(l, h) for l in range(2) for h in range(4)], 700, 3.0),
]


def _oracle_records(cfg, heads, T, budget, kcal_sq, vcal_sq, kors, vors):
    nkv = len(heads)
    xk = H.data_block(cfg, heads, "k", T)
    xv = H.data_block(cfg, heads, "v", T)
    kp = np.zeros((1, nkv, kcal_sq.packed_head_words(T)), np.uint32)
    vp = np.zeros((1, nkv, vcal_sq.packed_head_words(T)), np.uint32)
    rk, rv = [], []
    for k in range(nkv):
        r = oracle.compress(kors[k], xk[k])
        p = oracle.pack(kors[k].widths, kors[k].m, r.codes, r.z, r.gamma)
        kp[0, k, :len(p)] = p
        rk.append(r)
        r = oracle.compress(vors[k], xv[k])
        p = oracle.pack(vors[k].widths, 0, r.codes, r.z, r.gamma)
        vp[0, k, :len(p)] = p
        rv.append(r)
    return kp, vp, rk, rv


@pytest.mark.parametrize("name,cfgname,heads,T,budget", CASES, ids=[c[0] for c in CASES])
def test_decode_on_oracle_records(torch_dev, sq, name, cfgname, heads, T, budget):
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    nkv = len(heads)
    G = cfg.q_heads // cfg.kv_heads
    d = cfg.head_dim
    _case(f"sq_decode {name} T={T} G={G} d={d}")
    kcal, kors = H.calibrate_both(sq, cfg, heads, "k", budget, n_tokens=max(T, 256))
    vcal, vors = H.calibrate_both(sq, cfg, heads, "v", budget, n_tokens=max(T, 256))
    kcal.upload()
    vcal.upload()
    plan = sq.sq_plan_decode(kcal, vcal, 1, nkv * G, nkv, T)
    print(f"  plan: {plan.decode_launches} launch(es), {plan.decode_waves} waves, "
          f"{plan.decode_lds_bytes} B LDS; value tables {plan.attend_placement}", flush=True)
    assert plan.decode_launches == -(-G // 4)
    kp, vp, rk, rv = _oracle_records(cfg, heads, T, budget, kcal, vcal, kors, vors)
    q = wl.queries(cfg, 1, nkv * G)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    qd = torch.from_numpy(q).cuda().to(dt)
    q_used = qd.float().cpu().numpy().astype(np.float64)[0]
    scale = 1.0 / math.sqrt(d)
    ws = torch.empty(sq.sq_attend_workspace_bytes(1, nkv * G, T, d) // 4, dtype=torch.float32,
                     device="cuda")
    out = torch.full((1, nkv * G, d), float("nan"), dtype=torch.float32, device="cuda")
    sq.sq_decode(kcal, vcal, qd, torch.from_numpy(kp.view(np.int32)).cuda(),
                 torch.from_numpy(vp.view(np.int32)).cuda(), T, scale, ws, out, nkv)
    torch.cuda.synchronize()
    o = out.cpu().numpy()[0]
    worst = 0.0
    for k in range(nkv):
        qg = q_used[k * G:(k + 1) * G]
        s = oracle.scores_rotated(kors[k], qg, rk[k].codes, rk[k].z, rk[k].gamma)
        ref = oracle.attend(vors[k], s, scale, rv[k].codes)
        floor = np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(d)
        worst = max(worst, H.assert_close_floor(o[k * G:(k + 1) * G], ref, floor, f"decode head {k}"))
    print(f"  worst err/tol {worst:.3g}", flush=True)


def test_decode_empty_and_errors(torch_dev, sq):
    torch = torch_dev
    cfg = wl.CONFIGS["llama8b"]
    heads = [(0, 0), (0, 1)]
    _case("sq_decode T=0 and argument errors")
    kcal, _ = H.calibrate_both(sq, cfg, heads, "k", 3.0)
    vcal, _ = H.calibrate_both(sq, cfg, heads, "v", 3.0)
    kcal.upload()
    vcal.upload()
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((1, 2, kcal.packed_head_words(100)), dtype=torch.int32, device="cuda")
    vp = torch.zeros((1, 2, vcal.packed_head_words(100)), dtype=torch.int32, device="cuda")
    out = torch.full((1, 8, 128), 3.0, dtype=torch.float32, device="cuda")
    ws = torch.zeros(4, dtype=torch.float32, device="cuda")
    sq.sq_decode(kcal, vcal, q, kp, vp, 0, 1.0, ws, out, 2)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 0.0))
    out.fill_(3.0)
    with pytest.raises(sq.SQError) as e:  # workspace too small
        sq.sq_decode(kcal, vcal, q, kp, vp, 100, 1.0, ws, out, 2)
    assert e.value.status == 1
    with pytest.raises(sq.SQError) as e:  # values handle as keys: fine; 7 q heads over 2 KV heads: not
        sq.sq_decode(kcal, vcal, torch.zeros((1, 7, 128), dtype=torch.bfloat16, device="cuda"), kp, vp, 100,
                     1.0, ws, torch.zeros((1, 7, 128), dtype=torch.float32, device="cuda"), 2)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0))


@pytest.mark.parametrize("cfgname,heads,T", [("llama8b", [(0, h) for h in range(8)], 3000),
                                             ("gemma9b", [(0, 1), (0, 6)], 900)])
def test_decode_agrees_with_scores_then_attend(torch_dev, sq, cfgname, heads, T):
    """Consistency of the two read paths on GPU-compressed records: sq_decode
    and sq_scores followed by sq_attend give the same output to the parity
    tolerance (their score arithmetic differs: fp32 tables vs bf16x3 MFMA)."""
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    nkv, G, d = len(heads), cfg.q_heads // cfg.kv_heads, cfg.head_dim
    _case(f"sq_decode vs sq_scores + sq_attend {cfgname} T={T}")
    kcal, _ = H.calibrate_both(sq, cfg, heads, "k", 3.0)
    vcal, _ = H.calibrate_both(sq, cfg, heads, "v", 3.0)
    kcal.upload()
    vcal.upload()
    xk = torch.from_numpy(H.data_block(cfg, heads, "k", T)[None]).cuda().to(torch.bfloat16)
    xv = torch.from_numpy(H.data_block(cfg, heads, "v", T)[None]).cuda().to(torch.bfloat16)
    kp = torch.zeros((1, nkv, kcal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    vp = torch.zeros((1, nkv, vcal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    sq.sq_compress(kcal, xk, kp)
    sq.sq_compress(vcal, xv, vp)
    q = torch.from_numpy(wl.queries(cfg, 1, nkv * G)).cuda().to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    ws = torch.empty(sq.sq_attend_workspace_bytes(1, nkv * G, T, d) // 4, dtype=torch.float32, device="cuda")
    s = torch.empty((1, nkv * G, T), dtype=torch.float32, device="cuda")
    o1 = torch.empty((1, nkv * G, d), dtype=torch.float32, device="cuda")
    o2 = torch.empty((1, nkv * G, d), dtype=torch.float32, device="cuda")
    sq.sq_scores(kcal, q, kp, T, s, nkv)
    sq.sq_attend(vcal, s, scale, vp, T, ws, o1, nkv)
    sq.sq_decode(kcal, vcal, q, kp, vp, T, scale, ws, o2, nkv)
    torch.cuda.synchronize()
    a, b = o1.cpu().numpy()[0], o2.cpu().numpy()[0]
    floor = np.linalg.norm(a, axis=1, keepdims=True) / math.sqrt(d)
    worst = H.assert_close_floor(b, a, floor, "decode vs scores+attend")
    print(f"  worst err/tol {worst:.3g}", flush=True)
