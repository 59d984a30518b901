"""sq_attend_noalloc (partials in the library's fixed device scratch, nothing
allocated) against sq_attend (caller workspace) through the C ABI: the same
kernels, so the outputs must be identical bit for bit; two calls in a row,
the second smaller, so the second runs over the first one's scratch
contents.  A call whose partials exceed the scratch is refused before
anything is enqueued."""
import math
import sys

import numpy as np
import pytest

import harness as H
import workloads as wl

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import compression_sq_compress_amd as sq
    return torch, sq


def _inputs(torch, sq, cfg, heads, B, T, seed):
    nkv = len(heads)
    G = cfg.q_heads // cfg.kv_heads
    X = np.stack([wl.calibration_set(cfg, l, h, "v") for l, h in heads]).astype(np.float32)
    vcal = sq.sq_calibrate(X, 3.0, 0, None).upload()
    x = np.stack([np.stack([wl.kv_block(cfg, l, h, "v", T, "data", batch_index=b) for l, h in heads])
                  for b in range(B)])
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    vp = torch.zeros((B, nkv, vcal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    sq.sq_compress(vcal, xd, vp)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    s = torch.randn((B, nkv * G, T), generator=g, device="cuda") * 12.0
    return vcal, vp, s, nkv, G


@pytest.mark.parametrize("cfgname,heads,B,T", [
    ("llama8b", [(0, h) for h in range(8)], 3, 5000),   # first call: larger
    ("gemma9b", [(0, h) for h in range(2)], 1, 700),    # second call: smaller, head_dim 256
    ("llama8b", [(0, 1), (0, 4)], 2, 130),              # third: smaller still
])
def test_noalloc_matches_workspace_attend(env, cfgname, heads, B, T):
    torch, sq = env
    cfg = wl.CONFIGS[cfgname]
    _case(f"sq_attend_noalloc vs sq_attend {cfgname} B={B} H={len(heads)} T={T}")
    vcal, vp, s, nkv, G = _inputs(torch, sq, cfg, heads, B, T, seed=T)
    d = cfg.head_dim
    scale = 1.0 / math.sqrt(d)
    ws = torch.empty(sq.sq_attend_workspace_bytes(B, nkv * G, T, d) // 4, dtype=torch.float32,
                     device="cuda")
    out_ws = torch.full((B, nkv * G, d), float("nan"), dtype=torch.float32, device="cuda")
    out_na = torch.full((B, nkv * G, d), float("nan"), dtype=torch.float32, device="cuda")
    sq.sq_attend(vcal, s, scale, vp, T, ws, out_ws, nkv)
    sq.sq_attend_noalloc(vcal, s, scale, vp, T, out_na, nkv)
    torch.cuda.synchronize()
    a, b = out_ws.cpu().numpy(), out_na.cpu().numpy()
    assert np.all(np.isfinite(a))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_noalloc_refuses_partials_beyond_the_scratch(env):
    torch, sq = env
    cfg = wl.CONFIGS["decode"]
    B, Hkv, Hq, d, T = 64, 8, 32, 128, 65536
    _case(f"sq_attend_noalloc over the scratch limit B={B} T={T}")
    need = sq.sq_attend_workspace_bytes(B, Hq, T, d)
    assert need > 32 << 20
    X = np.stack([wl.calibration_set(cfg, 0, h, "v") for h in range(Hkv)]).astype(np.float32)
    vcal = sq.sq_calibrate(X, 3.0, 0, None).upload()
    vp = torch.zeros((B, Hkv, vcal.packed_head_words(T)), dtype=torch.int32, device="cuda")
    s = torch.zeros((B, Hq, T), dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, d), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(sq.SQError) as e:
        sq.sq_attend_noalloc(vcal, s, 1.0, vp, T, out, Hkv)
    assert e.value.status == 2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
