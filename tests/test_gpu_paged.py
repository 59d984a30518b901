"""Paged packed cache on the GPU: sq_compress_append_paged writes the same
record words as the contiguous sq_compress_append (checked word for word
after gathering the pool through the block table on the host), and
sq_decode_paged over the pool gives sq_decode's output over the contiguous
slots bit for bit.  Blocks are handed out in a seeded random order; appends
come in pieces of unaligned length, including single tokens (the decode-step
producer)."""
import math
import sys

import numpy as np
import pytest

import harness as H
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


def _gather(pool, table, B, Hn, n_tiles, bt, block_words, W, slot_words):
    """Host gather of a pool into contiguous slots [B][H][slot_words]."""
    out = np.zeros((B, Hn, slot_words), np.uint32)
    for b in range(B):
        for t in range(n_tiles):
            blk = table[b, t // bt]
            for h in range(Hn):
                src = (blk * Hn + h) * block_words + (t % bt) * W * 64
                out[b, h, t * W * 64:(t + 1) * W * 64] = pool[src:src + W * 64]
    return out


PIECES = [700, 1, 1, 37, 1, 160, 100]   # 1000 tokens in unaligned pieces


@pytest.mark.parametrize("cfgname,budget,bt,quantiser", [
    ("llama8b", 3.0, 1, "grid"),
    ("llama8b", 3.0, 4, "tree"),
    ("qwen14b", 2.5, 3, "grid"),
    ("gemma9b", 3.0, 2, "grid"),
    ("hd64", 3.0, 2, "grid"),
])
def test_paged_append_and_decode_match_contiguous(torch_dev, sq, cfgname, budget, bt, quantiser, monkeypatch):
    torch = torch_dev
    monkeypatch.setenv("SQ_QUANTISER", quantiser)
    cfg = wl.CONFIGS[cfgname]
    B, Hkv = 3, 4
    Hq = Hkv * 2
    heads = [(0, h) for h in range(Hkv)]
    T = sum(PIECES)
    _case(f"paged {cfgname} bt={bt} quantiser={quantiser} T={T}")
    Xk, Gk = H.calib_inputs(cfg, heads, "k")
    Xv, _ = H.calib_inputs(cfg, heads, "v")
    kcal = sq.sq_calibrate(Xk, budget, 1, Gk).upload()
    vcal = sq.sq_calibrate(Xv, budget, 0, None).upload()
    d = cfg.head_dim
    dt = torch.bfloat16
    xk = np.stack([np.stack([wl.kv_block(cfg, 0, h, "k", T, "data", batch_index=b) for h in range(Hkv)])
                   for b in range(B)])
    xv = np.stack([np.stack([wl.kv_block(cfg, 0, h, "v", T, "data", batch_index=b) for h in range(Hkv)])
                   for b in range(B)])
    K = torch.from_numpy(xk.astype(np.float32)).cuda().to(dt)
    V = torch.from_numpy(xv.astype(np.float32)).cuda().to(dt)
    n_tiles = (T + 63) // 64
    nlb = (n_tiles + bt - 1) // bt
    n_blocks = B * nlb + 5
    rng = np.random.default_rng(11)
    table = rng.permutation(n_blocks)[:B * nlb].reshape(B, nlb).astype(np.int32)
    table_d = torch.from_numpy(table).cuda()
    pg = sq.paged(table_d, bt, n_blocks)
    out = {}
    for name, cal, X in (("k", kcal, K), ("v", vcal, V)):
        W = cal.info(0).record_words
        Wm = max(cal.info(h).record_words for h in range(Hkv))
        slot = cal.packed_head_words(T)
        cont = torch.zeros((B, Hkv, slot), dtype=torch.int32, device="cuda")
        bw = sq.sq_paged_block_words(cal, bt)
        assert bw == bt * 64 * Wm
        pool = torch.full((n_blocks * Hkv * bw,), -1, dtype=torch.int32, device="cuda")
        t0 = 0
        for n in PIECES:
            piece = X[:, :, t0:t0 + n, :]
            sq.sq_compress_append(cal, piece, cont, t0)
            sq.sq_compress_append_paged(cal, piece, pool, pg, t0)
            t0 += n
        torch.cuda.synchronize()
        c = cont.cpu().numpy().view(np.uint32)
        p = pool.cpu().numpy().view(np.uint32)
        for h in range(Hkv):
            Wh = cal.info(h).record_words
            g = _gather(p, table, B, Hkv, n_tiles, bt, bw, Wh, n_tiles * Wh * 64)
            np.testing.assert_array_equal(g[:, h], c[:, h, :n_tiles * Wh * 64], err_msg=f"{name} head {h}")
        # blocks nobody owns stay untouched
        used = set(table.ravel().tolist())
        for blk in range(n_blocks):
            if blk not in used:
                assert (p[blk * Hkv * bw:(blk + 1) * Hkv * bw] == 0xFFFFFFFF).all()
        out[name] = (cont, pool)
    q = torch.from_numpy(wl.queries(cfg, B, Hq)).cuda().to(dt)
    ws = torch.empty(sq.sq_attend_workspace_bytes(B, Hq, T, d) // 4 + 1, dtype=torch.float32, device="cuda")
    o1 = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)
    scale = 1 / math.sqrt(d)
    try:
        sq.sq_decode(kcal, vcal, q, out["k"][0], out["v"][0], T, scale, ws, o1, Hkv)
    except sq.SQError as e:
        if e.status == 2:
            pytest.skip(f"sq_decode unsupported for {cfgname}: {e}")
        raise
    sq.sq_decode_paged(kcal, vcal, q, out["k"][1], out["v"][1], pg, T, scale, ws, o2, Hkv)
    torch.cuda.synchronize()
    a, b = o1.cpu().numpy(), o2.cpu().numpy()
    assert np.isfinite(a).all()
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("cfgname,scheme", [("llama8b", "norm"), ("hd64", "norm"), ("llama8b", "tq")])
def test_paged_normalized_append_matches_oracle(torch_dev, sq, cfgname, scheme):
    """Normalised records (the normalised SpectralQuant variant, and the
    TurboQuant-style keys and values) appended in unaligned pieces to a paged
    pool go through the general compress kernel's paged instances; the
    gathered records are compared with the oracle's under the acceptance
    rules (vector norms included)."""
    import oracle
    torch = torch_dev
    cfg = wl.CONFIGS[cfgname]
    B, Hkv, bt = 2, 2, 3
    heads = [(0, h) for h in range(Hkv)]
    T = sum(PIECES)
    d = cfg.head_dim
    _case(f"paged normalised {scheme} {cfgname} bt={bt} T={T}")
    if scheme == "norm":
        Xk, Gk = H.calib_inputs(cfg, heads, "k")
        Xv, _ = H.calib_inputs(cfg, heads, "v")
        kcal = sq.sq_calibrate(Xk, 3.0, 1, Gk, normalize=True).upload()
        vcal = sq.sq_calibrate(Xv, 3.0, 0, None, normalize=True).upload()
        kors = [oracle.calibrate(Xk[k], 3.0, 1, Gk[k], normalize=True) for k in range(Hkv)]
        vors = [oracle.calibrate(Xv[k], 3.0, 0, None, normalize=True) for k in range(Hkv)]
    else:
        rot = np.stack([wl.tq_rotation(cfg, l, h) for l, h in heads]).astype(np.float32)
        sk = np.stack([wl.tq_qjl(cfg, l, h) for l, h in heads]).astype(np.float32)
        kcal = sq.sq_calibrate_tq(rot, 3, True, sk).upload()
        vcal = sq.sq_calibrate_tq(rot, 3, False).upload()
        kors = [oracle.tq_calibration(rot[k].astype(np.float64), sk[k], 3, True) for k in range(Hkv)]
        vors = [oracle.tq_calibration(rot[k].astype(np.float64), None, 3, False) for k in range(Hkv)]
    n_tiles = (T + 63) // 64
    nlb = (n_tiles + bt - 1) // bt
    n_blocks = B * nlb + 3
    table = np.random.default_rng(5).permutation(n_blocks)[:B * nlb].reshape(B, nlb).astype(np.int32)
    table_d = torch.from_numpy(table).cuda()
    pg = sq.paged(table_d, bt, n_blocks)
    for which, cal, ors in (("k", kcal, kors), ("v", vcal, vors)):
        x = np.stack([np.stack([wl.kv_block(cfg, 0, h, which, T, "data", batch_index=b) for h in range(Hkv)])
                      for b in range(B)])
        X = torch.from_numpy(x.astype(np.float32)).cuda().to(torch.bfloat16)
        xr = X.float().cpu().numpy().astype(np.float64)  # the bf16 values both sides quantise
        bw = sq.sq_paged_block_words(cal, bt)
        pool = torch.full((n_blocks * Hkv * bw,), -1, dtype=torch.int32, device="cuda")
        t0 = 0
        for n in PIECES:
            sq.sq_compress_append_paged(cal, X[:, :, t0:t0 + n, :], pool, pg, t0)
            t0 += n
        torch.cuda.synchronize()
        p = pool.cpu().numpy().view(np.uint32)
        tot = dict(band=0, flips=0)
        for h in range(Hkv):
            Wh = cal.info(h).record_words
            g = _gather(p, table, B, Hkv, n_tiles, bt, bw, Wh, n_tiles * Wh * 64)
            for b in range(B):
                st, _ = H.compare_compress(ors[h], g[b, h], xr[b, h], T)
                for key in tot:
                    tot[key] += st[key]
        print(f"  {which}: in-band={tot['band']} flips={tot['flips']}", flush=True)
        assert tot["flips"] <= max(3, tot["band"] // 5)


def test_paged_argument_errors_and_bad_block_ids(torch_dev, sq):
    torch = torch_dev
    cfg = wl.CONFIGS["llama8b"]
    heads = [(0, 0), (0, 1)]
    X, G = H.calib_inputs(cfg, heads, "k")
    cal = sq.sq_calibrate(X, 3.0, 1, G).upload()
    _case("paged errors")
    x = torch.from_numpy(np.stack([wl.kv_block(cfg, 0, h, "k", 200, "data") for _, h in heads])[None]
                         .astype(np.float32)).cuda().to(torch.bfloat16)
    bw = sq.sq_paged_block_words(cal, 1)
    table = torch.tensor([[0, 1, 2]], dtype=torch.int32, device="cuda")   # 4 tiles needed
    pool = torch.zeros((4 * 2 * bw,), dtype=torch.int32, device="cuda")
    with pytest.raises(sq.SQError) as e:
        sq.sq_compress_append_paged(cal, x, pool, sq.paged(table, 1, 4), 0)
    assert e.value.status == 1 and "table_stride" in str(e.value)
    with pytest.raises(sq.SQError) as e:
        sq.sq_compress_append_paged(cal, x, pool, sq.paged(table, 0, 4), 0)
    assert e.value.status == 1
    # an id outside [0, n_blocks) is never written: its tile's words are dropped
    table = torch.tensor([[0, 7, 2, 3]], dtype=torch.int32, device="cuda")
    pool.fill_(-1)
    sq.sq_compress_append_paged(cal, x, pool, sq.paged(table, 1, 4), 0)
    torch.cuda.synchronize()
    p = pool.cpu().numpy().view(np.uint32)
    assert (p[1 * 2 * bw:2 * 2 * bw] == 0xFFFFFFFF).all()          # block 1: nobody's
    assert not (p[0:2 * bw] == 0xFFFFFFFF).all()                    # block 0: written
    assert sq.sq_paged_block_words(cal, 0) == -1
