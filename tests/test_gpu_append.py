"""Incremental append (sq_compress_append), the decode-time producer of the
packed cache.  A token's record depends only on its own vector, so appending
a sequence in pieces at arbitrary token offsets must leave exactly the words
one sq_compress over the whole sequence writes; the records must match the
oracle; and words outside the written range must stay as they were."""
import sys

import numpy as np
import pytest

import harness as H
import workloads as wl

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A


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


def _dev(torch, a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(dtype)


def _token_index(W, t):
    """Word offsets of token t's W record words in a slot."""
    return ((t // 64) * W + np.arange(W)) * 64 + t % 64


# (config, heads, which, T, pieces, dtype): pieces cut [0, T) in order; they
# cover unaligned starts, single tokens, pieces longer than a tile and pieces
# that cross tile boundaries, on both compress kernels (head_dim <= 128 and 256)
CASES = [
    ("llama8b", [(0, 0), (0, 3)], "k", 200, [100, 1, 37, 1, 1, 60], "bf16"),
    ("llama8b", [(0, 1)], "v", 131, [1, 1, 62, 1, 65, 1], "bf16"),
    ("qwen14b", [(7, 2), (7, 5)], "k", 96, [33, 31, 1, 31], "bf16"),
    ("gemma9b", [(0, 0)], "k", 150, [70, 1, 79], "bf16"),
    ("tiny", [(0, 0), (1, 2)], "k", 100, [5, 59, 1, 35], "f32"),
]


@pytest.mark.parametrize("cfgname,heads,which,T,pieces,dt", CASES)
def test_append_in_pieces_equals_whole(torch_dev, sq, cfgname, heads, which, T, pieces, dt):
    torch = torch_dev
    assert sum(pieces) == T
    _case(f"append {cfgname} {which} T={T} pieces={pieces} {dt}")
    cfg = wl.CONFIGS[cfgname]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    budget = cfg.budgets[0]
    cal, ors = H.calibrate_both(sq, cfg, heads, which, budget)
    cal.upload()
    x = H.data_block(cfg, heads, which, T)
    xd = _dev(torch, x[None], tdt)
    nh, words = len(heads), cal.packed_head_words(T)
    whole = torch.zeros((1, nh, words), dtype=torch.int32, device="cuda")
    sq.sq_compress(cal, xd, whole)
    inc = torch.full((1, nh, words), SENTINEL, dtype=torch.int32, device="cuda")
    t0 = 0
    for n in pieces:
        sq.sq_compress_append(cal, xd[:, :, t0:t0 + n], inc, t0)
        t0 += n
    torch.cuda.synchronize()
    wn = whole.cpu().numpy().view(np.uint32)[0]
    gn = inc.cpu().numpy().view(np.uint32)[0]
    n_tiles = -(-T // 64)
    for k in range(nh):
        W = ors[k].W
        used = n_tiles * 64 * W
        assert np.array_equal(gn[k, :used], wn[k, :used]), f"head {k}: appended words differ"
        assert np.all(gn[k, used:] == SENTINEL), f"head {k}: words past the last tile written"
        H.compare_compress(ors[k], gn[k], x[k], T)


def test_append_touches_only_its_range(torch_dev, sq):
    torch = torch_dev
    _case("append llama8b k: 5 tokens at token0=70 into a filled slot")
    cfg = wl.CONFIGS["llama8b"]
    heads = [(0, 2)]
    cal, ors = H.calibrate_both(sq, cfg, heads, "k", 3.0)
    cal.upload()
    T = 200
    x = H.data_block(cfg, heads, "k", T)
    xd = _dev(torch, x[None], torch.bfloat16)
    words = cal.packed_head_words(T)
    whole = torch.zeros((1, 1, words), dtype=torch.int32, device="cuda")
    sq.sq_compress(cal, xd, whole)
    slot = torch.full((1, 1, words), SENTINEL, dtype=torch.int32, device="cuda")
    sq.sq_compress_append(cal, xd[:, :, 70:75], slot, 70)
    torch.cuda.synchronize()
    wn = whole.cpu().numpy().view(np.uint32)[0, 0]
    gn = slot.cpu().numpy().view(np.uint32)[0, 0]
    W = ors[0].W
    written = np.zeros(words, dtype=bool)
    for t in range(64, 128):
        ix = _token_index(W, t)
        if 70 <= t < 75:
            assert np.array_equal(gn[ix], wn[ix]), f"token {t}"
        elif t >= 75:
            assert np.all(gn[ix] == 0), f"token {t}: tail of the tile not zeroed"
        else:
            assert np.all(gn[ix] == SENTINEL), f"token {t}: below token0 written"
        written[ix] = t >= 70
    assert np.all(gn[~written] == SENTINEL)


def test_append_argument_errors(torch_dev, sq):
    torch = torch_dev
    _case("append argument errors")
    cfg = wl.CONFIGS["llama8b"]
    cal, _ = H.calibrate_both(sq, cfg, [(0, 0)], "k", 3.0)
    cal.upload()
    x = torch.zeros((1, 1, 3, 128), dtype=torch.bfloat16, device="cuda")
    slot = torch.full((1, 1, cal.packed_head_words(64)), SENTINEL, dtype=torch.int32, device="cuda")
    with pytest.raises(sq.SQError):
        sq.sq_compress_append(cal, x, slot, -1)
    with pytest.raises(sq.SQError):  # tokens 62..64 need two tiles
        sq.sq_compress_append(cal, x, slot, 62)
    torch.cuda.synchronize()
    assert torch.all(slot == SENTINEL)


def test_append_batched_per_layer_calibration_strided_input(torch_dev, sq):
    """batch = 2 layers addressed through the calibration batch stride, input
    in [T][H][d] storage viewed as [H][T][d] (strided), appended in pieces:
    the same words as one sq_compress of the whole sequence."""
    torch = torch_dev
    _case("append qwen14b k: 2 layers (stride 4), strided input, pieces [1, 70, 1, 56]")
    cfg = wl.CONFIGS["qwen14b"]
    lheads = [(l, h) for l in (20, 21) for h in range(4)]
    cal, ors = H.calibrate_both(sq, cfg, lheads, "k", 2.5)
    cal.upload()
    T, pieces = 128, [1, 70, 1, 56]
    xl = np.stack([H.data_block(cfg, lheads[4 * b:4 * b + 4], "k", T) for b in range(2)])  # [B][H][T][d]
    xd = _dev(torch, np.ascontiguousarray(xl.transpose(0, 2, 1, 3)), torch.bfloat16).permute(0, 2, 1, 3)
    assert not xd.is_contiguous()
    words = cal.packed_head_words(T)
    whole = torch.zeros((2, 4, words), dtype=torch.int32, device="cuda")
    sq.sq_compress(cal, xd, whole, calib_batch_stride=4)
    inc = torch.full((2, 4, words), SENTINEL, dtype=torch.int32, device="cuda")
    t0 = 0
    for n in pieces:
        sq.sq_compress_append(cal, xd[:, :, t0:t0 + n], inc, t0, calib_batch_stride=4)
        t0 += n
    torch.cuda.synchronize()
    wn = whole.cpu().numpy().view(np.uint32)
    gn = inc.cpu().numpy().view(np.uint32)
    for b in range(2):
        for h in range(4):
            oc = ors[4 * b + h]
            used = 2 * 64 * oc.W
            assert np.array_equal(gn[b, h, :used], wn[b, h, :used]), f"batch {b} head {h}"
            H.compare_compress(oc, gn[b, h], xl[b, h], T)
