#!/usr/bin/env python3
"""Benchmark of the SpectralQuant hot path on one MI355X.

Workload (the decode configuration): 64 sequences x 32768 tokens, 8 KV heads
(32 query heads, groups of 4), head_dim 128, bf16 keys/values with the
Llama-shaped spectra, 3 bits per coordinate, keys with 1 QJL bit per signal
dimension.  One step = the whole hot path over that batch:
    sq_compress(K) + sq_compress(V)          (33.5 M vectors)
  + sq_scores (bf16 queries)                 (fp32 scores [64][32][32768])
  + sq_attend (softmax + value sum)          (fp32 out [64][32][128])
Inputs are resident in HBM before the timed region; calibration (host, one
time) is outside it.  ``value`` is KV vectors compressed per second of the
whole step; per-kernel rates, the roofline of the dominant kernel (the
compress kernel) and the CPU oracle on a bounded sample of the same workload
are reported beside it.

Every launch goes to one dedicated stream (default priority); the per-kernel
times come from HIP events recorded on that stream around each launch.
After the timed steps (outside them) the decode-time append is timed: one
new token per (sequence, KV head) for K and V through sq_compress_append.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
                       [--cpu-sample-seqs 4] [--copy-ref-mb 0]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "compress_kernel_decode_traffic.md")
COUNTER_FILE = os.path.join(ROOT, "profiles", "decode_kernels_shader_counters.md")
CLOCK_GHZ = 2.4                 # MI355X peak engine clock, published
N_CUS = 256
N_SIMDS = N_CUS * 4             # 256 CUs x 4 SIMDs


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=None, help="override sequences (default 64)")
    ap.add_argument("--tokens", type=int, default=None, help="override tokens (default 32768)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=4,
                    help="sequences (all KV heads, all tokens) the CPU oracle processes")
    ap.add_argument("--copy-ref-mb", type=int, default=0,
                    help="also run one fp32 copy kernel of this many MiB before the timed "
                         "region (reference for scaling HBM byte counters)")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "tiny", "llama8b", "qwen14b", "gemma9b"],
                    help="decode (default): the throughput benchmark; the others: one decode "
                         "step's latency over every layer of that model shape")
    ap.add_argument("--scheme", default="sq", choices=["sq", "tq"],
                    help="latency workloads: SpectralQuant (sq) or the TurboQuant-style baseline (tq)")
    ap.add_argument("--bits", type=float, default=None,
                    help="latency workloads: code bits per coordinate (default: the workload's first budget; "
                         "tq: an integer)")
    return ap.parse_args()


def kernel_source_digest() -> str:
    from compression_sq_compress_amd.digest import source_digest
    return source_digest()


def measured_traffic(kernel: str = "compress"):
    """HBM bytes per launch of ``kernel`` (compress, scores, decode) from the
    committed counter summary, or None when it is missing or was taken on
    other kernel sources."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m_src = re.search(r"kernel source sha256\[:16\]:\s*([0-9a-f]{16})", txt)
    m_b = re.search(r"HBM bytes per %s launch \(scaled\):\s*([0-9.eE+]+)" % kernel, txt)
    if not m_src or not m_b or m_src.group(1) != kernel_source_digest():
        return None
    return float(m_b.group(1))


def measured_counters_per_tile(column: int = 0):
    """Per-tile shader counters of one kernel column (0: the compress kernel)
    from the committed counter summary, or None when it is missing or was
    taken on other kernel sources."""
    try:
        txt = open(COUNTER_FILE).read()
    except OSError:
        return None
    m_src = re.search(r"kernel source sha256\[:16\]:\s*([0-9a-f]{16})", txt)
    if not m_src or m_src.group(1) != kernel_source_digest():
        return None
    out = {}
    for line in txt.splitlines():
        m = re.match(r"\|\s*(SQ_[A-Z_]+)\s*\|(.*)\|\s*$", line)
        if m:
            cells = [c.strip() for c in m.group(2).split("|")]
            try:
                out[m.group(1)] = float(cells[column])
            except (IndexError, ValueError):
                pass
    return out or None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, kcal_in, vcal_in, n_seqs, n_tokens):
    """Time the CPU oracle, as it stands, on a bounded sample of the workload:
    sequences 0..n_seqs-1, all KV heads, all ``n_tokens`` tokens of each;
    compress K and V (rotate, quantise, QJL, pack), score the query heads of
    each group, softmax + value sum.  Inputs are generated before the clock
    starts.  Returns KV vectors per second."""
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    Xk, Gk = kcal_in
    Xv = vcal_in
    H = cfg.kv_heads
    G = cfg.q_heads // H
    kors = [oracle.calibrate(Xk[h], 3.0, 1, Gk[h]) for h in range(H)]
    vors = [oracle.calibrate(Xv[h], 3.0, 0, None) for h in range(H)]
    q = wl.queries(cfg, n_seqs, cfg.q_heads)
    dt = 0.0
    for b in range(n_seqs):
        for h in range(H):
            xk = wl.kv_block(cfg, 0, h, "k", n_tokens, "data", batch_index=b)
            xv = wl.kv_block(cfg, 0, h, "v", n_tokens, "data", batch_index=b)
            t0 = time.perf_counter()
            rk = oracle.compress(kors[h], xk)
            oracle.pack(kors[h].widths, kors[h].m, rk.codes, rk.z, rk.gamma)
            rv = oracle.compress(vors[h], xv)
            oracle.pack(vors[h].widths, 0, rv.codes, rv.z, rv.gamma)
            s = oracle.scores_rotated(kors[h], q[b, h * G:(h + 1) * G], rk.codes, rk.z, rk.gamma)
            oracle.attend(vors[h], s, 1 / math.sqrt(cfg.head_dim), rv.codes)
            dt += time.perf_counter() - t0
    n_vec = 2 * n_seqs * H * n_tokens
    return dict(value=n_vec / dt, unit="KV vectors/s", cores=int(threads), kind="oracle",
                cpu_model=cpu_model(), host_cpus=os.cpu_count(),
                sample=(f"sequences 0-{n_seqs - 1}, {H} KV heads x {n_tokens} tokens each, K and V "
                        f"compress+pack, scores for the {G} query heads of each KV head, "
                        f"softmax+attend; {n_vec} vectors in {dt:.2f} s of oracle time"))


def latency(args):
    """One decode step of a whole model shape (every layer, batch 1): for each
    layer and KV head, append the new token's K and V (sq_compress_append),
    then scores + softmax + value sum over the T-token compressed cache, as
    sq_scores + sq_attend and as the fused sq_decode.  Layers are the batch
    dimension of one call (calibration head = layer * kv_heads + head).  The
    cache itself is compressed once before the timed region (its time is
    reported as prefill).  Prints one JSON line."""
    import torch
    import workloads as wl
    import compression_sq_compress_amd as sq
    cfg = wl.CONFIGS[args.workload]
    L, Hkv, Hq, d = cfg.layers, cfg.kv_heads, cfg.q_heads, cfg.head_dim
    T = args.tokens or cfg.tokens[-1]
    G = Hq // Hkv
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream
    heads = [(l, h) for l in range(L) for h in range(Hkv)]
    if args.scheme == "tq":
        bits = int(args.bits or 3)
        rot = np.stack([wl.tq_rotation(cfg, l, h) for l, h in heads]).astype(np.float32)
        sk = np.stack([wl.tq_qjl(cfg, l, h) for l, h in heads]).astype(np.float32)
        kcal = sq.sq_calibrate_tq(rot, bits, True, sk).upload(sh)
        vcal = sq.sq_calibrate_tq(rot, bits, False).upload(sh)
        label = f"TurboQuant-style, {bits} bits ({bits - 1}-bit keys + all-dims QJL)"
    else:
        bits = float(args.bits or cfg.budgets[0])
        Xk = np.stack([wl.calibration_set(cfg, l, h, "k") for l, h in heads]).astype(np.float32)
        Gk = np.stack([wl.qjl_gaussian(cfg, l, h) for l, h in heads])
        Xv = np.stack([wl.calibration_set(cfg, l, h, "v") for l, h in heads]).astype(np.float32)
        kcal = sq.sq_calibrate(Xk, bits, cfg.qjl_bits, Gk).upload(sh)
        vcal = sq.sq_calibrate(Xv, bits, 0, None).upload(sh)
        label = f"SpectralQuant, {bits} bits/coord + QJL on the signal dims"
    with torch.cuda.stream(stream):
        K = wl.layers_kv_on_device(cfg, "k", range(L), T + 1)
        V = wl.layers_kv_on_device(cfg, "v", range(L), T + 1)
        dtq = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        q = torch.from_numpy(wl.queries(cfg, L, Hq)).to(dev).to(dtq)
        kp = torch.zeros((L, Hkv, kcal.packed_head_words(T + 1)), dtype=torch.int32, device=dev)
        vp = torch.zeros((L, Hkv, vcal.packed_head_words(T + 1)), dtype=torch.int32, device=dev)
        s = torch.empty((L, Hq, T + 1), dtype=torch.float32, device=dev)
        ws = torch.empty(sq.sq_attend_workspace_bytes(L, Hq, T + 1, d) // 4, dtype=torch.float32, device=dev)
        out = torch.empty((L, Hq, d), dtype=torch.float32, device=dev)
        out2 = torch.empty_like(out)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    Kc, Vc = K[:, :, :T], V[:, :, :T]
    Kn, Vn = K[:, :, T:T + 1], V[:, :, T:T + 1]

    def prefill():
        sq.sq_compress(kcal, Kc, kp, calib_batch_stride=Hkv, stream=sh)
        sq.sq_compress(vcal, Vc, vp, calib_batch_stride=Hkv, stream=sh)

    def append():
        sq.sq_compress_append(kcal, Kn, kp, T, calib_batch_stride=Hkv, stream=sh)
        sq.sq_compress_append(vcal, Vn, vp, T, calib_batch_stride=Hkv, stream=sh)

    def split():
        sq.sq_scores(kcal, q, kp, T + 1, s, Hkv, calib_batch_stride=Hkv, stream=sh)
        sq.sq_attend(vcal, s, scale, vp, T + 1, ws, out, Hkv, calib_batch_stride=Hkv, stream=sh)

    fused_ok = True
    try:
        sq.sq_decode(kcal, vcal, q, kp, vp, T + 1, scale, ws, out2, Hkv, calib_batch_stride=Hkv, stream=sh)
    except sq.SQError as e:
        fused_ok = False
        fused_msg = str(e)

    def fused():
        sq.sq_decode(kcal, vcal, q, kp, vp, T + 1, scale, ws, out2, Hkv, calib_batch_stride=Hkv, stream=sh)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    ms_prefill = timed(prefill)
    ms_append = timed(append)
    ms_split = timed(split)
    ms_fused = timed(fused) if fused_ok else None
    step_ms = ms_append + (min(ms_split, ms_fused) if fused_ok else ms_split)
    res = {
        "metric": "decode step latency over every layer (append 1 token + scores + softmax + value sum)",
        "value": step_ms, "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": step_ms, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {L} layers x {Hkv} KV / {Hq} q heads, hd{d}, {T}-token cache, "
                               f"batch 1; {label}", "layers": L, "tokens": T, "scheme": args.scheme,
                   "bits": bits, "record_words_k": kcal.info(0).record_words,
                   "record_words_v": vcal.info(0).record_words},
        "ms": {"append_kv": ms_append, "scores_plus_attend": ms_split, "decode_fused": ms_fused,
               "prefill_compress_kv": ms_prefill},
        "note": ("working set below the 256 MB Infinity Cache (MALL): latency, not an HBM-bandwidth figure"
                 + ("" if fused_ok else f"; sq_decode refused: {fused_msg}")),
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here "
              "(the decode workload shards by KV head with no exchange; one GPU's share is "
              "what is measured).", file=sys.stderr)
        sys.exit(2)
    if args.workload != "decode":
        latency(args)
        return
    import torch
    import workloads as wl
    import compression_sq_compress_amd as sq

    cfg = wl.CONFIGS["decode"]
    B = args.batch or cfg.batch
    T = args.tokens or cfg.tokens[0]
    Hkv, Hq, d = cfg.kv_heads, cfg.q_heads, cfg.head_dim
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)       # default priority
    sh = stream.cuda_stream

    # one-time host calibration (512-token calibration set per KV head)
    Xk = np.stack([wl.calibration_set(cfg, 0, h, "k") for h in range(Hkv)]).astype(np.float32)
    Gk = np.stack([wl.qjl_gaussian(cfg, 0, h) for h in range(Hkv)])
    Xv = np.stack([wl.calibration_set(cfg, 0, h, "v") for h in range(Hkv)]).astype(np.float32)
    kcal = sq.sq_calibrate(Xk, 3.0, 1, Gk).upload(sh)
    vcal = sq.sq_calibrate(Xv, 3.0, 0, None).upload(sh)
    Wk = max(kcal.info(h).record_words for h in range(Hkv))
    Wv = max(vcal.info(h).record_words for h in range(Hkv))

    # synthetic inputs resident in HBM
    with torch.cuda.stream(stream):
        K = wl.decode_kv_on_device(cfg, "k", n_batch=B, n_tokens=T)
        V = wl.decode_kv_on_device(cfg, "v", n_batch=B, n_tokens=T)
        q = torch.from_numpy(wl.queries(cfg, B, Hq)).to(dev).to(torch.bfloat16)
        kp = torch.empty((B, Hkv, kcal.packed_head_words(T)), dtype=torch.int32, device=dev)
        vp = torch.empty((B, Hkv, vcal.packed_head_words(T)), dtype=torch.int32, device=dev)
        scores = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
        ws = torch.empty(sq.sq_attend_workspace_bytes(B, Hq, T, d) // 4, dtype=torch.float32,
                         device=dev)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev: ev[0].record(stream)
        sq.sq_compress(kcal, K, kp, stream=sh)
        if ev: ev[1].record(stream)
        sq.sq_compress(vcal, V, vp, stream=sh)
        if ev: ev[2].record(stream)
        sq.sq_scores(kcal, q, kp, T, scores, Hkv, stream=sh)
        if ev: ev[3].record(stream)
        sq.sq_attend(vcal, scores, scale, vp, T, ws, out, Hkv, stream=sh)
        if ev: ev[4].record(stream)

    if args.copy_ref_mb > 0:
        # one plain copy kernel of known size: N MiB read + N MiB written
        with torch.cuda.stream(stream):
            src = torch.ones(args.copy_ref_mb * (1 << 18), dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        print(f"copy reference: {args.copy_ref_mb} MiB read + written", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])  # ms
    ms_ck, ms_cv, ms_sc, ms_at = np.median(per, axis=0)  # median over the timed steps
    ms_step = wall * 1e3 / args.steps

    # the fused decode step (scores, softmax and value sum in one pass, no score
    # tensor), on the same records and queries, outside the timed steps
    out2 = torch.empty_like(out)
    for _ in range(args.warmup):
        sq.sq_decode(kcal, vcal, q, kp, vp, T, scale, ws, out2, Hkv, stream=sh)
    dev_ = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        dev_[k][0].record(stream)
        sq.sq_decode(kcal, vcal, q, kp, vp, T, scale, ws, out2, Hkv, stream=sh)
        dev_[k][1].record(stream)
    torch.cuda.synchronize()
    ms_dec = float(np.median([e[0].elapsed_time(e[1]) for e in dev_]))
    dec_err = float(((out2 - out).abs() / (out.abs() + out.norm(dim=-1, keepdim=True) / math.sqrt(d))).max())

    # decode-time append, outside the timed step: the last token of every
    # (sequence, KV head) compressed again into its slot (same words), K then V
    ka, va = K[:, :, T - 1:T], V[:, :, T - 1:T]
    aev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(20)]
    for k in range(len(aev) + 3):
        e = aev[k - 3] if k >= 3 else None
        if e: e[0].record(stream)
        sq.sq_compress_append(kcal, ka, kp, T - 1, stream=sh)
        sq.sq_compress_append(vcal, va, vp, T - 1, stream=sh)
        if e: e[1].record(stream)
    torch.cuda.synchronize()
    append_us = float(np.mean([e[0].elapsed_time(e[1]) for e in aev])) * 1e3

    # the same decode over a paged cache (blocks of 4 tiles handed out in a
    # seeded random order), outside the timed steps; must equal sq_decode bit for bit
    bt = 4
    nlb = ((T + 63) // 64 + bt - 1) // bt
    n_blocks = B * nlb
    perm = np.random.default_rng(7).permutation(n_blocks).astype(np.int32).reshape(B, nlb)
    table = torch.from_numpy(perm).to(dev)
    pg = sq.paged(table, bt, n_blocks)
    with torch.cuda.stream(stream):
        kpool = torch.empty((n_blocks * Hkv * sq.sq_paged_block_words(kcal, bt),), dtype=torch.int32, device=dev)
        vpool = torch.empty((n_blocks * Hkv * sq.sq_paged_block_words(vcal, bt),), dtype=torch.int32, device=dev)
    sq.sq_compress_append_paged(kcal, K, kpool, pg, 0, stream=sh)
    sq.sq_compress_append_paged(vcal, V, vpool, pg, 0, stream=sh)
    out3 = torch.empty_like(out)
    for _ in range(args.warmup):
        sq.sq_decode_paged(kcal, vcal, q, kpool, vpool, pg, T, scale, ws, out3, Hkv, stream=sh)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        pev[k][0].record(stream)
        sq.sq_decode_paged(kcal, vcal, q, kpool, vpool, pg, T, scale, ws, out3, Hkv, stream=sh)
        pev[k][1].record(stream)
    torch.cuda.synchronize()
    ms_pdec = float(np.median([e[0].elapsed_time(e[1]) for e in pev]))
    paged_equal = bool(torch.equal(out3.view(torch.int32), out2.view(torch.int32)))
    del kpool, vpool

    # one-time calibration: host (C++, all host threads) against the device
    # path, for this workload's 8 key heads and for 48 layers' worth of heads
    def _wall(fn):
        torch.cuda.synchronize()
        t = time.perf_counter()
        r = fn()
        torch.cuda.synchronize()
        return r, (time.perf_counter() - t) * 1e3
    _, cal_host_ms = _wall(lambda: sq.sq_calibrate(Xk, 3.0, 1, Gk))
    Xk_d = torch.from_numpy(Xk).to(dev)
    sq.sq_calibrate_device(Xk_d, 3.0, 1, Gk)  # warm-up (module load)
    _, cal_dev_ms = _wall(lambda: sq.sq_calibrate_device(Xk_d, 3.0, 1, Gk))
    Xk48 = Xk_d.repeat(48, 1, 1).contiguous()
    Gk48 = np.concatenate([Gk] * 48)
    _, cal_dev48_ms = _wall(lambda: sq.sq_calibrate_device(Xk48, 3.0, 1, Gk48))
    _, cal_host48_ms = _wall(lambda: sq.sq_calibrate(Xk48.cpu().numpy(), 3.0, 1, Gk48))
    del Xk48

    n_vec = B * Hkv * T
    # algorithmic bytes: compress reads d bf16 and writes one record per vector
    bytes_ck = n_vec * (2 * d + 4 * Wk)
    bytes_cv = n_vec * (2 * d + 4 * Wv)
    bytes_sc = n_vec * 4 * Wk + B * Hq * T * 4 + B * Hq * d * 2
    bytes_at = n_vec * 4 * Wv + B * Hq * T * 4 + B * Hq * d * 4
    bytes_dec = n_vec * 4 * (Wk + Wv) + B * Hq * d * (2 + 4)   # both records, q in, out
    gbps = lambda b, ms: b / (ms * 1e-3) / 1e9
    comp_ms = ms_ck + ms_cv
    # the compress kernel runs twice per step (K, V): per-launch averages
    comp_launch_bytes = (bytes_ck + bytes_cv) / 2
    comp_launch_ms = comp_ms / 2
    comp_gbps = gbps(comp_launch_bytes, comp_launch_ms)
    flops_comp = 2 * n_vec * 2 * d * d   # algorithmic rotation flops (K and V)
    traffic = measured_traffic()
    res = {
        "metric": "KV vectors compressed/s + compressed q·K score GB/s (hd128), % HBM roofline",
        "value": 2 * n_vec / (ms_step * 1e-3),
        "unit": "KV vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode: {B} seqs x {T} tokens, {Hq} q / {Hkv} KV heads, hd{d}, "
                               f"bf16 K/V, 3 bits/coord, 1 QJL bit per key signal dim",
                   "batch": B, "tokens": T, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "avg_bits": 3.0, "record_words_k": Wk, "record_words_v": Wv,
                   "step": "sq_compress of every K and V vector of the cache (the metric's compress leg, "
                           "not a serving step), then sq_scores and sq_attend over it"},
        "kernels_ms": {"compress_k": ms_ck, "compress_v": ms_cv, "scores": ms_sc, "attend": ms_at},
        "compress_vectors_per_s": 2 * n_vec / (comp_ms * 1e-3),
        "compress_GBps": gbps(bytes_ck + bytes_cv, comp_ms),
        "compress_mfma_frac_alg": flops_comp / (comp_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        "compress_mfma_frac_issued": 3 * flops_comp / (comp_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        # the third roofline of the compress kernel, VALU issue: its non-MFMA
        # VALU instructions per 64-token tile (committed counter summary, same
        # sources) x 4 cycles per wave64 instruction, over the SIMD cycles of
        # a launch at the peak clock; null when the summary is stale
        "compress_valu_frac": (None if not (cc := measured_counters_per_tile(0)) else
                               (cc["SQ_INSTS_VALU"] - cc["SQ_INSTS_MFMA"]) * 4 * (n_vec / 64) /
                               (N_SIMDS * comp_launch_ms * 1e-3 * CLOCK_GHZ * 1e9)),
        "compress_mfma_busy_frac": (None if not cc else
                                    cc["SQ_VALU_MFMA_BUSY_CYCLES"] * (n_vec / 64) /
                                    (N_SIMDS * comp_launch_ms * 1e-3 * CLOCK_GHZ * 1e9)),
        "score_GBps": gbps(bytes_sc, ms_sc),
        "score_hbm_frac": gbps(bytes_sc, ms_sc) / HBM_PEAK_GBPS,
        "score_packedK_GBps": gbps(n_vec * 4 * Wk, ms_sc),
        "attend_GBps": gbps(bytes_at, ms_at),
        "attend_hbm_frac": gbps(bytes_at, ms_at) / HBM_PEAK_GBPS,
        "decode_fused": {"what": "sq_decode: scores, online softmax and value sum in one pass over the "
                                 "packed K and V (no score tensor), same records and queries",
                         "ms": ms_dec, "GBps": gbps(bytes_dec, ms_dec),
                         "hbm_frac": gbps(bytes_dec, ms_dec) / HBM_PEAK_GBPS,
                         "alg_bytes": bytes_dec, "split_path_ms": ms_sc + ms_at,
                         "max_rel_diff_vs_split": dec_err},
        "append_decode": {"what": f"1 new token per (sequence, KV head), K and V: {2 * B * Hkv} vectors "
                                  f"into slots at token {T - 1}", "us": append_us},
        "decode_paged": {"what": f"sq_decode_paged: the fused decode over paged K/V pools (blocks of "
                                 f"{bt * 64} tokens, random block order)", "ms": ms_pdec,
                         "GBps": gbps(bytes_dec, ms_pdec), "equal_to_contiguous": paged_equal},
        "calibration": {"what": "one-time key calibration, 512 samples per head, hd128 (host: C++ on "
                                f"{os.cpu_count()} threads; device: covariance, Jacobi and rotation on the GPU, "
                                "Lloyd-Max on the host)",
                        "heads_8": {"host_ms": cal_host_ms, "device_ms": cal_dev_ms},
                        "heads_384": {"host_ms": cal_host48_ms, "device_ms": cal_dev48_ms}},
        "roofline": {"bound": "hbm", "kernel": "compress2_kernel<128,bf16> (register quantiser; per launch, K and V averaged)",
                     "achieved": comp_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": comp_gbps / HBM_PEAK_GBPS, "traffic": traffic,
                     "alg_bytes_per_launch": comp_launch_bytes, "launch_ms": comp_launch_ms},
        "roofline_scores": {"bound": "hbm", "kernel": "scores_kernel (split-K waves, 4x4x4 bf16 MFMA, joint tables)",
                            "achieved": gbps(bytes_sc, ms_sc), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": gbps(bytes_sc, ms_sc) / HBM_PEAK_GBPS,
                            "traffic": measured_traffic("scores"), "alg_bytes_per_launch": bytes_sc,
                            "launch_ms": ms_sc,
                            # its LDS roofline: LDS-busy cycles per 64-token tile (committed counter
                            # summary, same sources) over the CU cycles of the launch at 2.4 GHz
                            "lds_busy_frac": (None if not (cs := measured_counters_per_tile(1)) else
                                              cs["SQ_LDS_IDX_ACTIVE"] * (n_vec / 64) /
                                              (N_CUS * ms_sc * 1e-3 * CLOCK_GHZ * 1e9))},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, (Xk, Gk), Xv, args.cpu_sample_seqs, T)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
