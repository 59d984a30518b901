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
KERNEL_SRC = os.path.join(ROOT, "compression_sq_compress_amd", "csrc", "kernels.hip")


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
    return ap.parse_args()


def kernel_source_digest() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per compress launch from the committed counter summary, or
    None when it is missing or was taken on a different kernel source."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m_src = re.search(r"kernel source sha256\[:16\]:\s*([0-9a-f]{16})", txt)
    m_b = re.search(r"HBM bytes per compress launch \(scaled\):\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != kernel_source_digest():
        return None
    return float(m_b.group(1))


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
                sample=(f"sequences 0-{n_seqs - 1}, {H} KV heads x {n_tokens} tokens each, K and V "
                        f"compress+pack, scores for the {G} query heads of each KV head, "
                        f"softmax+attend; {n_vec} vectors in {dt:.2f} s of oracle time"))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here "
              "(the decode workload shards by KV head with no exchange; one GPU's share is "
              "what is measured).", file=sys.stderr)
        sys.exit(2)
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
    ms_ck, ms_cv, ms_sc, ms_at = per.mean(axis=0)
    ms_step = wall * 1e3 / args.steps

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

    n_vec = B * Hkv * T
    # algorithmic bytes: compress reads d bf16 and writes one record per vector
    bytes_ck = n_vec * (2 * d + 4 * Wk)
    bytes_cv = n_vec * (2 * d + 4 * Wv)
    bytes_sc = n_vec * 4 * Wk + B * Hq * T * 4 + B * Hq * d * 2
    bytes_at = n_vec * 4 * Wv + B * Hq * T * 4 + B * Hq * d * 4
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
                   "avg_bits": 3.0, "record_words_k": Wk, "record_words_v": Wv},
        "kernels_ms": {"compress_k": ms_ck, "compress_v": ms_cv, "scores": ms_sc, "attend": ms_at},
        "compress_vectors_per_s": 2 * n_vec / (comp_ms * 1e-3),
        "compress_GBps": gbps(bytes_ck + bytes_cv, comp_ms),
        "compress_mfma_frac_alg": flops_comp / (comp_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        "compress_mfma_frac_issued": 3 * flops_comp / (comp_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        "score_GBps": gbps(bytes_sc, ms_sc),
        "score_hbm_frac": gbps(bytes_sc, ms_sc) / HBM_PEAK_GBPS,
        "score_packedK_GBps": gbps(n_vec * 4 * Wk, ms_sc),
        "attend_GBps": gbps(bytes_at, ms_at),
        "attend_hbm_frac": gbps(bytes_at, ms_at) / HBM_PEAK_GBPS,
        "append_decode": {"what": f"1 new token per (sequence, KV head), K and V: {2 * B * Hkv} vectors "
                                  f"into slots at token {T - 1}", "us": append_us},
        "roofline": {"bound": "hbm", "kernel": "compress2_kernel<128,bf16> (register quantiser; per launch, K and V averaged)",
                     "achieved": comp_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": comp_gbps / HBM_PEAK_GBPS, "traffic": traffic,
                     "alg_bytes_per_launch": comp_launch_bytes, "launch_ms": comp_launch_ms},
        "roofline_scores": {"bound": "hbm", "kernel": "scores_kernel (split-K waves, 4x4x4 bf16 MFMA, joint tables)",
                            "achieved": gbps(bytes_sc, ms_sc), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": gbps(bytes_sc, ms_sc) / HBM_PEAK_GBPS,
                            "traffic": None, "alg_bytes_per_launch": bytes_sc, "launch_ms": ms_sc},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, (Xk, Gk), Xv, args.cpu_sample_seqs, T)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
