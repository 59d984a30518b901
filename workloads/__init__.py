"""Seeded synthetic workloads for the SpectralQuant KV-cache hot path.

This module only draws random numbers and shapes them into the workloads the
SpectralQuant pages describe (the spectra, norms, shapes and dtypes of the five
configurations below).  It holds none of the method's arithmetic: no
covariance, eigendecomposition, bit allocation, codebook, quantisation or
packing.  Both the CPU oracle (through the tests) and the GPU path (through the
tests and the benchmark) consume what it returns, so the two sides always see
bit-identical inputs.

Random numbers the method itself draws (the QJL Gaussian sketch matrix, the
TurboQuant-style random rotation) are drawn here too and handed to both sides
as explicit inputs.

Streams: every array comes from NumPy's PCG64 seeded by
``SeedSequence(seed, spawn_key=(config id, layer, head, stream id))`` so any
(layer, head, stream) chunk can be regenerated on its own.  The large decode
configuration is generated on the GPU with torch's seeded generator instead
(``decode_kv_on_device``); tests read the sampled rows back from device memory.

Rounding to bfloat16 is round-to-nearest-even of the float32 value
(float64 draw -> float32 RNE -> bfloat16 RNE).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# The ten seeds the SpectralQuant README lists for its confidence-interval runs
# (README "Random Seeds"); 42 is the default.
SEEDS = (42, 123, 7, 2024, 31415, 99, 1337, 8675309, 271828, 314159)
DEFAULT_SEED = 42

_STREAMS = {
    "basis_k": 1, "basis_v": 2, "calib_k": 3, "calib_v": 4, "keys": 5,
    "values": 6, "queries": 7, "qjl_k": 8, "qjl_v": 9, "tq_rot": 10,
    "tq_qjl": 11, "scores": 12, "misc": 13,
}


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload shape.  ``layers * kv_heads`` calibration heads, each with
    its own eigenbasis; ``q_heads`` query heads share KV heads in contiguous
    groups of ``q_heads // kv_heads``."""
    name: str
    cid: int
    head_dim: int
    layers: int
    kv_heads: int
    q_heads: int
    tokens: tuple          # sequence lengths to run
    batch: int
    dtype: str             # "f32" or "bf16"
    calib_tokens: int      # 0 = calibrate on the data itself
    budgets: tuple         # average code bits per coordinate
    qjl_bits: int          # QJL bits per signal dimension (keys)
    key_spectrum: str
    value_spectrum: str
    key_mean_norm: Optional[float]
    value_mean_norm: Optional[float]


# The five workloads (the SpectralQuant benchmark configuration list):
#  tiny    - head_dim 32, 4 heads x 3 layers x 256 tokens, fp32, sharp-gap spectrum
#            diag(50 x8, 1 x24) as in the test fixtures of the SpectralQuant
#            repository (tests/conftest.py, ``sharp_gap_kv_data``), calibrated on
#            the same 256 tokens, 3 bits, 1 QJL bit per signal dim, 8 queries.
#  llama8b - one Llama-3.1-8B-shaped layer: 8 KV heads (32 q heads), hd128,
#            2048 tokens, bf16, 512-token calibration set, 3 bits.
#  qwen14b - 48 layers, 40 q / 8 KV heads, hd128, bf16, T in {512,1024,2048},
#            budgets 2.5 and 3.5.
#  decode  - 64 sequences x 32768 tokens, 32 q / 8 KV heads, hd128, 3 bits.
#  gemma9b - 42 layers, 16 q / 8 KV heads, hd256, 4096 tokens, bf16, 3 bits.
CONFIGS = {
    "tiny": Config("tiny", 0, 32, 3, 4, 4 * 8, (256,), 1, "f32", 0, (3.0,), 1,
                   "sharp_gap", "sharp_gap", None, None),
    "llama8b": Config("llama8b", 1, 128, 1, 8, 32, (2048,), 1, "bf16", 512, (3.0,), 1,
                      "keys128", "values128", 170.0, 3.0),
    "qwen14b": Config("qwen14b", 2, 128, 48, 8, 40, (512, 1024, 2048), 1, "bf16", 512,
                      (2.5, 3.5), 1, "keys128", "values128", 170.0, 3.0),
    "decode": Config("decode", 3, 128, 1, 8, 32, (32768,), 64, "bf16", 512, (3.0,), 1,
                     "keys128", "values128", 170.0, 3.0),
    "gemma9b": Config("gemma9b", 4, 256, 42, 8, 16, (4096,), 1, "bf16", 512, (3.0,), 1,
                      "keys256", "values256", 170.0, 3.0),
}


def population_spectrum(kind: str, d: int) -> np.ndarray:
    """Unscaled population eigenvalues (descending) for a spectrum name.

    sharp_gap : 50 on 8 dims, 1 on the rest (test-fixture spectrum).
    keys128   : 400, 200, 100, 50, then a geometric decay 1 -> 0.01 over the
                remaining dims (Llama-shaped keys).
    keys256   : 400 on 9 dims then geometric 1 -> 0.01 (top ~3.5% dominant).
    values128 : exp(-i / 24.2422), whose participation ratio is 48.
    values256 : exp(-i / 50.6400), whose participation ratio is 100.
    flat      : identity.
    """
    if kind == "sharp_gap":
        return np.concatenate([np.full(8, 50.0), np.ones(d - 8)])
    if kind == "keys128":
        return np.concatenate([[400.0, 200.0, 100.0, 50.0], np.geomspace(1.0, 0.01, d - 4)])
    if kind == "keys256":
        return np.concatenate([np.full(9, 400.0), np.geomspace(1.0, 0.01, d - 9)])
    if kind == "values128":
        return np.exp(-np.arange(d) / 24.24224051619744)
    if kind == "values256":
        return np.exp(-np.arange(d) / 50.63999520234728)
    if kind == "flat":
        return np.ones(d)
    raise ValueError(kind)


def rng_for(seed: int, cid: int, layer: int, head: int, stream: str) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(cid, layer, head, _STREAMS[stream]))
    return np.random.Generator(np.random.PCG64(ss))


def random_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    """Haar-random orthogonal matrix: QR of a Gaussian with the signs of R's
    diagonal folded into Q (the test-fixture construction plus sign fix)."""
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(x32)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Values of ``x`` rounded to bfloat16 (returned as float32)."""
    return bf16_bits_to_f32(to_bf16_bits(to_f32(x)))


_SCALE_CACHE: dict = {}


def norm_scale(kind: str, d: int, mean_norm: Optional[float]) -> float:
    """Factor that gives vectors of spectrum ``kind`` the stated mean norm.

    Estimated once from a fixed Monte-Carlo draw (seed 0, 200k vectors), so it is
    a deterministic constant of the workload."""
    if mean_norm is None:
        return 1.0
    key = (kind, d, mean_norm)
    if key not in _SCALE_CACHE:
        lam = population_spectrum(kind, d)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(0)))
        z = rng.standard_normal((200_000, d)) * np.sqrt(lam)[None, :]
        _SCALE_CACHE[key] = float(mean_norm / np.linalg.norm(z, axis=1).mean())
    return _SCALE_CACHE[key]


def _spec(cfg: Config, which: str):
    kind = cfg.key_spectrum if which == "k" else cfg.value_spectrum
    mn = cfg.key_mean_norm if which == "k" else cfg.value_mean_norm
    return kind, mn


def head_basis(cfg: Config, layer: int, head: int, which: str, seed: int = DEFAULT_SEED) -> np.ndarray:
    """Orthonormal basis Q (columns) of one (layer, KV head) for keys ('k') or values ('v')."""
    return random_orthogonal(rng_for(seed, cfg.cid, layer, head, "basis_" + which), cfg.head_dim)


def head_covariance_factor(cfg: Config, layer: int, head: int, which: str,
                           seed: int = DEFAULT_SEED) -> np.ndarray:
    """Matrix A with x = z @ A for z ~ N(0, I): A = diag(sqrt(lambda)) Q^T * scale."""
    kind, mn = _spec(cfg, which)
    lam = population_spectrum(kind, cfg.head_dim)
    q = head_basis(cfg, layer, head, which, seed)
    return (np.sqrt(lam)[:, None] * q.T) * norm_scale(kind, cfg.head_dim, mn)


def _round(cfg: Config, x: np.ndarray) -> np.ndarray:
    return to_f32(x) if cfg.dtype == "f32" else round_bf16(x)


def kv_block(cfg: Config, layer: int, head: int, which: str, n: int, stream: str,
             seed: int = DEFAULT_SEED, batch_index: int = 0) -> np.ndarray:
    """n vectors of one (layer, head) for keys/values, float32 holding values
    exactly representable in the configuration's dtype.  ``stream`` is
    'calib' (calibration set) or 'data' (the sequence to compress)."""
    a = head_covariance_factor(cfg, layer, head, which, seed)
    sname = ("calib_" + which) if stream == "calib" else ("keys" if which == "k" else "values")
    rng = rng_for(seed, cfg.cid, layer, head + 1000 * batch_index, sname)
    z = rng.standard_normal((n, cfg.head_dim))
    return _round(cfg, z @ a)


def calibration_set(cfg: Config, layer: int, head: int, which: str, seed: int = DEFAULT_SEED,
                    n_tokens: Optional[int] = None) -> np.ndarray:
    """Calibration samples of one head.  With ``calib_tokens == 0`` (tiny) the
    calibration set is the data itself (the first sequence)."""
    if cfg.calib_tokens == 0:
        return kv_block(cfg, layer, head, which, n_tokens or cfg.tokens[0], "data", seed)
    return kv_block(cfg, layer, head, which, cfg.calib_tokens, "calib", seed)


def qjl_gaussian(cfg: Config, layer: int, head: int, which: str = "k",
                 seed: int = DEFAULT_SEED, qjl_bits: Optional[int] = None) -> np.ndarray:
    """Standard-normal matrix [qjl_bits*d, d] (float32) from which the QJL
    sketch S = G[:m, :d_eff] is taken.  Drawn here so that both sides of the
    parity tests use the same S."""
    qb = cfg.qjl_bits if qjl_bits is None else qjl_bits
    rng = rng_for(seed, cfg.cid, layer, head, "qjl_" + which)
    return to_f32(rng.standard_normal((max(qb, 1) * cfg.head_dim, cfg.head_dim)))


def queries(cfg: Config, n_batch: int, n_q_heads: int, seed: int = DEFAULT_SEED,
            layer: int = 0) -> np.ndarray:
    """Queries [n_batch][n_q_heads][d] ~ N(0, 1), rounded to the config dtype."""
    rng = rng_for(seed, cfg.cid, layer, 0, "queries")
    return _round(cfg, rng.standard_normal((n_batch, n_q_heads, cfg.head_dim)))


def tq_rotation(cfg: Config, layer: int, head: int, seed: int = DEFAULT_SEED) -> np.ndarray:
    """Haar-random rotation for the TurboQuant-style baseline (float64)."""
    return random_orthogonal(rng_for(seed, cfg.cid, layer, head, "tq_rot"), cfg.head_dim)


def tq_qjl(cfg: Config, layer: int, head: int, seed: int = DEFAULT_SEED) -> np.ndarray:
    """d x d Gaussian sketch for the TurboQuant-style baseline's all-dims QJL."""
    rng = rng_for(seed, cfg.cid, layer, head, "tq_qjl")
    return rng.standard_normal((cfg.head_dim, cfg.head_dim))


def flat_data(n: int, d: int, seed: int = DEFAULT_SEED) -> np.ndarray:
    """Identity-covariance samples (flat spectrum)."""
    rng = rng_for(seed, 99, 0, 0, "misc")
    return rng.standard_normal((n, d))


def rank_k_isotropic(n: int, d: int, k: int, seed: int = DEFAULT_SEED) -> np.ndarray:
    """Samples on a random k-dim subspace with equal variances, no noise."""
    rng = rng_for(seed, 98, 0, k, "misc")
    q = random_orthogonal(rng, d)[:, :k]
    return rng.standard_normal((n, k)) @ q.T


def rank4_fixture(n: int = 256, d: int = 32, seed: int = DEFAULT_SEED) -> np.ndarray:
    """Rank-4 data with variances 100/50/20/10 along a Gaussian (non-orthonormal)
    U, plus 0.01 isotropic noise (the repository's ``low_rank_data`` fixture shape)."""
    rng = rng_for(seed, 97, 0, 0, "misc")
    u = rng.standard_normal((d, 4))
    z = rng.standard_normal((n, 4))
    x = (z * np.sqrt([100.0, 50.0, 20.0, 10.0])[None, :]) @ u.T
    return x + rng.standard_normal((n, d)) * 0.01


def decode_kv_on_device(cfg: Config, which: str, seed: int = DEFAULT_SEED, device="cuda",
                        n_batch: Optional[int] = None, n_tokens: Optional[int] = None):
    """Large decode-configuration K or V tensor [batch][kv_heads][T][d] bf16 on
    the GPU, drawn with torch's seeded generator.  z ~ N(0, I) in float32 on the
    device, times the same per-head factor A as ``head_covariance_factor``
    (float32), rounded to bfloat16 (RNE)."""
    import torch
    B = cfg.batch if n_batch is None else n_batch
    T = cfg.tokens[0] if n_tokens is None else n_tokens
    d = cfg.head_dim
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + cfg.cid * 101 + (1 if which == "k" else 2))
    out = torch.empty((B, cfg.kv_heads, T, d), dtype=torch.bfloat16, device=device)
    facs = [torch.from_numpy(head_covariance_factor(cfg, 0, h, which, seed).astype(np.float32)).to(device)
            for h in range(cfg.kv_heads)]
    for b in range(B):
        for h in range(cfg.kv_heads):
            z = torch.randn((T, d), generator=g, device=device, dtype=torch.float32)
            out[b, h] = (z @ facs[h]).to(torch.bfloat16)
    return out


def layers_kv_on_device(cfg: Config, which: str, layers, n_tokens: int, seed: int = DEFAULT_SEED,
                        device="cuda"):
    """K or V of several layers of one sequence, [len(layers)][kv_heads][T][d] in
    the configuration's dtype on the GPU (layers as the batch dimension, the
    calibration heads of layer l being l * kv_heads + h), drawn with torch's
    seeded generator times each (layer, head)'s factor A."""
    import torch
    d = cfg.head_dim
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + cfg.cid * 101 + (1 if which == "k" else 2) + 7919)
    out = torch.empty((len(layers), cfg.kv_heads, n_tokens, d), dtype=dt, device=device)
    for i, l in enumerate(layers):
        for h in range(cfg.kv_heads):
            a = torch.from_numpy(head_covariance_factor(cfg, l, h, which, seed).astype(np.float32)).to(device)
            z = torch.randn((n_tokens, d), generator=g, device=device, dtype=torch.float32)
            out[i, h] = (z @ a).to(dt)
    return out
