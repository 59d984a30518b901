"""CPU oracle for the SpectralQuant KV-cache hot path -- TEST INFRASTRUCTURE.

This package is a plain, slow, float64 NumPy statement of what SpectralQuant
computes: calibration (second-moment matrix, eigendecomposition, participation
ratio d_eff, spectral gap, reverse water-filling of the bit budget, per-region
Lloyd-Max codebooks), compression (rotation, per-coordinate quantisation,
selective QJL on the signal dimensions, bit-dense record packing), and the
decode-time read side (dequantisation, q.k scores, softmax-weighted value sum),
plus a TurboQuant-style random-rotation baseline and the quality metrics.

It exists only to check the GPU library.  Only the test suite, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
It shares no code, tables or constants with the HIP library and imports
nothing from it.

Sources (cited by page title and section in each function):
  * "SpectralQuant" README (Overview, Repository Structure, Headline Results).
  * spectralquant ``tests/conftest.py`` (fixture ``pre_computed_calibration``:
    uncentered second moment, eigh reversed to descending order, d_eff as the
    rounded participation ratio, spectral gap).
  * the ossradar.top summary of the repository (core capabilities: spectral
    rotation, QJL only on signal dimensions, water-filled non-uniform bit
    allocation, Lloyd-Max codebooks per region).
  * the scos-lab "TurboQuant" README (Algorithm Correctness distortion table,
    Project Structure: MSE/Prod quantisers, random rotation, QJL).

Where the pages leave a step open, the reading taken is stated at the function.
Parity status of every function is listed in ``PARITY`` below.
"""
from .spectralquant import (  # noqa: F401
    Calibration, calibrate, second_moment, eigenbasis, participation_ratio,
    effective_dim, spectral_gap, water_fill, regions, lloyd_max_samples,
    lloyd_max_gaussian, gaussian_distortion, rotate, quantize, compress,
    dequantize, scores_plain, scores_rotated, softmax, attend, band_mask,
    qjl_band_mask, CompressResult,
)
from .record import record_words, field_offsets, pack, unpack  # noqa: F401
from .turboquant import tq_prod_keys, tq_mse_values, tq_mse_unit  # noqa: F401
from .metrics import cosine, rel_mse, bits_per_coord, compression_ratio  # noqa: F401

# Every oracle function is pinned by at least one test in tests/test_oracle_*.py
# against something other than itself (closed forms, printed values, brute
# force, invariants).  The exceptions are listed here and in the design notes.
PARITY = {
    "calibrate": "pinned",
    "lloyd_max_samples": "pinned",
    "lloyd_max_gaussian": "pinned",
    "water_fill": "pinned",
    "compress": "pinned",
    "dequantize": "pinned",
    "scores_plain": "pinned",
    "scores_rotated": "pinned",
    "attend": "pinned",
    "pack/unpack": "pinned",
    "tq_prod_keys/tq_mse_values": "pinned",
}
