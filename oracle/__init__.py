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
    qjl_band_mask, CompressResult, effective_dim_cumvar, coefficient_of_variation,
    calibration_stability,
)
from .record import record_words, field_offsets, norm_position, pack, unpack  # noqa: F401
from .turboquant import tq_prod_keys, tq_mse_values, tq_mse_unit, tq_calibration  # noqa: F401
from .metrics import cosine, rel_mse, bits_per_coord, compression_ratio  # noqa: F401

# Pin map: every oracle function and the tests that hold it to something other
# than itself (closed forms, printed values, brute force, invariants).  A
# function with no such test would be listed as "parity unpinned"; none is.
PARITY = {
    "second_moment": "pinned: test_second_moment_is_uncentered",
    "eigenbasis": "pinned: planted-basis recovery, R R^T = I, eigen-residuals, sign rule",
    "participation_ratio/effective_dim": "pinned: identity, isotropic rank-k, Wishart mean, "
                                         "half-to-even rounding, PR <= rank",
    "spectral_gap": "pinned: test_spectral_gap",
    "effective_dim_cumvar": "pinned: flat spectrum ceil(f d), geometric closed form, exact "
                            "boundary ties, fraction 1 gives the rank (test_oracle_calib_variants.py)",
    "coefficient_of_variation/calibration_stability": "pinned: two planted spectra of known PR give "
                                                      "|a-b|/(a+b); identical and rescaled splits give 0",
    "water_fill": "pinned: brute-force optimum, monotone widths, real-valued water level, caps, ties",
    "regions": "pinned: hand-worked map; uniform vs Gaussian laws at equal width give the "
               "closed-form Lloyd-Max levels of each law (test_oracle_regions_bands_tq.py)",
    "lloyd_max_samples": "pinned: midpoint and cell-mean conditions by direct masks, "
                         "convergence to Max (1960)",
    "lloyd_max_gaussian/gaussian_distortion": "pinned: Max (1960) table, closed form vs sampling",
    "quantize": "pinned: brute-force nearest centroid, tie and NaN rules",
    "compress (QJL, gamma)": "pinned: estimator mean and variance over 6000 sketches",
    "dequantize/scores_plain/scores_rotated": "pinned: the two score routes agree; S = 0 identity",
    "softmax/attend": "pinned: sum p = 1, one-hot limit, linearity",
    "band_mask/qjl_band_mask": "pinned: brute-force distance loops",
    "pack/unpack/record_words": "pinned: hand-worked word, brute-force bit writer",
    "tq_mse_unit/tq_mse_values": "pinned: scos-lab distortion table; nearest Max level",
    "tq_prod_keys": "pinned: estimator unbiased with closed-form variance over 5000 sketches",
    "tq_calibration (normalised pipeline)": "pinned: codes equal the nearest-level rule; reconstructions "
                                            "equal tq_prod_keys / tq_mse_values to the half rounding "
                                            "of the stored norms",
    "normalised variant (calibrate/compress normalize)": "pinned: codes invariant under scaling; "
                                                         "reconstruction scales with the vector",
    "cosine/rel_mse/bits_per_coord/compression_ratio": "pinned: README headline ratios; "
                                                       "SQ > TQ ordering on every workload",
}
