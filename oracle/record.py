"""Bit-dense record layout of one compressed K/V vector (test infrastructure).

The pages ask for a bit-dense cache but fix no layout, so this is the layout
contract of this implementation, written out plainly for the oracle:

  * per (head, token) a record of W 32-bit words, bits numbered LSB-first
    (bit p is bit p % 32 of word p // 32);
  * code fields in eigen-coordinate order i = 0..d-1, b_i bits each, starting
    at bit 0 and packed back to back (a field may straddle two words);
  * then the m QJL bits, bit j = z_j;
  * if m > 0, the residual norm gamma as an IEEE half in bits [32W-16, 32W);
  * for a normalised calibration (per-vector norm, as TurboQuant stores it),
    the vector norm nu as an IEEE half: in bits [32W-32, 32W-16) when m > 0,
    else in bits [32W-16, 32W);
  * W = max(1, ceil((sum b_i + m + 16 [m > 0] + 16 [normalised]) / 32));
    unused bits are 0;
  * storage interleaves words in 64-token blocks: word w of token t is the
    32-bit element ((t // 64) * W + w) * 64 + t % 64 of the head's buffer; T is
    padded to a multiple of 64 and pad tokens are all-zero records.
"""
from __future__ import annotations

import numpy as np


def record_words(widths, m: int, norm: bool = False) -> int:
    bits = int(np.sum(widths)) + int(m) + (16 if m > 0 else 0) + (16 if norm else 0)
    return max(1, -(-bits // 32))


def norm_position(W: int, m: int) -> int:
    """First bit of the 16-bit vector-norm field of a normalised record."""
    return 32 * W - (32 if m > 0 else 16)


def field_offsets(widths) -> np.ndarray:
    w = np.asarray(widths, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(w)[:-1]]) if len(w) else np.zeros(0, np.int64)


def _put(words: np.ndarray, pos: int, width: int, vals: np.ndarray) -> None:
    """OR ``width``-bit values into bit position ``pos`` of every token row."""
    if width == 0:
        return
    v = vals.astype(np.uint64) & np.uint64((1 << width) - 1)
    w, s = pos // 32, pos % 32
    sh = v << np.uint64(s)
    words[:, w] |= sh & np.uint64(0xFFFFFFFF)
    if s + width > 32:
        words[:, w + 1] |= sh >> np.uint64(32)


def _get(words: np.ndarray, pos: int, width: int) -> np.ndarray:
    w, s = pos // 32, pos % 32
    lo = words[:, w]
    hi = words[:, w + 1] if w + 1 < words.shape[1] else np.zeros_like(lo)
    both = lo | (hi << np.uint64(32))
    return ((both >> np.uint64(s)) & np.uint64((1 << width) - 1)).astype(np.int64)


def pack(widths, m: int, codes: np.ndarray, z: np.ndarray, gamma: np.ndarray,
         nu: np.ndarray = None) -> np.ndarray:
    """Records of T tokens -> uint32 buffer of ceil(T/64)*64*W elements.  nu:
    the per-vector norms (float16) of a normalised calibration, else None."""
    widths = np.asarray(widths, dtype=np.int64)
    T = codes.shape[0]
    W = record_words(widths, m, nu is not None)
    Tp = -(-T // 64) * 64
    words = np.zeros((Tp, W), dtype=np.uint64)
    pos = 0
    for i, b in enumerate(widths):
        _put(words[:T], pos, int(b), codes[:, i])
        pos += int(b)
    for j in range(m):
        _put(words[:T], pos + j, 1, z[:, j])
    if m > 0:
        g = np.asarray(gamma, dtype=np.float16).view(np.uint16)
        _put(words[:T], 32 * W - 16, 16, g)
    if nu is not None:
        _put(words[:T], norm_position(W, m), 16, np.asarray(nu, dtype=np.float16).view(np.uint16))
    return (words.astype(np.uint32).reshape(Tp // 64, 64, W)
            .transpose(0, 2, 1).reshape(-1).copy())


def unpack(widths, m: int, packed: np.ndarray, T: int, norm: bool = False):
    """uint32 buffer -> (codes [T, d], z [T, m] uint8, gamma [T] float16), and
    nu [T] float16 as a fourth element when norm is set."""
    widths = np.asarray(widths, dtype=np.int64)
    W = record_words(widths, m, norm)
    Tp = -(-T // 64) * 64
    words = (np.asarray(packed, dtype=np.uint32)[:Tp * W].reshape(Tp // 64, W, 64)
             .transpose(0, 2, 1).reshape(Tp, W)[:T].astype(np.uint64))
    d = len(widths)
    codes = np.zeros((T, d), dtype=np.int64)
    pos = 0
    for i, b in enumerate(widths):
        if b > 0:
            codes[:, i] = _get(words, pos, int(b))
        pos += int(b)
    z = np.zeros((T, m), dtype=np.uint8)
    for j in range(m):
        z[:, j] = _get(words, pos + j, 1)
    if m > 0:
        gamma = _get(words, 32 * W - 16, 16).astype(np.uint16).view(np.float16)
    else:
        gamma = np.zeros(T, dtype=np.float16)
    if norm:
        nu = _get(words, norm_position(W, m), 16).astype(np.uint16).view(np.float16)
        return codes, z, gamma, nu
    return codes, z, gamma
