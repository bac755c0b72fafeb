"""Rotary position embedding applied on the way into the cache (test oracle).

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.

The pages only cite rotary position embedding (the RoFormer entry in the
reference list of the pith.science review page).  The models they evaluate
apply it to q and k before attention.  What this module computes is that
published method, restated:

* head dimension D splits into D/2 pairs; pair i turns by the angle
  p * theta_i at token position p, with theta_i = base^(-2i/D);
* a pair (a, b) becomes (a cos - b sin, a sin + b cos).

Readings taken (none of this is on the pages):

R1. Two pairings are offered: pair i = dims (2i, 2i+1) (interleaved, as in
    the RoFormer formulation) or dims (i, i + D/2) (the half-split layout many
    checkpoints use).  They differ only by a fixed permutation of the dims.
R2. p is the token's absolute position in its sequence (its cache position),
    the same for retrieval and streaming heads: the streaming cache keeps the
    original positions and is not re-indexed.
R3. The angles are exact (fp64 here); the library must stay accurate at
    positions in the millions, where an fp32 product p * theta loses whole
    radians.
R4. K is stored rotated, in the cache's format: bf16 with round to nearest
    even.  Every key that attention uses -- cached, or from the current chunk
    -- is that stored value.  q is rotated and used as is; V is not rotated.
"""

from __future__ import annotations

import numpy as np

INTERLEAVED = 0
HALF = 1


def rope_frequencies(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/D) for the D/2 pairs, float64."""
    if d % 2:
        raise ValueError("head dimension must be even")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def pair_dims(d: int, style: int) -> tuple[np.ndarray, np.ndarray]:
    """The two dims of every pair (reading R1)."""
    i = np.arange(d // 2)
    if style == INTERLEAVED:
        return 2 * i, 2 * i + 1
    if style == HALF:
        return i, i + d // 2
    raise ValueError("unknown pairing")


def apply_rope(x, positions, base: float, style: int) -> np.ndarray:
    """Rotate rows of ``x`` (shape (..., T, D)) at ``positions`` (T,), float64."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.float64)
    d = x.shape[-1]
    ang = pos[:, None] * rope_frequencies(d, base)[None, :]  # (T, D/2)
    c, s = np.cos(ang), np.sin(ang)
    ia, ib = pair_dims(d, style)
    a, b = x[..., ia], x[..., ib]
    out = np.empty_like(x)
    out[..., ia] = a * c - b * s
    out[..., ib] = a * s + b * c
    return out


def round_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 precision (8 significant bits), ties to
    even, returned as float64.  Values stay in bf16's normal range here."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def rotated_qk(q_seq, k_seq, base: float, style: int):
    """The q and K values attention uses for one sequence (readings R2, R4).

    ``q_seq`` (T, Hq, D) and ``k_seq`` (T, Hkv, D) hold the un-rotated rows
    by position 0..T-1.  Returns (q rotated, float64; K rotated and rounded to
    bf16, as float64)."""
    q_seq = np.asarray(q_seq, dtype=np.float64)
    k_seq = np.asarray(k_seq, dtype=np.float64)
    pos = np.arange(q_seq.shape[0])
    qr = np.swapaxes(apply_rope(np.swapaxes(q_seq, 0, 1), pos, base, style), 0, 1)
    kr = np.swapaxes(apply_rope(np.swapaxes(k_seq, 0, 1), pos, base, style), 0, 1)
    return qr, round_bf16(kr)
