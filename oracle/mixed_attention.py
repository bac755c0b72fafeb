"""fp64 definition of DuoAttention's per-head mixed attention (test oracle).

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.

What is computed, by token position only (no cache, ring, chunk or split):

* Retrieval heads attend to every earlier position and to themselves
  (DuoAttention abstract: retrieval heads need full attention across all
  tokens; sourcepulse card, "How It Works": they keep the full KV cache).
* Streaming heads attend only to the attention sinks and to the recent tokens
  (DuoAttention abstract: streaming heads focus on recent tokens and
  attention sinks and do not need full attention).

Readings taken where the pages are silent (the pith.science referee report,
minor comment 3, notes that the cache size and the sink handling have no
equation):

1. The sinks are the first ``sink`` positions of the sequence.
2. The recent window includes the query's own position: a streaming query at
   position t sees positions t-recent+1 .. t.  Together with the sinks that
   is min(t+1, sink+recent) positions, which is exactly what a constant-length
   cache of sink+recent slots can hold once the new token is stored.
3. Sinks and window may overlap while t < sink+recent; the allowed set is
   their union, so no position is counted twice.
4. Query head h belongs to KV head h // G with G = Hq / Hkv (grouped-query
   attention); all query heads of a group share that KV head's type.
5. No positional encoding is applied inside the path; ``scale`` defaults to
   1/sqrt(D).
6. Scores of positions outside the allowed set are excluded (weight exactly
   zero), not given a large negative value.

Arithmetic is float64 throughout; inputs of any float dtype are converted to
float64 slice by slice, so large contexts do not need a float64 copy of the
whole cache.
"""

from __future__ import annotations

import math

import numpy as np


def allowed_positions(t: int, retrieval: bool, sink: int, recent: int) -> np.ndarray:
    """Positions that a query at position ``t`` attends to (readings 1-3).

    Retrieval: 0..t.  Streaming: {j <= t : j < sink or j >= t - recent + 1}.
    Returned in increasing order as an int64 array.
    """
    if t < 0:
        raise ValueError("query position must be >= 0")
    if sink < 0 or recent < 1:
        raise ValueError("need sink >= 0 and recent >= 1")
    j = np.arange(t + 1, dtype=np.int64)
    if retrieval:
        return j
    keep = (j < sink) | (j >= t - recent + 1)
    return j[keep]


def attention_weights_row(q, keys, scale: float) -> np.ndarray:
    """Softmax weights of one query over the given key rows.

    ``q`` is [D]; ``keys`` is [n, D] holding exactly the allowed keys.  The
    score of key j is scale * <q, k_j>; the weights are exp(s_j - max s)
    normalised to sum to one.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    s = scale * (keys @ q)
    e = np.exp(s - s.max())
    return e / e.sum()


def attend_rows(q_rows, t_rows, k_seq, v_seq, retrieval: bool, sink: int,
                recent: int, scale: float) -> np.ndarray:
    """Attention output of several queries of ONE head of ONE sequence.

    ``q_rows`` [R, D]: the queries; ``t_rows`` [R]: their positions.
    ``k_seq``/``v_seq`` [T, D]: that head's keys/values indexed by position
    (T > max(t_rows)).  Returns float64 [R, D].
    """
    q_rows = np.asarray(q_rows)
    out = np.empty((len(t_rows), q_rows.shape[-1]), dtype=np.float64)
    for i, t in enumerate(t_rows):
        a = allowed_positions(int(t), retrieval, sink, recent)
        w = attention_weights_row(q_rows[i], k_seq[a], scale)
        out[i] = w @ np.asarray(v_seq[a], dtype=np.float64)
    return out


def mixed_attention(q, k, v, kv_is_retrieval, sink: int, recent: int,
                    scale: float | None = None, rows=None) -> np.ndarray:
    """DuoAttention mixed attention of every (or selected) query position.

    ``q``: [B, T, Hq, D]; ``k``, ``v``: [B, T, Hkv, D]; position = index on
    axis 1.  ``kv_is_retrieval``: [Hkv] booleans (reading 4).  ``rows``:
    optional positions to evaluate (default: all T).  Returns float64
    [B, len(rows), Hq, D].
    """
    q = np.asarray(q)
    b_n, t_n, hq, d = q.shape
    hkv = k.shape[2]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(t_n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((b_n, len(rows), hq, d), dtype=np.float64)
    for b in range(b_n):
        for h in range(hq):
            kvh = h // g
            out[b, :, h, :] = attend_rows(q[b, rows, h, :], rows, k[b, :, kvh, :],
                                          v[b, :, kvh, :], bool(kv_is_retrieval[kvh]),
                                          sink, recent, scale)
    return out
