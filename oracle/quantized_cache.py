"""int8 retrieval KV cache: quantisation, and the K/V values attention sees (test oracle).

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.

The pages say DuoAttention reaches a 3.3-million-token context on one GPU
when it is combined with quantization (abstract as reproduced on the
pith.science review page; sourcepulse card, "Highlighted Details"; ajithp.com
blog, "Performance and Efficiency Gains" and "DuoAttention Implementation
Details", item 5).  They do not say which scheme; the review page cites KV
quantization work (KIVI, KVQuant, QServe) only in its reference list.  The
readings taken here:

Q1. Only the retrieval heads' cached K and V rows are quantized.  The
    streaming heads' caches are constant-length and stay bf16.
Q2. A row is the D values of one (sequence, KV head, position).  Symmetric
    int8 with one fp32 scale per row, every step in fp32 with round to
    nearest even:
        amax  = max_d |x_d|
        scale = amax / 127
        code_d = clamp(rint(x_d / scale), -127, 127)      (rint: halves to even)
    A zero row has scale 0 and codes 0.  Codes are stored as offset-binary
    bytes code + 128 (so byte 128 is zero).
Q3. The dequantized value is code * scale.
Q4. A call sees the rows that earlier calls stored through their dequantized
    values, and the rows of its own chunk (or its decode token) at input
    precision: those are the call's inputs.  So with a quantized cache a
    chunked prefill differs from a one-shot prefill, by the quantization of
    the rows stored between the chunks.

The quantization decides integers from floating point, so this module takes
those decisions in fp32, the precision the GPU kernels use, and the codes and
scales are compared bit for bit.  Attention itself stays fp64
(``mixed_attention``), on the K/V values this module hands it.
"""

from __future__ import annotations

import numpy as np

QMAX = 127
OFFSET = 128


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantize the rows of ``x`` (shape (..., D), any real dtype whose values
    are exact in fp32, e.g. bf16 data) following Q2.

    Returns (codes uint8 (..., D) offset-binary, scales float32 (...))."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = (amax / np.float32(QMAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (x32 / safe[..., None]).astype(np.float32)
    q = np.clip(np.rint(ratio), -QMAX, QMAX)  # a zero row: ratio 0, code 0
    codes = (q.astype(np.int32) + OFFSET).astype(np.uint8)
    return codes, scale


def dequantize_rows(codes, scales) -> np.ndarray:
    """code * scale (Q3) in float64, shape (..., D)."""
    c = np.asarray(codes, dtype=np.int64) - OFFSET
    return c.astype(np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def seen_rows(x_seq, retrieval: bool, stored_before: int) -> np.ndarray:
    """The K (or V) values of one (sequence, KV head) that a call sees (Q1, Q4).

    ``x_seq`` [T, D] holds the sequence's rows by position; positions below
    ``stored_before`` were stored by earlier calls.  Retrieval heads see those
    rows dequantized; every other row, and every row of a streaming head, is
    seen as given.  Returns float64 [T, D]."""
    out = np.array(x_seq, dtype=np.float64, copy=True)
    if retrieval and stored_before > 0:
        codes, scales = quantize_rows(np.asarray(x_seq)[:stored_before])
        out[:stored_before] = dequantize_rows(codes, scales)
    return out
