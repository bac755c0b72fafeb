"""Pins of the int8 retrieval-cache oracle (oracle/quantized_cache.py).

The pages fix no quantization scheme (abstract on the pith.science review
page: 3.3M context 'combined with quantization'), so the scheme is the
reading stated in the oracle; these tests pin the oracle to that reading by
hand-derived rows, closed-form bounds and invariants, and to the unquantized
oracle where quantization is exact."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import mixed_attention
from oracle.quantized_cache import OFFSET, QMAX, dequantize_rows, quantize_rows, seen_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8_rows.json")


def bf16_rows(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).float().numpy()


def test_golden_rows():
    rows = json.load(open(GOLDEN))["rows"]
    for r in rows:
        codes, scale = quantize_rows(np.array(r["x"], dtype=np.float32))
        assert list(codes) == r["codes"], r["name"]
        assert float(scale) == r["scale_num"] / r["scale_den"], r["name"]


def test_error_bound_and_extreme_code():
    x = bf16_rows((64, 128), 1)
    codes, scales = quantize_rows(x)
    xh = dequantize_rows(codes, scales)
    err = np.abs(xh - x)
    # |x - code*scale| <= scale/2, plus the fp32 rounding of x/scale (tiny)
    assert np.all(err <= scales[:, None] * (0.5 + 1e-5))
    c = codes.astype(np.int64) - OFFSET
    assert np.all(np.abs(c) <= QMAX)
    # the element of largest magnitude maps to +-127
    i = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(c[np.arange(64), i]) == QMAX)
    assert np.all(np.sign(c[np.arange(64), i]) == np.sign(x[np.arange(64), i]))


def test_symmetry_and_power_of_two_invariance():
    x = bf16_rows((32, 64), 2)
    c1, s1 = quantize_rows(x)
    c2, s2 = quantize_rows(-x)
    assert np.array_equal(c1.astype(np.int64) - OFFSET, -(c2.astype(np.int64) - OFFSET))
    assert np.array_equal(s1, s2)
    c3, s3 = quantize_rows(x * 4.0)  # exact in fp32: every quotient unchanged
    assert np.array_equal(c1, c3)
    assert np.array_equal(s3, s1 * np.float32(4.0))


def test_zero_row_and_single_value():
    c, s = quantize_rows(np.zeros((3, 8), np.float32))
    assert np.all(c == OFFSET) and np.all(s == 0)
    x = np.zeros((1, 8), np.float32)
    x[0, 5] = -0.75
    c, s = quantize_rows(x)
    assert c[0, 5] == OFFSET - QMAX and np.all(np.delete(c[0], 5) == OFFSET)
    assert dequantize_rows(c, s)[0, 5] == pytest.approx(-0.75, rel=1e-6)


def test_seen_rows_provenance():
    x = bf16_rows((40, 16), 3)
    # streaming heads: untouched whatever was stored before
    assert np.array_equal(seen_rows(x, False, 40), x.astype(np.float64))
    y = seen_rows(x, True, 25)
    assert np.array_equal(y[25:], x[25:].astype(np.float64))  # the call's own rows
    c, s = quantize_rows(x[:25])
    assert np.array_equal(y[:25], dequantize_rows(c, s))
    assert not np.array_equal(y[:25], x[:25])  # N(0,1) rows are not exactly representable
    assert np.array_equal(seen_rows(x, True, 0), x.astype(np.float64))


def test_exact_rows_give_unquantized_attention():
    """Integer-valued rows whose largest magnitude is 127 quantize exactly
    (scale 1), so attention over the rows a quantized cache returns equals the
    unquantized oracle bit for bit."""
    rng = np.random.default_rng(4)
    T, H, D = 24, 2, 16
    k = rng.integers(-127, 128, size=(1, T, H, D)).astype(np.float64)
    v = rng.integers(-127, 128, size=(1, T, H, D)).astype(np.float64)
    k[..., 0] = 127.0
    v[..., 1] = -127.0
    q = rng.standard_normal((1, T, H, D)) * 0.01
    ref = mixed_attention(q, k, v, [1, 0], sink=2, recent=5)
    ks = np.stack([seen_rows(k[0, :, h], h == 0, 17) for h in range(H)], axis=1)[None]
    vs = np.stack([seen_rows(v[0, :, h], h == 0, 17) for h in range(H)], axis=1)[None]
    assert np.array_equal(ks, k) and np.array_equal(vs, v)
    out = mixed_attention(q, ks, vs, [1, 0], sink=2, recent=5)
    assert np.array_equal(out, ref)


def test_quantized_attention_close_to_unquantized():
    """Dequantization error of N(0,1) rows stays within the bf16-level
    tolerance the parity tests use (a sanity check of the scheme, not of the
    GPU)."""
    T, H, D = 96, 2, 64
    q = bf16_rows((1, T, H, D), 5)
    k = bf16_rows((1, T, H, D), 6)
    v = bf16_rows((1, T, H, D), 7)
    ref = mixed_attention(q, k, v, [1, 1], sink=4, recent=16)
    ks = np.stack([seen_rows(k[0, :, h], True, T) for h in range(H)], axis=1)[None]
    vs = np.stack([seen_rows(v[0, :, h], True, T) for h in range(H)], axis=1)[None]
    out = mixed_attention(q, ks, vs, [1, 1], sink=4, recent=16)
    d = np.abs(out - ref)
    assert d.max() < 2e-2
    assert np.linalg.norm(d) / np.linalg.norm(ref) < 1e-2
