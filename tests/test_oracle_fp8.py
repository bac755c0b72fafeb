"""Pins of the fp8 (e4m3) cache oracle (oracle/fp8_cache.py).

The pages fix no quantization scheme; the format is the OCP E4M3 8-bit
float and the rounding a stated reading.  Pinned by hand-derived codes
(tests/golden/e4m3.json), round trips of every code, the nearest-value and
half-ulp properties checked by brute force, and torch's own float8_e4m3fn
conversion (a library routine) inside the finite range."""

import json
import os

import numpy as np
import pytest
import torch

from oracle.fp8_cache import (E4M3_MAX, E4M3_VALUES, dequantize_rows_fp8, e4m3_decode, e4m3_encode,
                              quantize_rows_fp8, seen_rows_fp8)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e4m3.json")))


def test_golden_codes():
    for c in GOLDEN["cases"]:
        got = int(e4m3_encode(np.array([c["x"]]))[0])
        assert got == int(c["code"], 16), (c, hex(got))


def test_every_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes)
    assert np.array_equal(e4m3_encode(vals), codes)
    assert np.nanmax(np.abs(E4M3_VALUES)) == E4M3_MAX
    assert np.isnan(E4M3_VALUES[0x7F]) and np.isnan(E4M3_VALUES[0xFF])


def test_nearest_and_half_ulp_by_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000) * 50, rng.uniform(-0.02, 0.02, 2000)])
    got = e4m3_decode(e4m3_encode(x))
    finite = E4M3_VALUES[np.isfinite(E4M3_VALUES)]
    best = np.abs(x[:, None] - finite[None, :]).min(axis=1)
    assert np.allclose(np.abs(x - got), best, rtol=0, atol=0)  # no representable value is closer
    normal = np.abs(x) >= 2.0 ** -6
    assert (np.abs(x - got)[normal] <= 2.0 ** -4 * np.abs(x[normal])).all()
    assert (np.abs(x - got)[~normal] <= 2.0 ** -10).all()


def test_monotone_and_clamped():
    x = np.linspace(-600, 600, 20001)
    v = e4m3_decode(e4m3_encode(x))
    assert (np.diff(v) >= 0).all()
    assert v.max() == 448 and v.min() == -448


def test_matches_torch_float8_in_range():
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    x = (torch.randn(8192, generator=torch.Generator().manual_seed(5)) * 60).clamp(-448, 448)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x.double().numpy()), ref)


def test_scaled_rows_and_seen_values():
    x = np.random.default_rng(4).standard_normal((6, 64)) * 3
    for scale in (1.0, 0.25, 4.0):
        codes = quantize_rows_fp8(x, scale)
        assert np.array_equal(codes, e4m3_encode(x / scale))
        assert np.array_equal(dequantize_rows_fp8(codes, scale), e4m3_decode(codes) * scale)
        assert np.array_equal(seen_rows_fp8(x, True, scale), dequantize_rows_fp8(codes, scale))
        assert np.array_equal(seen_rows_fp8(x, False, scale), x)
    with pytest.raises(ValueError):
        quantize_rows_fp8(x, 0.3)


def test_golden_scaled_codes_and_seen_values():
    """Hand-derived scaled cases (tests/golden/e4m3.json, scaled_cases): the
    code of x / scale and the stored value code * scale, through every
    scaled entry of the oracle.  A scale applied in the wrong direction, or
    not at all on decode, fails them."""
    for c in GOLDEN["scaled_cases"]:
        x, scale, code, seen = c["x"], c["scale"], int(c["code"], 16), c["seen"]
        got = quantize_rows_fp8(np.array([[x]]), scale)
        assert int(got[0, 0]) == code, (c, hex(int(got[0, 0])))
        assert dequantize_rows_fp8(np.array([[code]], dtype=np.uint8), scale)[0, 0] == seen, c
        assert seen_rows_fp8(np.array([[x]]), True, scale)[0, 0] == seen, c
        assert seen_rows_fp8(np.array([[x]]), False, scale)[0, 0] == x, c
