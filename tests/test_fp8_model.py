"""CPU pins of the fp8-matrix-core prefill's error model (tests/fp8_model.py).

The kernel's arithmetic on the values it rounds is emulated in numpy (fp64
around the roundings): q scaled by scale * log2 e and a power of two that
puts its largest magnitude in [224, 448), rounded to e4m3; base-2 scores
against the stored K; weights 2^(s - mu + 7) rounded to e4m3 with mu the
row maximum; the row sum from the rounded weights; the output rounded to
bf16.  Against the oracle (fp64 over the stored values) such an emulation
must sit inside the model's bar with room to spare, and plausible mistakes
must fall outside it: a K scale applied twice, weights rounded to 2
significant bits instead of 4, a window one position short."""

import math

import numpy as np
import pytest

from fp8_model import L2_FACTOR, MAX_SIGMAS, assert_fp8_mfma_close, mfma_sigma
from oracle import attend_rows
from oracle.fp8_cache import e4m3_decode, e4m3_encode, seen_rows_fp8


def round_sig(x, bits):
    """Round to `bits` significant bits, nearest (ties away; only a planted
    mistake uses this)."""
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 2.0 ** bits) / 2.0 ** bits, e)


def round_bf16(x):
    return round_sig(x, 8)


def emulate(q_rows, pos, ks, vs, retrieval, sink, recent, scale, weight_bits=None, k_scale_twice=1.0,
            window_short=0):
    c = scale / math.log(2.0)
    out = np.empty((len(pos), q_rows.shape[1]))
    for r, t in enumerate(pos):
        qc = q_rows[r] * c
        e = math.floor(math.log2(np.abs(qc).max() / 224.0))
        q8 = e4m3_decode(e4m3_encode(qc * 2.0 ** -e)) * 2.0 ** e
        j = np.arange(t + 1)
        keep = (j < sink) | (j >= t - (recent - window_short) + 1) if not retrieval else np.ones(t + 1, bool)
        a = j[keep]
        s = (ks[a] * k_scale_twice) @ q8
        x = 2.0 ** (s - s.max() + 7)
        p = e4m3_decode(e4m3_encode(x)) if weight_bits is None else round_sig(x, weight_bits)
        out[r] = round_bf16((p @ vs[a]) / p.sum())
    return out


def case(seed, n, d, q_mul, retrieval, sink=4, recent=64, rows=24):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, d)) * q_mul
    k = seen_rows_fp8(rng.standard_normal((n, d)), True, 1.0)
    v = seen_rows_fp8(rng.standard_normal((n, d)), True, 1.0)
    pos = sorted(set([0, 1, n - 1] + rng.integers(0, n, rows).tolist()))
    scale = 1.0 / math.sqrt(d)
    ref = attend_rows(q[pos], pos, k, v, retrieval, sink, recent, scale)
    sig = mfma_sigma(q[pos], pos, k, v, retrieval, sink, recent, scale)
    return q, k, v, pos, scale, ref, sig


CASES = [(1, 2048, 128, 1.0, True), (2, 1500, 64, 1.0, True), (3, 1024, 128, 8.0, True),
         (4, 900, 128, 1.0, False), (5, 4096, 128, 0.3, True)]


@pytest.mark.parametrize("seed,n,d,q_mul,retrieval", CASES)
def test_emulated_kernel_sits_inside_the_bar(seed, n, d, q_mul, retrieval):
    q, k, v, pos, scale, ref, sig = case(seed, n, d, q_mul, retrieval)
    got = emulate(q[pos], pos, k, v, retrieval, 4, 64, scale)
    l2, mx = assert_fp8_mfma_close(got[:, None], ref[:, None], sig[:, None], "emulated")
    assert l2 <= 0.75 * L2_FACTOR and mx <= 0.8 * MAX_SIGMAS, (l2, mx)


@pytest.mark.parametrize("mistake", ["k_scale_twice", "weights_2_bits", "window_short"])
def test_planted_mistakes_fail_the_bar(mistake):
    q, k, v, pos, scale, ref, sig = case(7, 2048, 128, 1.0, mistake != "window_short")
    kw = {"k_scale_twice": dict(k_scale_twice=2.0), "weights_2_bits": dict(weight_bits=2),
          "window_short": dict(window_short=1)}[mistake]
    got = emulate(q[pos], pos, k, v, mistake != "window_short", 4, 64, scale, **kw)
    with pytest.raises(AssertionError):
        assert_fp8_mfma_close(got[:, None], ref[:, None], sig[:, None], mistake)


def test_exact_rows_have_only_the_output_rounding():
    """t = 0: one key, weight 1 -- the output is the stored value itself,
    which bf16 holds exactly; the model predicts only the output rounding."""
    q, k, v, pos, scale, ref, sig = case(9, 64, 128, 1.0, True)
    i = pos.index(0)
    assert np.allclose(sig[i], np.sqrt((2.0 ** -8) ** 2 / 3.0) * np.abs(v[0]), rtol=1e-12, atol=0)
    got = emulate(q[[0]], [0], k, v, True, 4, 64, scale)
    assert np.array_equal(got[0], v[0])
