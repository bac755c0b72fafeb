"""Pins of the fp64 oracle against things other than itself.

Each check below uses an independent source of truth: hand-derived fixtures
(tests/golden), the token-at-a-time cache simulator, closed forms, a library
routine (torch fp64 scaled_dot_product_attention with causal or explicit
boolean masks built by torch itself), and pure-Python brute force on tiny
inputs.  The oracle's own allowed-set rule is never used to build an
expected value.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (
    CacheSimulator,
    allowed_positions,
    attend_rows,
    attention_weights_row,
    mixed_attention,
    streaming_slot_of_position,
    streaming_slot_positions,
)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- fixtures

def test_golden_allowed_sets(golden_dir):
    fx = _load(golden_dir, "tiny_streaming_sets.json")
    for case in fx["cases"]:
        for t, expect in case["allowed"].items():
            got = allowed_positions(int(t), False, case["sink"], case["recent"])
            assert got.tolist() == expect, (case["sink"], case["recent"], t)
            # retrieval heads see every position up to t
            assert allowed_positions(int(t), True, case["sink"], case["recent"]).tolist() == \
                list(range(int(t) + 1))


def test_golden_slot_contents(golden_dir):
    fx = _load(golden_dir, "tiny_streaming_sets.json")
    for case in fx["cases"]:
        s, w = case["sink"], case["recent"]
        for n, expect in case["slots_after_n_tokens"].items():
            assert streaming_slot_positions(int(n), s, w).tolist() == expect
            sim = CacheSimulator(s, w)
            for _ in range(int(n)):
                sim.append()
            assert sim.slot_positions().tolist() == expect


def test_worked_example(golden_dir):
    fx = _load(golden_dir, "worked_example_d2.json")
    a = np.array(fx["a"])
    k = np.stack([np.log(a), np.zeros(4)], axis=1)
    v = np.array(fx["values"])
    q = np.zeros((4, 2))
    q[3] = fx["q_t3"]
    for case in fx["cases"]:
        retrieval = case["kind"] == "retrieval"
        out = mixed_attention(q[None, :, None, :], k[None, :, None, :], v[None, :, None, :],
                              [retrieval], case["sink"], case["recent"], scale=1.0, rows=[3])
        np.testing.assert_allclose(out[0, 0, 0], case["output"], rtol=1e-13, atol=1e-13)
        pos = allowed_positions(3, retrieval, case["sink"], case["recent"])
        assert pos.tolist() == case["allowed"]
        w = attention_weights_row(q[3], k[pos], 1.0)
        full_w = np.zeros(4)
        full_w[pos] = w
        np.testing.assert_allclose(full_w, case["weights"], rtol=1e-13, atol=1e-15)


# ------------------------------------------------------ cache simulator pins

@pytest.mark.parametrize("sink,recent", [(0, 1), (0, 5), (1, 1), (3, 4), (4, 64), (7, 3)])
def test_simulator_matches_closed_form(sink, recent):
    sim = CacheSimulator(sink, recent)
    for n in range(1, 3 * (sink + recent) + 5):
        slot = sim.append()
        assert slot == streaming_slot_of_position(n - 1, sink, recent)
        assert sim.slot_positions().tolist() == streaming_slot_positions(n, sink, recent).tolist()


@pytest.mark.parametrize("sink,recent", [(0, 1), (0, 4), (2, 3), (4, 64), (5, 2)])
def test_cache_contents_equal_allowed_set(sink, recent):
    """After token t is stored, a constant-length cache holds exactly what query t may see."""
    sim = CacheSimulator(sink, recent)
    for t in range(3 * (sink + recent) + 3):
        sim.append()
        assert sim.positions().tolist() == allowed_positions(t, False, sink, recent).tolist()
        assert len(sim.positions()) == min(t + 1, sink + recent)


# ------------------------------------------------------------ closed forms

def test_uniform_weights_reveal_allowed_set():
    """Q = 0 gives equal scores, V = I turns each output row into its weight row."""
    n, d = 24, 32
    for sink, recent in [(2, 5), (0, 3), (4, 64), (1, 1)]:
        q = np.zeros((1, n, 2, d))
        k = np.random.default_rng(0).standard_normal((1, n, 2, d))
        v = np.zeros((1, n, 2, d))
        v[0, :, :, :n] = np.eye(n)[:, None, :]
        out = mixed_attention(q, k, v, [True, False], sink, recent)
        sim = CacheSimulator(sink, recent)
        for t in range(n):
            sim.append()
            full = np.zeros(d)
            full[: t + 1] = 1.0 / (t + 1)
            np.testing.assert_allclose(out[0, t, 0], full, rtol=0, atol=1e-15)
            kept = sim.positions()
            stream = np.zeros(d)
            stream[kept] = 1.0 / len(kept)
            np.testing.assert_allclose(out[0, t, 1], stream, rtol=0, atol=1e-15)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(1)
    for n in [1, 2, 7, 100]:
        q = rng.standard_normal(16) * 5
        keys = rng.standard_normal((n, 16))
        w = attention_weights_row(q, keys, 0.25)
        assert abs(w.sum() - 1.0) < 1e-12
        assert np.all(w > 0)


def test_first_position_and_constant_values():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 10, 2, 8))
    k = rng.standard_normal((1, 10, 2, 8))
    v = rng.standard_normal((1, 10, 2, 8))
    out = mixed_attention(q, k, v, [True, False], 1, 3)
    np.testing.assert_array_equal(out[0, 0], v[0, 0])  # t = 0 sees only itself
    vc = np.broadcast_to(rng.standard_normal(8), (1, 10, 2, 8)).copy()
    outc = mixed_attention(q, k, vc, [True, False], 1, 3)
    np.testing.assert_allclose(outc, vc, rtol=1e-14, atol=1e-14)


def test_two_keys_logistic():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 1, 4))
    k = rng.standard_normal((1, 2, 1, 4))
    v = rng.standard_normal((1, 2, 1, 4))
    scale = 0.7
    out = mixed_attention(q, k, v, [True], 0, 8, scale=scale)
    s0 = scale * float(q[0, 1, 0] @ k[0, 0, 0])
    s1 = scale * float(q[0, 1, 0] @ k[0, 1, 0])
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    np.testing.assert_allclose(out[0, 1, 0], (1 - w1) * v[0, 0, 0] + w1 * v[0, 1, 0], rtol=1e-13)



def test_large_scores_stay_finite():
    """Scores near 800 overflow exp() unless the row maximum is subtracted first."""
    q = np.zeros((1, 2, 1, 2))
    q[0, 1, 0] = [1.0, 0.0]
    k = np.array([[800.0, 0.0], [790.0, 0.0]])[None, :, None, :]
    v = np.array([[1.0, 0.0], [0.0, 1.0]])[None, :, None, :]
    out = mixed_attention(q, k, v, [True], 0, 4, scale=1.0, rows=[1])
    w1 = 1.0 / (1.0 + math.exp(10.0))
    np.testing.assert_allclose(out[0, 0, 0], [1.0 - w1, w1], rtol=1e-12)

# ------------------------------------------------------ library special cases

def _sdpa(q, k, v, mask_or_causal, scale):
    """torch fp64 SDPA over [T, D] arrays; mask True = attend."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    if isinstance(mask_or_causal, str):
        o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    else:
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask_or_causal[None, None], scale=scale)
    return o[0, 0].numpy()


def _sim_mask(n, sink, recent):
    """Boolean [n, n] mask whose row t = positions held by a simulated cache after t+1 tokens."""
    m = torch.zeros(n, n, dtype=torch.bool)
    sim = CacheSimulator(sink, recent)
    for t in range(n):
        sim.append()
        m[t, torch.from_numpy(sim.positions())] = True
    return m


@pytest.mark.parametrize("g", [1, 2, 3])
def test_against_torch_sdpa(g):
    rng = np.random.default_rng(10 + g)
    b, n, hkv, d = 2, 45, 3, 16
    hq = hkv * g
    sink, recent = 3, 7
    mask = [True, False, False]
    q = rng.standard_normal((b, n, hq, d))
    k = rng.standard_normal((b, n, hkv, d))
    v = rng.standard_normal((b, n, hkv, d))
    out = mixed_attention(q, k, v, mask, sink, recent)
    scale = 1 / math.sqrt(d)
    band = _sim_mask(n, sink, recent)
    krep = np.repeat(k, g, axis=2)  # query head h reads KV head h // g
    vrep = np.repeat(v, g, axis=2)
    for bi in range(b):
        for h in range(hq):
            ref = _sdpa(q[bi, :, h], krep[bi, :, h], vrep[bi, :, h],
                        "causal" if mask[h // g] else band, scale)
            np.testing.assert_allclose(out[bi, :, h], ref, rtol=1e-12, atol=1e-12)


def test_window_covering_sequence_equals_full():
    rng = np.random.default_rng(4)
    n = 30
    q = rng.standard_normal((1, n, 1, 8))
    k = rng.standard_normal((1, n, 1, 8))
    v = rng.standard_normal((1, n, 1, 8))
    full = mixed_attention(q, k, v, [True], 0, 1)
    for sink, recent in [(0, n), (5, n - 5), (n, 1), (10, 40)]:
        out = mixed_attention(q, k, v, [False], sink, recent)
        np.testing.assert_array_equal(out, full)
    # and a window that is one short of the sequence differs on the last row only
    out = mixed_attention(q, k, v, [False], 0, n - 1)
    np.testing.assert_array_equal(out[:, : n - 1], full[:, : n - 1])
    assert np.abs(out[0, n - 1] - full[0, n - 1]).max() > 1e-6


def test_zero_sinks_is_sliding_window():
    rng = np.random.default_rng(5)
    n, d, recent = 33, 8, 5
    q = rng.standard_normal((1, n, 1, d))
    k = rng.standard_normal((1, n, 1, d))
    v = rng.standard_normal((1, n, 1, d))
    out = mixed_attention(q, k, v, [False], 0, recent)
    ones = torch.ones(n, n, dtype=torch.bool)
    band = torch.tril(ones) & torch.triu(ones, diagonal=-(recent - 1))
    ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0], band, 1 / math.sqrt(d))
    np.testing.assert_allclose(out[0, :, 0], ref, rtol=1e-12, atol=1e-12)


def test_stress_inputs_against_sdpa():
    """Peaky softmax, monotone scores and a planted sink (the case a dropped sink fails)."""
    rng = np.random.default_rng(6)
    n, d, sink, recent = 40, 16, 2, 6
    band = _sim_mask(n, sink, recent)
    cases = []
    q = rng.standard_normal((n, d)) * 8
    cases.append((q, rng.standard_normal((n, d))))
    base = rng.standard_normal(d)
    q2 = np.tile(base, (n, 1))
    k2 = np.outer(np.arange(n) / 4.0, base) + 0.01 * rng.standard_normal((n, d))
    cases.append((q2, k2))
    k3 = rng.standard_normal((n, d))
    k3[0] = base * 3
    cases.append((q2, k3))
    for qq, kk in cases:
        vv = rng.standard_normal((n, d))
        for retrieval in (True, False):
            out = mixed_attention(qq[None, :, None], kk[None, :, None], vv[None, :, None],
                                  [retrieval], sink, recent)
            ref = _sdpa(qq, kk, vv, "causal" if retrieval else band, 1 / math.sqrt(d))
            np.testing.assert_allclose(out[0, :, 0], ref, rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------ brute force

def test_brute_force_tiny():
    """Pure-Python loops with the allowed set taken from the simulated cache."""
    rng = np.random.default_rng(7)
    for sink, recent in [(1, 2), (0, 3), (2, 2), (3, 5)]:
        n, d = 12, 3
        q = rng.standard_normal((1, n, 1, d)).round(3)
        k = rng.standard_normal((1, n, 1, d)).round(3)
        v = rng.standard_normal((1, n, 1, d)).round(3)
        out = mixed_attention(q, k, v, [False], sink, recent, scale=0.5)
        sim = CacheSimulator(sink, recent)
        for t in range(n):
            sim.append()
            kept = [int(p) for p in sim.positions()]
            scores = [0.5 * sum(float(q[0, t, 0, e]) * float(k[0, j, 0, e]) for e in range(d)) for j in kept]
            top = max(scores)
            ex = [math.exp(s - top) for s in scores]
            tot = sum(ex)
            ref = [sum(ex[i] / tot * float(v[0, j, 0, e]) for i, j in enumerate(kept)) for e in range(d)]
            np.testing.assert_allclose(out[0, t, 0], ref, rtol=1e-12, atol=1e-13)


def test_selected_rows_match_all_rows():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((2, 20, 4, 8))
    k = rng.standard_normal((2, 20, 2, 8))
    v = rng.standard_normal((2, 20, 2, 8))
    full = mixed_attention(q, k, v, [False, True], 2, 4)
    rows = [0, 5, 19, 6]
    part = mixed_attention(q, k, v, [False, True], 2, 4, rows=rows)
    np.testing.assert_array_equal(part, full[:, rows])


def test_attend_rows_accepts_low_precision_inputs():
    rng = np.random.default_rng(9)
    k = rng.standard_normal((16, 8)).astype(np.float32)
    v = rng.standard_normal((16, 8)).astype(np.float32)
    q = rng.standard_normal((2, 8)).astype(np.float32)
    out = attend_rows(q, [3, 15], k, v, True, 0, 1, 0.3)
    assert out.dtype == np.float64
    ref = attend_rows(q.astype(np.float64), [3, 15], k.astype(np.float64), v.astype(np.float64),
                      True, 0, 1, 0.3)
    np.testing.assert_array_equal(out, ref)


def test_invalid_arguments():
    with pytest.raises(ValueError):
        allowed_positions(-1, True, 0, 1)
    with pytest.raises(ValueError):
        allowed_positions(3, False, 0, 0)
    with pytest.raises(ValueError):
        CacheSimulator(-1, 2)
    with pytest.raises(ValueError):
        mixed_attention(np.zeros((1, 2, 3, 4)), np.zeros((1, 2, 2, 4)), np.zeros((1, 2, 2, 4)),
                        [True, True], 0, 1)
