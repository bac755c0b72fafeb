"""Pins of the rotary-position-embedding oracle (oracle/rope.py).

The pages only cite rotary position embedding (RoFormer, in the pith.science
review page's reference list); the oracle restates that method.  It is
pinned here by a hand-derived example (tests/golden/rope_d4.json), the
rotation group law, the relative-position property that defines the method,
norm preservation, the fixed permutation between the two pairings, and its
bf16 rounding by hand-derived ties and by torch's own conversion."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.rope import HALF, INTERLEAVED, apply_rope, pair_dims, rope_frequencies, rotated_qk, round_bf16

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rope_d4.json")))


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("style,key", [(INTERLEAVED, "interleaved"), (HALF, "half")])
def test_golden_d4(style, key):
    g = GOLDEN
    out = apply_rope(np.array([g["x"]]), [g["position"]], g["base"], style)[0]
    assert np.allclose(out, g[key]["expected"], rtol=0, atol=1e-14)


def test_position_zero_is_identity():
    x = _rand((5, 64), 1)
    for style in (INTERLEAVED, HALF):
        assert np.array_equal(apply_rope(x, np.zeros(5), 10000.0, style), x)


@pytest.mark.parametrize("style", [INTERLEAVED, HALF])
def test_group_law(style):
    """Turning by p1 then by p2 equals turning by p1 + p2, up to positions of
    a million (the angle is linear in the position)."""
    x = _rand((6, 128), 2)
    p1 = np.array([0, 1, 17, 1000, 300000, 500000])
    p2 = np.array([5, 2, 100, 4095, 700001, 500000])
    two = apply_rope(apply_rope(x, p1, 10000.0, style), p2, 10000.0, style)
    one = apply_rope(x, p1 + p2, 10000.0, style)
    assert np.allclose(two, one, rtol=0, atol=1e-8)


@pytest.mark.parametrize("style", [INTERLEAVED, HALF])
def test_relative_position(style):
    """q at m against k at n depends only on m - n (what rotary embedding
    is for)."""
    q, k = _rand((1, 128), 3), _rand((1, 128), 4)
    ref = (apply_rope(q, [7], 500000.0, style) @ apply_rope(k, [3], 500000.0, style).T).item()
    for s in (1, 100, 12345, 1 << 20):
        got = (apply_rope(q, [7 + s], 500000.0, style) @ apply_rope(k, [3 + s], 500000.0, style).T).item()
        assert abs(got - ref) < 1e-9


def test_pairs_keep_norm():
    x = _rand((9, 64), 5)
    pos = np.arange(9) * 1000
    for style in (INTERLEAVED, HALF):
        y = apply_rope(x, pos, 10000.0, style)
        ia, ib = pair_dims(64, style)
        assert np.allclose(y[:, ia] ** 2 + y[:, ib] ** 2, x[:, ia] ** 2 + x[:, ib] ** 2, rtol=1e-13)


def test_half_is_permuted_interleaved():
    """Half-split pairing = interleaved pairing after moving dim i to 2i and
    dim i + D/2 to 2i + 1."""
    d = 128
    x = _rand((4, d), 6)
    pos = [0, 3, 999, 65537]
    perm = np.empty(d, dtype=np.int64)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    y_half = apply_rope(x, pos, 10000.0, HALF)
    y_int = apply_rope(x[:, perm], pos, 10000.0, INTERLEAVED)
    assert np.allclose(y_half[:, perm], y_int, rtol=0, atol=1e-14)


def test_frequencies_geometric_from_one():
    th = rope_frequencies(128, 10000.0)
    assert th[0] == 1.0
    ratio = th[1:] / th[:-1]
    assert np.allclose(ratio, ratio[0], rtol=1e-13) and ratio[0] < 1


def test_round_bf16_ties_and_torch():
    t = GOLDEN["bf16_ties"]
    assert list(round_bf16(np.array(t["x"]))) == t["expected"]
    x = (torch.randn(4096, generator=torch.Generator().manual_seed(7)) * 3).numpy()  # fp32 values
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x.astype(np.float64)), ref)
    assert round_bf16(np.array([0.0]))[0] == 0.0


def test_rotated_qk_rounds_k_only():
    q, k = _rand((10, 4, 64), 8), _rand((10, 2, 64), 9)
    qr, kr = rotated_qk(q, k, 10000.0, HALF)
    pos = np.arange(10)
    assert np.array_equal(qr[:, 1], apply_rope(q[:, 1], pos, 10000.0, HALF))
    assert np.array_equal(kr[:, 0], round_bf16(apply_rope(k[:, 0], pos, 10000.0, HALF)))
    assert not np.array_equal(kr, apply_rope(np.swapaxes(k, 0, 1), pos, 10000.0, HALF).swapaxes(0, 1))
