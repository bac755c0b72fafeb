"""Error model of the fp8-matrix-core prefill (DUO_FP8_PREFILL_MFMA) and the
bar derived from it.

Beyond the stored K and V (which the oracle already sees through their
e4m3 codes), that kernel rounds two more things to e4m3 and one to bf16:

  * q, after a power-of-two scale per query row: element i gets a relative
    error delta_i with |delta_i| <= u = 2^-4 (e4m3 keeps 4 significant
    bits), so the base-2 score of key j, c <q, k_j> with c = scale log2 e,
    moves by ds_j = c sum_i q_i delta_i k_ji;
  * the softmax weight of key j, p_j = 2^(s_j - mu + 7) with the reference
    mu at most 1.75 below the running maximum (so the largest weight is at
    least 2^7): relative error <= u where p_j >= 2^-6 (normal e4m3), an
    absolute error <= 2^-10 below it (subnormals, spacing 2^-9); the row
    sum l is taken from the same rounded weights, so the output stays a
    convex combination of V rows;
  * the output, rounded to bf16: relative error <= 2^-8.

Model: every rounding error is independent and uniform over its interval,
variance (bound)^2 / 3.  A weight perturbed to p_j (1 + e_j) moves the
output by sum_j w_j e_j (v_j - o) to first order (w_j = p_j / l), where
e_j collects the weight's own rounding and ln 2 ds_j from the score.  So
per output element

    var(o_d) = sum_j var(p_j e_j) (v_jd - o_d)^2 / l^2 + (2^-8)^2 / 3 o_d^2,
    var(p_j e_j) = p_j^2 (u^2 / 3) (1 + (ln 2 c)^2 sum_i q_i^2 k_ji^2)
                   (p_j >= 2^-6; (2^-10)^2 / 3 + the score term below it).

The largest weight is taken as 2^7, the least the kernel allows: more
weights then count as subnormal, which only raises the predicted variance.

The bar, per (sequence, query head) slice of compared rows: the L2 norm of
the error at most twice the predicted RMS norm, and every element within 6
predicted standard deviations.  Uniform rounding errors have a variance
below u^2 / 3 in relative terms, and a sum over the many keys of a row is
close to normal, so a correct kernel sits well inside; a wrong operand,
index or scale moves the output by far more than 2^-4 of its spread.
"""

from __future__ import annotations

import math

import numpy as np

U_E4M3 = 2.0 ** -4
U_BF16 = 2.0 ** -8
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_HALF_SPACING_SUB = 2.0 ** -10
L2_FACTOR = 2.0
MAX_SIGMAS = 6.0


def mfma_sigma(qr, pos, ks, vs, retrieval: bool, sink: int, recent: int, scale: float):
    """Predicted standard deviation of the fp8-MFMA prefill's error, per
    output element.  qr [R, D]: the query rows as the kernel rounds them
    (rotated where rotary embedding applies); pos [R]: their positions;
    ks, vs [T, D]: the stored (e4m3) K and V values by position, T > max(pos).
    Returns [R, D] float64."""
    qr = np.asarray(qr, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    t = int(pos.max()) + 1
    k = np.asarray(ks[:t], dtype=np.float64)
    v = np.asarray(vs[:t], dtype=np.float64)
    c = scale / math.log(2.0)
    s = c * (qr @ k.T)  # [R, T] base-2 scores
    j = np.arange(t)[None, :]
    p_ = pos[:, None]
    ok = j <= p_
    if not retrieval:
        ok &= (j < sink) | (j >= p_ - recent + 1)
    s = np.where(ok, s, -np.inf)
    p = 2.0 ** 7 * np.exp2(s - s.max(axis=1, keepdims=True))  # largest weight 2^7, masked keys 0
    l = p.sum(axis=1)
    o = (p @ v) / l[:, None]
    var_s = (U_E4M3 ** 2 / 3.0) * (math.log(2.0) * c) ** 2 * ((qr ** 2) @ (k ** 2).T)  # [R, T]
    var_p = np.where(p >= E4M3_MIN_NORMAL, (U_E4M3 ** 2 / 3.0) * p ** 2,
                     np.where(ok, E4M3_HALF_SPACING_SUB ** 2 / 3.0, 0.0)) + var_s * p ** 2
    a = var_p @ (v ** 2)
    b = var_p @ v
    cs = var_p.sum(axis=1)[:, None]
    var_o = (a - 2.0 * o * b + o ** 2 * cs) / (l[:, None] ** 2) + (U_BF16 ** 2 / 3.0) * o ** 2
    return np.sqrt(np.maximum(var_o, 0.0))


def assert_fp8_mfma_close(got, ref, sigma, what):
    """got / ref / sigma [R, H, D] for the compared rows of one sequence.
    Returns the worst (L2 ratio, max |d| / sigma) over the heads."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    worst = (0.0, 0.0)
    for hh in range(got.shape[1]):
        d = got[:, hh] - ref[:, hh]
        sg = np.maximum(sigma[:, hh], 1e-12)
        l2 = np.linalg.norm(d) / max(np.sqrt((sg ** 2).sum()), 1e-30)
        mx = float((np.abs(d) / sg).max())
        worst = (max(worst[0], l2), max(worst[1], mx))
        assert l2 <= L2_FACTOR and mx <= MAX_SIGMAS, \
            f"{what} head {hh}: |d|_2 / predicted = {l2:.3f}, max |d| / sigma = {mx:.2f}"
    return worst
