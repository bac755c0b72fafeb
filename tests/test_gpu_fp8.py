"""GPU parity of the fp8 (e4m3) retrieval cache and its fp8 prefill.

Bit-exact: every stored retrieval row's codes equal the oracle's encoding
(oracle/fp8_cache.py, readings E2-E3); streaming slots hold the bf16 input.
Decode attends through the stored values in fp32 (q enters as an exact f16
multiple), so it is held to the usual bar against the oracle on those
values (reading E4).  Retrieval heads' prefill runs on fp8 matrix cores and
rounds two more things to e4m3: q (after a power-of-two scale per query
row) and the softmax weights.  Each rounding is at most 2^-4 relative; an
output row is a convex combination of V rows, so the weights' rounding moves
it by at most about 2^-4 of the spread of those rows, and q's rounding
moves every score by at most 2^-4 of sum |q_i k_i| scale.  The fp8 bar
below is per (sequence, query head): max |d| <= 2^-3 * max |V| of the head
and ||d|| / ||ref|| <= 2^-4.  Streaming heads keep the bf16 path and the
usual bar.  Inputs scaled with the tensor scales are compared in units of
the V scale (the output is linear in V).  Every cache buffer starts as NaN
bytes."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from oracle import attend_rows, streaming_slot_positions
from oracle.fp8_cache import quantize_rows_fp8, seen_rows_fp8
from parity_util import assert_close, require_gpu, run_sequence, to_np32
from workloads import qkv

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-fp8] {msg}", flush=True)


def new_cache_fp8(batch, hq, hkv, d, max_len, sink, recent, mask, sk=1.0, sv=1.0, **kw):
    cfg = duo.Config(batch, hq, hkv, d, max_len, sink, recent, [int(x) for x in mask], kv_format=duo.DUO_KV_FP8,
                     kv_scale_k=sk, kv_scale_v=sv, **kw)
    buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
    return duo.duo_cache_init(cfg, buf)


def oracle_fp8(q, k, v, mask, sink, recent, rows_by_b, sk, sv):
    b_n, _t, hq, d = q.shape
    hkv = k.shape[2]
    g = hq // hkv
    scale = 1.0 / math.sqrt(d)
    out = {}
    for b in range(b_n):
        rows = np.asarray(rows_by_b[b], dtype=np.int64)
        if len(rows) == 0:
            continue
        tmax = int(rows.max()) + 1
        res = np.empty((len(rows), hq, d))
        for kvh in range(hkv):
            ks = seen_rows_fp8(k[b, :tmax, kvh], bool(mask[kvh]), sk)
            vs = seen_rows_fp8(v[b, :tmax, kvh], bool(mask[kvh]), sv)
            for h in range(kvh * g, (kvh + 1) * g):
                res[:, h] = attend_rows(q[b, rows, h], rows, ks, vs, bool(mask[kvh]), sink, recent, scale)
        out[b] = res
    return out


def assert_fp8_close(got, ref, vmax, what):
    """The fp8 prefill bar (module docstring); got/ref [rows, H, D]."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    worst = (0.0, 0.0)
    for hh in range(got.shape[1]):
        d = got[:, hh] - ref[:, hh]
        mx = np.abs(d).max()
        rel = np.linalg.norm(d) / max(np.linalg.norm(ref[:, hh]), 1e-30)
        worst = (max(worst[0], mx / vmax[hh]), max(worst[1], rel))
        assert mx <= 2.0 ** -3 * vmax[hh] and rel <= 2.0 ** -4, f"{what} head {hh}: max|d|={mx:.3e} relL2={rel:.3e}"
    return worst


def check_cache_fp8(cache, k32, v32, k_bf, v_bf, mask, n_tokens, sk, sv):
    views = duo.cache_views(cache)
    cfg = cache.cfg
    hidx = cache.head_index()
    assert views["lengths"].cpu().tolist() == list(n_tokens)
    rk, rv = views["rk"].cpu().numpy(), views["rv"].cpu().numpy()
    sk_, sv_ = views["sk"].view(torch.int16).cpu(), views["sv"].view(torch.int16).cpu()
    kb, vb = k_bf.view(torch.int16).cpu(), v_bf.view(torch.int16).cpu()
    for b in range(cfg.batch):
        n = n_tokens[b]
        slots = streaming_slot_positions(n, cfg.sink, cfg.recent)
        for kvh in range(cfg.num_kv_heads):
            i = hidx[kvh]
            if mask[kvh]:
                assert np.array_equal(rk[b, i, :n], quantize_rows_fp8(k32[b, :n, kvh], sk)), f"k codes b{b} kv{kvh}"
                assert np.array_equal(rv[b, i, :n], quantize_rows_fp8(v32[b, :n, kvh], sv)), f"v codes b{b} kv{kvh}"
            else:
                for s, p in enumerate(slots):
                    if p >= 0:
                        assert torch.equal(sk_[b, i, s], kb[b, p, kvh]), f"sk b{b} kv{kvh} slot{s}"
                        assert torch.equal(sv_[b, i, s], vb[b, p, kvh]), f"sv b{b} kv{kvh} slot{s}"


def run_fp8(cache, q, k, v, mask, chunks, steps, sk, sv, what):
    cfg = cache.cfg
    outp, outd, done = run_sequence(cache, q, k, v, chunks, steps)
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    b_n = q.shape[0]
    pre = [sum(c[b] for c in chunks) for b in range(b_n)]
    ref = oracle_fp8(qn, kn, vn, mask, cfg.sink, cfg.recent, {b: list(range(pre[b] + steps)) for b in range(b_n)},
                     sk, sv)
    g = cfg.num_q_heads // cfg.num_kv_heads
    worst = (0.0, 0.0)
    for b in range(b_n):
        if pre[b]:
            got = to_np32(outp[b, :pre[b]])
            r = ref[b][:pre[b]]
            retr = [h for h in range(cfg.num_q_heads) if mask[h // g]]
            strm = [h for h in range(cfg.num_q_heads) if not mask[h // g]]
            if retr:
                vmax = [np.abs(seen_rows_fp8(vn[b, :pre[b], h // g], True, sv)).max() for h in retr]
                w = assert_fp8_close(got[:, retr], r[:, retr], vmax, f"{what} prefill b{b}")
                worst = (max(worst[0], w[0]), max(worst[1], w[1]))
            if strm:  # the output is linear in V: compare in units of the V scale
                assert_close(got[:, strm] / sv, r[:, strm] / sv, f"{what} prefill streaming b{b}")
        if steps:
            assert_close(to_np32(outd[:, b]) / sv, ref[b][pre[b]:] / sv, f"{what} decode b{b}")
    _say(f"{what}: fp8 prefill worst max|d|/max|V| = {worst[0]:.3e}, relL2 = {worst[1]:.3e}")
    check_cache_fp8(cache, kn, vn, k, v, mask, done, sk, sv)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_chunked_prefill_and_decode(d):
    require_gpu()
    _say(f"chunked d={d}")
    mask = [1, 0, 1, 0]
    q, k, v = qkv(2, 430, 8, 4, d, 91, "cuda")
    cache = new_cache_fp8(2, 8, 4, d, 430, 4, 16, mask)
    run_fp8(cache, q, k, v, mask, [[100, 50], [64, 1], [1, 63], [65, 0], [0, 130], [130, 100]], 12, 1.0, 1.0,
            f"d{d}")


@pytest.mark.parametrize("hq,hkv,mask,sk,sv", [(32, 8, [1, 0, 0, 1, 1, 0, 1, 0], 0.5, 4.0),
                                               (16, 2, [1, 0], 2.0, 0.25), (24, 3, [0, 1, 1], 1.0, 1.0)])
def test_fp8_groups_and_scales(hq, hkv, mask, sk, sv):
    """G = 4, 8, 8 with tensor scales other than 1 (inputs scaled to match)."""
    require_gpu()
    _say(f"groups Hq={hq} Hkv={hkv} scales {sk} {sv}")
    q, k, v = qkv(3, 300, hq, hkv, 128, 92, "cuda")
    k, v = (k.float() * sk).to(torch.bfloat16), (v.float() * sv).to(torch.bfloat16)
    cache = new_cache_fp8(3, hq, hkv, 128, 300, 8, 32, mask, sk, sv)
    run_fp8(cache, q, k, v, mask, [[200, 3, 77], [50, 140, 0]], 6, sk, sv, f"G{hq // hkv}")


def test_fp8_long_one_shot_prefill_then_decode():
    """A 4096-token one-shot prefill (64 key tiles per late query tile, the
    reference moving as maxima grow) and decode steps with many splits."""
    require_gpu()
    _say("one-shot 4096")
    mask = [1, 0, 0, 1]
    q, k, v = qkv(1, 4100, 4, 4, 128, 93, "cuda")
    cache = new_cache_fp8(1, 4, 4, 128, 4100, 64, 256, mask)
    run_fp8(cache, q, k, v, mask, [[4096]], 4, 1.0, 1.0, "4096")


def test_fp8_append_then_decode_paged():
    """A 9000-token prefix stored by duo_cache_append into a paged fp8 cache,
    then decode."""
    require_gpu()
    _say("append 9000 paged + decode")
    mask = [1, 0]
    n, steps = 9000, 3
    q, k, v = qkv(2, n + steps, 8, 2, 128, 94, "cuda")
    cache = new_cache_fp8(2, 8, 2, 128, n + steps, 64, 256, mask, page_tokens=1024, num_pages=16)
    lens = [n, n - 4000]
    duo.duo_cache_append(cache, k[:, :n].contiguous(), v[:, :n].contiguous(), lens)
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    done = list(lens)
    for s in range(steps):
        q1 = torch.stack([q[b, done[b]] for b in range(2)]).contiguous()
        k1 = torch.stack([k[b, done[b]] for b in range(2)]).contiguous()
        v1 = torch.stack([v[b, done[b]] for b in range(2)]).contiguous()
        o1 = torch.empty_like(q1)
        duo.duo_decode(cache, q1, k1, v1, o1)
        ref = oracle_fp8(qn, kn, vn, mask, 64, 256, [[done[b]] for b in range(2)], 1.0, 1.0)
        got = to_np32(o1)
        for b, r in ref.items():
            assert_close(got[b][None], r, f"decode step {s} b{b}")
        done = [p + 1 for p in done]
    torch.cuda.synchronize()
    check_cache_fp8(cache, kn, vn, k, v, mask, done, 1.0, 1.0)


def test_fp8_first_token_decode():
    require_gpu()
    _say("decode from empty")
    mask = [1, 1]
    q, k, v = qkv(1, 5, 4, 2, 64, 95, "cuda")
    cache = new_cache_fp8(1, 4, 2, 64, 8, 2, 4, mask)
    run_fp8(cache, q, k, v, mask, [], 5, 1.0, 1.0, "empty")


def test_fp8_paged_chunked_prefill_and_decode():
    """fp8 rows in pages (P = 512): chunked prefill across page boundaries (the
    fp8 prefill looks up the page of every 64-row tile), then decode steps
    that open new pages; codes read back through the page table."""
    require_gpu()
    _say("paged chunked")
    mask = [1, 0, 1, 1]
    t = 1700
    q, k, v = qkv(2, t, 8, 4, 128, 96, "cuda")
    cache = new_cache_fp8(2, 8, 4, 128, t, 4, 64, mask, page_tokens=512, num_pages=8)
    run_fp8(cache, q, k, v, mask, [[700, 300], [600, 1000], [380, 390]], 6, 1.0, 1.0, "paged")


def test_fp8_paged_equals_contiguous():
    """The same calls into a paged and a contiguous fp8 cache give bitwise
    equal prefill outputs and stored codes."""
    require_gpu()
    _say("paged == contiguous")
    mask = [1, 1, 0, 1]
    t = 2600
    q, k, v = qkv(2, t, 16, 4, 128, 97, "cuda")
    chunks = [[1500, 900], [1100, 1700]]
    paged = new_cache_fp8(2, 16, 4, 128, t, 64, 256, mask, page_tokens=1024, num_pages=6)
    flat = new_cache_fp8(2, 16, 4, 128, t, 64, 256, mask)
    op, _, _ = run_sequence(paged, q, k, v, chunks, 0)
    fp, _, _ = run_sequence(flat, q, k, v, chunks, 0)
    assert torch.equal(op.view(torch.int16), fp.view(torch.int16))
    a, b = duo.cache_views(paged), duo.cache_views(flat)
    for name in ("rk", "rv"):  # the paged view holds whole pages: compare the stored rows
        assert torch.equal(a[name][:, :, :t], b[name][:, :, :t]), name


def test_fp8_varlen_equals_padded():
    """Packed rows with cu_seqlens into an fp8 cache give the padded call's
    prefill outputs and cache bit for bit (including an empty sequence)."""
    require_gpu()
    _say("varlen == padded")
    mask = [0, 1, 1, 0]
    lens = [300, 0, 1029, 64]
    b_n, c = 4, max(lens)
    q, k, v = qkv(b_n, c, 8, 4, 128, 98, "cuda")
    pad = new_cache_fp8(b_n, 8, 4, 128, 2048, 8, 32, mask)
    packed = new_cache_fp8(b_n, 8, 4, 128, 2048, 8, 32, mask)
    out_pad = torch.zeros_like(q)
    duo.duo_prefill(pad, q, k, v, lens, out_pad)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    qp = torch.cat([q[b, :lens[b]] for b in range(b_n)]).contiguous()
    kp = torch.cat([k[b, :lens[b]] for b in range(b_n)]).contiguous()
    vp = torch.cat([v[b, :lens[b]] for b in range(b_n)]).contiguous()
    out_p = torch.zeros_like(qp)
    duo.duo_prefill_varlen(packed, qp, kp, vp, cu, out_p)
    torch.cuda.synchronize()
    for b in range(b_n):
        assert torch.equal(out_p[cu[b]:cu[b + 1]].view(torch.int16), out_pad[b, :lens[b]].view(torch.int16)), f"b{b}"
    a, bb = duo.cache_views(pad), duo.cache_views(packed)
    for name in ("rk", "rv"):
        assert torch.equal(a[name], bb[name]), name
    for name in ("sk", "sv"):
        assert torch.equal(a[name].view(torch.int16), bb[name].view(torch.int16)), name
    assert pad.lengths() == packed.lengths() == lens
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    ref = oracle_fp8(qn, kn, vn, mask, 8, 32, {b: list(range(lens[b])) for b in range(b_n)}, 1.0, 1.0)
    g = 2
    for b in range(b_n):
        if lens[b]:
            got = to_np32(out_p[cu[b]:cu[b + 1]])
            retr = [h for h in range(8) if mask[h // g]]
            strm = [h for h in range(8) if not mask[h // g]]
            vmax = [np.abs(seen_rows_fp8(vn[b, :lens[b], h // g], True, 1.0)).max() for h in retr]
            assert_fp8_close(got[:, retr], ref[b][:, retr], vmax, f"varlen b{b}")
            assert_close(got[:, strm], ref[b][:, strm], f"varlen streaming b{b}")
