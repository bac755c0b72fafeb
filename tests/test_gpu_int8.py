"""GPU parity of the int8 retrieval cache (DUO_KV_INT8) against the oracle.

Bit-exact: every stored retrieval row's codes and fp32 scale equal the
oracle's quantization of the input row (oracle/quantized_cache.py, reading
Q2); streaming slots hold the bf16 input rows.  Within tolerance: prefill
and decode outputs against the fp64 oracle on the K/V values each call sees
(reading Q4: rows stored by earlier calls dequantized, the call's own rows as
given).  Every cache buffer starts as 0xFF bytes: an unwritten row has a NaN
scale and would poison the output."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from oracle import attend_rows, quantize_rows, seen_rows, streaming_slot_positions
from parity_util import assert_close, require_gpu, staging_workspace, to_np32
from workloads import qkv

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-int8] {msg}", flush=True)


def new_cache_q8(batch, hq, hkv, d, max_len, sink, recent, mask, staged=False, **kw):
    """staged: with a full prefill staging workspace (prefill_staging), else none
    (every tile decodes its stored rows)."""
    cfg = duo.Config(batch, hq, hkv, d, max_len, sink, recent, [int(x) for x in mask], kv_format=duo.DUO_KV_INT8,
                     **kw)
    if staged:
        staging_workspace(cfg)
    buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
    return duo.duo_cache_init(cfg, buf)


def oracle_q8(q, k, v, mask, sink, recent, rows_by_b, stored_before):
    """fp64 oracle for the query rows rows_by_b[b] of one call whose cache held
    stored_before[b] tokens.  q [B,T,Hq,D], k/v [B,T,Hkv,D] numpy fp32."""
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
            ks = seen_rows(k[b, :tmax, kvh], bool(mask[kvh]), stored_before[b])
            vs = seen_rows(v[b, :tmax, kvh], bool(mask[kvh]), stored_before[b])
            for h in range(kvh * g, (kvh + 1) * g):
                res[:, h] = attend_rows(q[b, rows, h], rows, ks, vs, bool(mask[kvh]), sink, recent, scale)
        out[b] = res
    return out


def check_cache_q8(cache, k32, v32, k_bf, v_bf, mask, n_tokens):
    """Codes and scales of every stored retrieval row (bit-exact against the
    oracle's quantization), streaming slots (bitwise bf16), device lengths."""
    views = duo.cache_views(cache)
    cfg = cache.cfg
    hidx = cache.head_index()
    assert views["lengths"].cpu().tolist() == list(n_tokens)
    rk, rv = views["rk"].cpu().numpy(), views["rv"].cpu().numpy()
    rks, rvs = views["rks"].cpu().numpy(), views["rvs"].cpu().numpy()
    sk, sv = views["sk"].view(torch.int16).cpu(), views["sv"].view(torch.int16).cpu()
    kb, vb = k_bf.view(torch.int16).cpu(), v_bf.view(torch.int16).cpu()
    for b in range(cfg.batch):
        n = n_tokens[b]
        slots = streaming_slot_positions(n, cfg.sink, cfg.recent)
        for kvh in range(cfg.num_kv_heads):
            i = hidx[kvh]
            if mask[kvh]:
                for name, codes, scales, src in (("k", rk, rks, k32), ("v", rv, rvs, v32)):
                    c_ref, s_ref = quantize_rows(src[b, :n, kvh])
                    assert np.array_equal(codes[b, i, :n], c_ref), f"{name} codes b{b} kv{kvh}"
                    assert np.array_equal(scales[b, i, :n].view(np.uint32), s_ref.view(np.uint32)), \
                        f"{name} scales b{b} kv{kvh}"
            else:
                for s, p in enumerate(slots):
                    if p >= 0:
                        assert torch.equal(sk[b, i, s], kb[b, p, kvh]), f"sk b{b} kv{kvh} slot{s}"
                        assert torch.equal(sv[b, i, s], vb[b, p, kvh]), f"sv b{b} kv{kvh} slot{s}"


def run_q8(cache, q, k, v, chunks, decode_steps, mask):
    """Prefill in the chunk plan, then decode; every call checked against the
    oracle on the values it sees.  q/k/v bf16 cuda [B,T,H,D]."""
    cfg = cache.cfg
    q32, k32, v32 = to_np32(q), to_np32(k), to_np32(v)
    done = [0] * cfg.batch
    for n_new in chunks:
        c = max(max(n_new), 1)
        qc = torch.zeros(cfg.batch, c, cfg.num_q_heads, cfg.head_dim, dtype=torch.bfloat16, device="cuda")
        kc = torch.zeros(cfg.batch, c, cfg.num_kv_heads, cfg.head_dim, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        for b in range(cfg.batch):
            qc[b, :n_new[b]] = q[b, done[b]:done[b] + n_new[b]]
            kc[b, :n_new[b]] = k[b, done[b]:done[b] + n_new[b]]
            vc[b, :n_new[b]] = v[b, done[b]:done[b] + n_new[b]]
        oc = torch.zeros_like(qc)
        duo.duo_prefill(cache, qc, kc, vc, n_new, oc)
        got = to_np32(oc)
        ref = oracle_q8(q32, k32, v32, mask, cfg.sink, cfg.recent,
                        [list(range(done[b], done[b] + n_new[b])) for b in range(cfg.batch)], done)
        for b, r in ref.items():
            assert_close(got[b, :n_new[b]], r, f"prefill call {n_new} b{b}")
        done = [done[b] + n_new[b] for b in range(cfg.batch)]
    for s in range(decode_steps):
        q1 = torch.stack([q[b, done[b]] for b in range(cfg.batch)]).contiguous()
        k1 = torch.stack([k[b, done[b]] for b in range(cfg.batch)]).contiguous()
        v1 = torch.stack([v[b, done[b]] for b in range(cfg.batch)]).contiguous()
        o1 = torch.empty_like(q1)
        duo.duo_decode(cache, q1, k1, v1, o1)
        got = to_np32(o1)
        ref = oracle_q8(q32, k32, v32, mask, cfg.sink, cfg.recent, [[done[b]] for b in range(cfg.batch)], done)
        for b, r in ref.items():
            assert_close(got[b][None], r, f"decode step {s} b{b}")
        done = [p + 1 for p in done]
    torch.cuda.synchronize()
    check_cache_q8(cache, k32, v32, k, v, mask, done)
    return done


STAGED = pytest.mark.parametrize("staged", [False, True], ids=["tiled", "staged"])


@STAGED
@pytest.mark.parametrize("d", [64, 128])
def test_q8_chunked_prefill_and_decode(d, staged):
    require_gpu()
    _say(f"chunked prefill + decode D={d} staged={staged}")
    mask = [1, 0, 1, 0]
    q, k, v = qkv(2, 420, 8, 4, d, 41, "cuda")
    cache = new_cache_q8(2, 8, 4, d, 420, 4, 16, mask, staged)
    run_q8(cache, q, k, v, [[100, 50], [64, 1], [1, 63], [65, 0], [0, 130], [130, 100]], 12, mask)


@pytest.mark.parametrize("hq,hkv,mask", [(32, 8, [1, 0, 0, 1, 1, 0, 1, 0]), (16, 2, [1, 0]), (4, 4, [1, 1, 0, 1]),
                                          (24, 3, [0, 1, 1])])
@STAGED
def test_q8_group_sizes(hq, hkv, mask, staged):
    """G = 4, 8, 1, 8: with an int8 cache a decode work-group serves at most
    4 query heads, so G = 8 runs two head chunks per KV head."""
    require_gpu()
    _say(f"groups Hq={hq} Hkv={hkv} staged={staged}")
    q, k, v = qkv(3, 300, hq, hkv, 128, 42, "cuda")
    cache = new_cache_q8(3, hq, hkv, 128, 300, 8, 32, mask, staged)
    run_q8(cache, q, k, v, [[200, 3, 77], [50, 140, 0]], 6, mask)


def test_q8_append_then_long_decode():
    """A long stored prefix filled by duo_cache_append (quantized on store),
    then decode with many split-K work-groups and dynamic pair claims."""
    require_gpu()
    _say("append + long decode")
    mask = [1, 0]
    n, steps = 9000, 3
    q, k, v = qkv(2, n + steps, 8, 2, 128, 43, "cuda")
    cache = new_cache_q8(2, 8, 2, 128, n + steps, 64, 256, mask)
    lens = [n, n - 4000]
    duo.duo_cache_append(cache, k[:, :n].contiguous(), v[:, :n].contiguous(), lens)
    q32, k32, v32 = to_np32(q), to_np32(k), to_np32(v)
    done = list(lens)
    for s in range(steps):
        q1 = torch.stack([q[b, done[b]] for b in range(2)]).contiguous()
        k1 = torch.stack([k[b, done[b]] for b in range(2)]).contiguous()
        v1 = torch.stack([v[b, done[b]] for b in range(2)]).contiguous()
        o1 = torch.empty_like(q1)
        duo.duo_decode(cache, q1, k1, v1, o1)
        ref = oracle_q8(q32, k32, v32, mask, 64, 256, [[done[b]] for b in range(2)], done)
        got = to_np32(o1)
        for b, r in ref.items():
            assert_close(got[b][None], r, f"decode step {s} b{b}")
        done = [p + 1 for p in done]
    torch.cuda.synchronize()
    # the stored rows, sequence 1 shorter: its rows past its length untouched
    check_cache_q8(cache, k32, v32, k, v, mask, done)


def test_q8_first_token_decode():
    """Decode into an empty int8 cache: no stored row, only the new token."""
    require_gpu()
    _say("decode from empty")
    mask = [1, 1]
    q, k, v = qkv(1, 5, 4, 2, 64, 44, "cuda")
    cache = new_cache_q8(1, 4, 2, 64, 8, 2, 4, mask)
    run_q8(cache, q, k, v, [], 5, mask)


@pytest.mark.parametrize("variant", ["contiguous", "paged", "rope", "rope_paged"])
def test_q8_staged_prefill_equals_tiled(variant):
    """The staged prefill (stored rows decoded once per call into the
    workspace) and the tiled one (decoded in every tile) attend the same
    values: outputs and caches equal bit for bit, also when a workspace too
    small for the later calls makes them fall back to the tiled path.  The
    chunk plan mixes sequences with and without new rows, prefixes that end
    inside a tile, and chunks of one row."""
    require_gpu()
    _say(f"staged == tiled, {variant}")
    mask = [1, 0, 1, 1]
    b_n, hq, hkv, d, t = 3, 8, 4, 128, 1500
    kw = {}
    if "paged" in variant:
        kw.update(page_tokens=512, num_pages=b_n * 3)
    if "rope" in variant:
        kw.update(rope_base=10000.0, rope_style=duo.DUO_ROPE_HALF)
    q, k, v = qkv(b_n, t, hq, hkv, d, 45, "cuda")
    plan = [[300, 0, 130], [1, 700, 64], [500, 1, 0], [0, 300, 900], [699, 499, 1]]
    cfg0 = duo.Config(b_n, hq, hkv, d, t, 8, 64, mask, kv_format=duo.DUO_KV_INT8, **kw)
    n_r = sum(mask)
    # enough for rows up to 820 (the first three calls), not for the last two
    small = 4 * b_n * n_r * d * 820
    outs = {}
    caches = {}
    for mode, nbytes in (("tiled", None), ("staged", duo.prefill_staging_bytes(cfg0)), ("small", small)):
        cfg = duo.Config(**{**cfg0.__dict__})
        if nbytes is not None:
            staging_workspace(cfg, nbytes)
        buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
        cache = duo.duo_cache_init(cfg, buf)
        done = [0] * b_n
        res = []
        for n_new in plan:
            c = max(n_new)
            qc = torch.zeros(b_n, c, hq, d, dtype=torch.bfloat16, device="cuda")
            kc = torch.zeros(b_n, c, hkv, d, dtype=torch.bfloat16, device="cuda")
            vc = torch.zeros_like(kc)
            for b in range(b_n):
                qc[b, :n_new[b]] = q[b, done[b]:done[b] + n_new[b]]
                kc[b, :n_new[b]] = k[b, done[b]:done[b] + n_new[b]]
                vc[b, :n_new[b]] = v[b, done[b]:done[b] + n_new[b]]
            oc = torch.zeros_like(qc)
            duo.duo_prefill(cache, qc, kc, vc, n_new, oc)
            res.append(oc)
            done = [done[b] + n_new[b] for b in range(b_n)]
        torch.cuda.synchronize()
        assert all(torch.isfinite(o.float()).all() for o in res), mode
        outs[mode] = res
        caches[mode] = cache
    for mode in ("staged", "small"):
        for i, (a, b) in enumerate(zip(outs["tiled"], outs[mode])):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{mode} call {i}"
        for name in ("rk", "rv", "rks", "rvs", "sk", "sv"):
            va = duo.cache_views(caches["tiled"])[name]
            vb = duo.cache_views(caches[mode])[name]
            assert torch.equal(va.view(torch.uint8), vb.view(torch.uint8)), f"{mode} {name}"
