"""GPU parity of rotary position embedding inside the library against the oracle.

The library gets UN-rotated q and k and turns them to each token's position
(oracle/rope.py, readings R1-R4): K is stored rotated in bf16 and every key
is attended through that stored value, q is rotated before the product.
The oracle rotates in fp64 and rounds K to bf16; the GPU rotates in fp32
from fp64-reduced angles.  A stored K element may therefore differ from
the oracle's by one bf16 step where the exact value sits next to a rounding
tie, plus the fp32 rotation error, at most about 2^-22 (|a| + |b|) for the
pair (a, b): visible only where the rotated value nearly cancels.  The
cache check allows one step plus 1e-6 (|a| + |b|) for a small fraction of
elements and checks V bit for bit.  Outputs are held to the usual bar.  Every cache
buffer starts as NaN bytes."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from oracle import attend_rows, streaming_slot_positions
from oracle.rope import apply_rope, pair_dims, round_bf16
from parity_util import assert_close, require_gpu, run_sequence, staging_workspace, to_np32
from workloads import qkv

pytestmark = pytest.mark.gpu

INTERLEAVED, HALF = duo.DUO_ROPE_INTERLEAVED, duo.DUO_ROPE_HALF


def _say(msg):
    print(f"[gpu-rope] {msg}", flush=True)


def new_cache_rope(batch, hq, hkv, d, max_len, sink, recent, mask, base, style):
    cfg = duo.Config(batch, hq, hkv, d, max_len, sink, recent, [int(x) for x in mask], rope_base=base,
                     rope_style=style)
    buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
    return duo.duo_cache_init(cfg, buf)


def rotated_keys(k_seq, base, style):
    """Stored K of one (sequence, KV head): rows by position, rotated and
    rounded to bf16 (reading R4), float64 [T, D]."""
    return round_bf16(apply_rope(k_seq, np.arange(k_seq.shape[0]), base, style))


def oracle_rope(q, k, v, mask, sink, recent, rows_by_b, base, style):
    """fp64 oracle for the query positions rows_by_b[b].  q [B,T,Hq,D],
    k/v [B,T,Hkv,D] numpy fp32 (bf16 values), un-rotated."""
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
            ks = rotated_keys(k[b, :tmax, kvh], base, style)
            vs = np.asarray(v[b, :tmax, kvh], dtype=np.float64)
            for h in range(kvh * g, (kvh + 1) * g):
                qr = apply_rope(q[b, rows, h], rows, base, style)
                res[:, h] = attend_rows(qr, rows, ks, vs, bool(mask[kvh]), sink, recent, scale)
        out[b] = res
    return out


def pair_magnitude(x, style):
    """|a| + |b| of the (un-rotated) pair each element belongs to."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    ia, ib = pair_dims(x.shape[-1], style)
    m = np.empty_like(x)
    m[..., ia] = m[..., ib] = x[..., ia] + x[..., ib]
    return m


def assert_bf16_near(got, ref, pair_mag, what, max_frac=1e-3):
    """got/ref float64 arrays of bf16 values: equal, except elements within
    one bf16 step plus the fp32 rotation error bound, in at most max_frac of
    the elements."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    diff = np.abs(got - ref)
    step = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8)  # bf16 spacing at |ref|
    bound = step * 1.0000001 + 1e-6 * pair_mag
    assert (diff <= bound).all(), f"{what}: max diff {diff.max():.3e} beyond one bf16 step + rotation error"
    frac = float((diff > 0).mean())
    assert frac <= max_frac, f"{what}: {frac:.2e} of elements differ"


def check_cache_rope(cache, k_all, v_all, mask, n_tokens, base, style):
    views = duo.cache_views(cache)
    cfg = cache.cfg
    hidx = cache.head_index()
    assert views["lengths"].cpu().tolist() == list(n_tokens)
    kn = to_np32(k_all)
    vb = v_all.view(torch.int16).cpu()
    rk, rv = views["rk"].float().cpu().numpy(), views["rv"].view(torch.int16).cpu()
    sk, sv = views["sk"].float().cpu().numpy(), views["sv"].view(torch.int16).cpu()
    for b in range(cfg.batch):
        n = n_tokens[b]
        slots = streaming_slot_positions(n, cfg.sink, cfg.recent)
        for kvh in range(cfg.num_kv_heads):
            i = hidx[kvh]
            kr = rotated_keys(kn[b, :n, kvh], base, style)
            mag = pair_magnitude(kn[b, :n, kvh], style)
            if mask[kvh]:
                assert_bf16_near(rk[b, i, :n], kr, mag, f"rk b{b} kv{kvh}")
                assert torch.equal(rv[b, i, :n], vb[b, :n, kvh]), f"rv b{b} kv{kvh}"
            else:
                for s, p in enumerate(slots):
                    if p >= 0:
                        assert_bf16_near(sk[b, i, s], kr[p], mag[p], f"sk b{b} kv{kvh} slot{s}", max_frac=1.0 / 16)
                        assert torch.equal(sv[b, i, s], vb[b, p, kvh]), f"sv b{b} kv{kvh} slot{s}"


def run_and_check(cache, q, k, v, mask, chunks, steps, base, style, what):
    cfg = cache.cfg
    outp, outd, done = run_sequence(cache, q, k, v, chunks, steps)
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    b_n = q.shape[0]
    pre = [sum(c[b] for c in chunks) for b in range(b_n)]
    rows = {b: list(range(pre[b] + steps)) for b in range(b_n)}
    ref = oracle_rope(qn, kn, vn, mask, cfg.sink, cfg.recent, rows, base, style)
    for b in range(b_n):
        if pre[b]:
            assert_close(to_np32(outp[b, :pre[b]]), ref[b][:pre[b]], f"{what} prefill b{b}")
        if steps:
            assert_close(to_np32(outd[:, b]), ref[b][pre[b]:], f"{what} decode b{b}")
    check_cache_rope(cache, k, v, mask, done, base, style)


@pytest.mark.parametrize("style", [INTERLEAVED, HALF])
@pytest.mark.parametrize("d", [64, 128])
def test_rope_chunked_prefill_and_decode(d, style):
    """Chunks around the window (W=16, S=4): streaming tiles mix sink, ring
    and chunk rows; retrieval rows come from the cache, stored first."""
    require_gpu()
    _say(f"chunked d={d} style={style}")
    mask = [1, 0, 1, 0]
    q, k, v = qkv(2, 430, 8, 4, d, 51, "cuda")
    cache = new_cache_rope(2, 8, 4, d, 430, 4, 16, mask, 10000.0, style)
    run_and_check(cache, q, k, v, mask, [[100, 50], [64, 1], [1, 63], [65, 0], [0, 130], [130, 100]], 12,
                  10000.0, style, f"d{d} s{style}")


@pytest.mark.parametrize("hq,hkv,mask", [(32, 8, [1, 0, 0, 1, 1, 0, 1, 0]), (16, 2, [1, 0]), (24, 3, [0, 1, 1])])
def test_rope_group_sizes(hq, hkv, mask):
    """G = 4, 8, 8 (head chunks of 4 and 8 in decode), Llama-3-style base."""
    require_gpu()
    _say(f"groups Hq={hq} Hkv={hkv}")
    q, k, v = qkv(3, 300, hq, hkv, 128, 52, "cuda")
    cache = new_cache_rope(3, hq, hkv, 128, 300, 8, 32, mask, 500000.0, HALF)
    run_and_check(cache, q, k, v, mask, [[200, 3, 77], [50, 140, 0]], 6, 500000.0, HALF, f"G{hq // hkv}")


def test_rope_one_shot_long_prefill():
    """One 1000-token call: every streaming band tile is staged and turned."""
    require_gpu()
    _say("one-shot 1000")
    mask = [0, 1]
    q, k, v = qkv(1, 1004, 4, 2, 128, 53, "cuda")
    cache = new_cache_rope(1, 4, 2, 128, 1004, 64, 256, mask, 10000.0, INTERLEAVED)
    run_and_check(cache, q, k, v, mask, [[1000]], 4, 10000.0, INTERLEAVED, "one-shot")


def test_rope_append_then_long_decode():
    """A 9000-token prefix stored (rotated) by duo_cache_append, then decode
    with many splits."""
    require_gpu()
    _say("append 9000 + decode")
    mask = [1, 0]
    n, steps = 9000, 3
    q, k, v = qkv(2, n + steps, 8, 2, 128, 54, "cuda")
    cache = new_cache_rope(2, 8, 2, 128, n + steps, 64, 256, mask, 10000.0, HALF)
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
        ref = oracle_rope(qn, kn, vn, mask, 64, 256, [[done[b]] for b in range(2)], 10000.0, HALF)
        got = to_np32(o1)
        for b, r in ref.items():
            assert_close(got[b][None], r, f"decode step {s} b{b}")
        done = [p + 1 for p in done]
    torch.cuda.synchronize()
    check_cache_rope(cache, k, v, mask, done, 10000.0, HALF)


def test_rope_first_token_decode():
    """Decode into an empty cache: only the new (rotated) token."""
    require_gpu()
    _say("decode from empty")
    mask = [1, 0]
    q, k, v = qkv(1, 6, 4, 2, 64, 55, "cuda")
    cache = new_cache_rope(1, 4, 2, 64, 8, 2, 4, mask, 10000.0, INTERLEAVED)
    run_and_check(cache, q, k, v, mask, [], 6, 10000.0, INTERLEAVED, "empty")


def test_rope_million_positions():
    """Positions past 2^20: an fp32 angle p * theta would be off by whole
    radians there.  2^20 tokens appended in 4 calls, then a 96-token prefill
    (retrieval keys from the cache, streaming chunk rows turned on load) and
    2 decode steps; sampled prefill rows and every decode step checked."""
    require_gpu()
    _say("million positions")
    mask = [1, 0]
    n0, c, steps, d = 1 << 20, 96, 2, 64
    t = n0 + c + steps
    q, k, v = qkv(1, t, 2, 2, d, 56, "cuda")
    cache = new_cache_rope(1, 2, 2, d, t, 4, 64, mask, 10000.0, HALF)
    part = n0 // 4
    for i in range(4):
        duo.duo_cache_append(cache, k[:, i * part:(i + 1) * part].contiguous(),
                             v[:, i * part:(i + 1) * part].contiguous(), [part])
    outp, outd, done = run_sequence_from(cache, q, k, v, n0, [[c]], steps)
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    rows = [n0, n0 + 1, n0 + 47, n0 + 63, n0 + 64, n0 + 95]
    ref = oracle_rope(qn, kn, vn, mask, 4, 64, [rows + [n0 + c + s for s in range(steps)]], 10000.0, HALF)[0]
    got = np.concatenate([to_np32(outp[0, [r - n0 for r in rows]]), to_np32(outd[:, 0])])
    assert_close(got, ref, "million")


def run_sequence_from(cache, q, k, v, start, chunks, steps):
    """run_sequence for a cache that already holds `start` tokens of every
    sequence (q/k/v index positions from 0)."""
    sl = slice(start, None)
    return run_sequence(cache, q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(), chunks, steps)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "bf16_staged"])
@pytest.mark.parametrize("style", [INTERLEAVED, HALF])
@pytest.mark.parametrize("d", [64, 128])
def test_rope_chunked_equals_one_shot_bitwise(d, style, fmt):
    """Chunk boundaries on multiples of 64 positions, so every query row meets
    the same keys in the same tiles and waves as in one call over the whole
    sequence.  Outputs and caches then equal bit for bit -- which holds only
    if a key gets the same turned value where a tile load turns it (the
    call's own rows of streaming heads) and where it is stored and read back
    (rows of earlier chunks: the streaming ring, every retrieval row)."""
    require_gpu()
    _say(f"chunked == one-shot, d={d} style={style} {fmt}")
    mask = [1, 0, 1, 0]
    b_n, hq, hkv, t = 2, 8, 4, 1024
    q, k, v = qkv(b_n, t, hq, hkv, d, 71, "cuda")
    kw = dict(kv_format=duo.DUO_KV_FP8) if fmt == "fp8" else {}
    plans = {"one": [[t, t]], "chunked": [[256, 128], [128, 448], [640, 448]]}
    outs, views = {}, {}
    for name, plan in plans.items():
        cfg = duo.Config(b_n, hq, hkv, d, t, 8, 64, mask, rope_base=10000.0, rope_style=style, **kw)
        if fmt == "bf16_staged":
            staging_workspace(cfg)
        buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
        cache = duo.duo_cache_init(cfg, buf)
        out = torch.zeros(b_n, t, hq, d, dtype=torch.bfloat16, device="cuda")
        done = [0] * b_n
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
            for b in range(b_n):
                out[b, done[b]:done[b] + n_new[b]] = oc[b, :n_new[b]]
            done = [done[b] + n_new[b] for b in range(b_n)]
        torch.cuda.synchronize()
        outs[name] = out
        views[name] = {n: x.clone() for n, x in duo.cache_views(cache).items()}
    assert torch.equal(outs["one"].view(torch.int16), outs["chunked"].view(torch.int16))
    for n in ("rk", "rv", "sk", "sv"):
        a, b = views["one"][n], views["chunked"][n]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), n


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_rope_staged_prefill_equals_tiled(paged, fmt):
    """With the prefill staging workspace a call turns its streaming heads'
    chunk K rows once (and an 8-bit cache's retrieval rows are staged as
    bf16); without it every tile turns them.  Both turn a key the one way, so
    outputs and caches are equal bit for bit -- also when the workspace is
    too small for some calls or parts (which then fall back: for fp8 the
    first call stages its rows but not the turned chunk, the later ones at
    most the turned chunk).  Chunks mix sequences with and without new rows and
    windows that straddle the chunk boundary."""
    require_gpu()
    _say(f"rope staged == tiled, {fmt} paged={paged}")
    mask = [1, 0, 0, 1]
    b_n, hq, hkv, d, t = 3, 8, 4, 128, 1500
    kw = dict(rope_base=10000.0, rope_style=HALF)
    if paged:
        kw.update(page_tokens=512, num_pages=b_n * 3)
    if fmt == "fp8":
        kw.update(kv_format=duo.DUO_KV_FP8)
    elif fmt == "int8":
        kw.update(kv_format=duo.DUO_KV_INT8)
    q, k, v = qkv(b_n, t, hq, hkv, d, 72, "cuda")
    plan = [[300, 0, 130], [1, 700, 64], [500, 1, 0], [0, 300, 900], [699, 499, 1]]
    cfg0 = duo.Config(b_n, hq, hkv, d, t, 8, 64, mask, **kw)
    outs, views = {}, {}
    # "small": room for the turned rows of the first three calls' chunks only
    small = 2 * b_n * (hkv - sum(mask)) * d * 700 + (4 * b_n * sum(mask) * d * 820 if fmt == "int8" else 0)
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
        views[mode] = {n: x.clone() for n, x in duo.cache_views(cache).items()}
    for mode in ("staged", "small"):
        for i, (a, b) in enumerate(zip(outs["tiled"], outs[mode])):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{mode} call {i}"
        for name in views["tiled"]:
            assert torch.equal(views["tiled"][name].view(torch.uint8), views[mode][name].view(torch.uint8)), \
                f"{mode} {name}"


@pytest.mark.parametrize("staged", [False, True], ids=["tiled", "staged"])
@pytest.mark.parametrize("d", [64, 128])
def test_rope_all_retrieval_and_staged_chunks(d, staged):
    """Every KV head a retrieval head (the kernels then read every turned key
    from the cache, with or without a workspace), and with streaming heads
    the staged path (the chunk's turned K rows read from the call's copy)
    checked against the oracle on chunked prefill and decode."""
    require_gpu()
    _say(f"all retrieval + staged d={d} staged={staged}")
    for mask in ([1, 1, 1, 1], [1, 0, 0, 1]):
        q, k, v = qkv(2, 420, 8, 4, d, 73, "cuda")
        cfg = duo.Config(2, 8, 4, d, 420, 4, 16, mask, rope_base=10000.0, rope_style=INTERLEAVED)
        if staged:
            staging_workspace(cfg)
        buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
        cache = duo.duo_cache_init(cfg, buf)
        run_and_check(cache, q, k, v, mask, [[100, 50], [64, 1], [1, 63], [0, 130], [130, 100]], 6, 10000.0,
                      INTERLEAVED, f"mask {mask} staged={staged}")
