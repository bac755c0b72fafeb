"""GPU parity of rotary position embedding together with the 8-bit retrieval
caches (DUO_KV_INT8, DUO_KV_FP8) against the oracle.

The library turns K to its position, rounds it to bf16 and encodes that
row; q is turned before the product.  The oracle composes its two pinned
parts: the rotation of oracle/rope.py (readings R1-R4: fp64 angles, K
rounded to bf16) and, on the rotated rows, the int8 view of a call
(oracle/quantized_cache.py, Q1-Q4: rows stored by earlier calls through
their codes, the call's own rows as given) or the fp8 view (oracle/
fp8_cache.py, E1-E4: every retrieval row through its codes).

The GPU rotates in fp32 from fp64-reduced angles, so a rotated K element
can sit one bf16 step from the oracle's next to a rounding tie; its code
then moves by at most one step (int8: one code, the row scale by at most
one bf16 step of the row's largest magnitude; e4m3: one e4m3 step).  The
cache check allows that for a small fraction of the K codes, holds V codes
and scales bit for bit, and streaming K slots to the rope tests' bound.
Outputs keep each format's bar: the usual one for int8, for fp8 decode
and streaming heads, and for the exact fp8 prefill (the default); the
rounding model of tests/fp8_model.py for the fp8-matrix-core prefill of
retrieval heads (DUO_FP8_PREFILL_MFMA).  Every cache
buffer starts as 0xFF bytes (NaN scales and bf16 rows)."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from oracle import attend_rows, quantize_rows, seen_rows, streaming_slot_positions
from oracle.fp8_cache import e4m3_decode, quantize_rows_fp8, seen_rows_fp8
from oracle.rope import apply_rope
from parity_util import assert_close, require_gpu, run_sequence, staging_workspace, to_np32
from fp8_model import assert_fp8_mfma_close, mfma_sigma
from test_gpu_rope import assert_bf16_near, pair_magnitude, rotated_keys
from workloads import qkv

pytestmark = pytest.mark.gpu

INTERLEAVED, HALF = duo.DUO_ROPE_INTERLEAVED, duo.DUO_ROPE_HALF
BASE = 10000.0


def _say(msg):
    print(f"[gpu-rope-8bit] {msg}", flush=True)


def new_cache(fmt, batch, hq, hkv, d, max_len, sink, recent, mask, style, base=BASE, staged=False, **kw):
    """staged (DUO_KV_INT8): with a full prefill staging workspace."""
    cfg = duo.Config(batch, hq, hkv, d, max_len, sink, recent, [int(x) for x in mask], kv_format=fmt,
                     rope_base=base, rope_style=style, **kw)
    if staged:
        staging_workspace(cfg)
    buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
    return duo.duo_cache_init(cfg, buf)


def oracle(fmt, q, k, v, mask, sink, recent, rows_by_b, stored_before, base, style, sk=1.0, sv=1.0):
    """fp64 outputs of the query positions rows_by_b[b] of one call whose cache
    held stored_before[b] tokens (int8; fp8 attends every retrieval row
    through its codes).  q [B,T,Hq,D], k/v [B,T,Hkv,D] fp32 numpy, un-rotated."""
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
            retr = bool(mask[kvh])
            kr = rotated_keys(k[b, :tmax, kvh], base, style)
            if fmt == duo.DUO_KV_INT8:
                ks = seen_rows(kr, retr, stored_before[b])
                vs = seen_rows(v[b, :tmax, kvh], retr, stored_before[b])
            else:
                ks = seen_rows_fp8(kr, retr, sk)
                vs = seen_rows_fp8(v[b, :tmax, kvh], retr, sv)
            for h in range(kvh * g, (kvh + 1) * g):
                qr = apply_rope(q[b, rows, h], rows, base, style)
                res[:, h] = attend_rows(qr, rows, ks, vs, retr, sink, recent, scale)
        out[b] = res
    return out


def _codes_near(got, ref, what, max_frac=1e-2):
    diff = np.abs(got.astype(np.int64) - ref.astype(np.int64))
    assert diff.max() <= 1, f"{what}: a code {diff.max()} steps away"
    frac = float((diff > 0).mean())
    assert frac <= max_frac, f"{what}: {frac:.2e} of the codes differ"


def check_cache(cache, fmt, k, v, mask, n_tokens, base, style, sk=1.0, sv=1.0):
    views = duo.cache_views(cache)
    cfg = cache.cfg
    hidx = cache.head_index()
    assert views["lengths"].cpu().tolist() == list(n_tokens)
    kn, vn = to_np32(k), to_np32(v)
    rk, rv = views["rk"].cpu().numpy(), views["rv"].cpu().numpy()
    sk_, sv_ = views["sk"].float().cpu().numpy(), views["sv"].view(torch.int16).cpu()
    vb = v.view(torch.int16).cpu()
    for b in range(cfg.batch):
        n = n_tokens[b]
        slots = streaming_slot_positions(n, cfg.sink, cfg.recent)
        for kvh in range(cfg.num_kv_heads):
            i = hidx[kvh]
            kr = rotated_keys(kn[b, :n, kvh], base, style)
            if mask[kvh]:
                if fmt == duo.DUO_KV_INT8:
                    rks, rvs = views["rks"].cpu().numpy(), views["rvs"].cpu().numpy()
                    c_ref, s_ref = quantize_rows(kr)
                    _codes_near(rk[b, i, :n], c_ref, f"k codes b{b} kv{kvh}")
                    rel = np.abs(rks[b, i, :n].astype(np.float64) / s_ref - 1.0)
                    assert rel.max() <= 2.0 ** -7, f"k scales b{b} kv{kvh}: {rel.max():.3e}"
                    cv_ref, sv_ref = quantize_rows(vn[b, :n, kvh])
                    assert np.array_equal(rv[b, i, :n], cv_ref), f"v codes b{b} kv{kvh}"
                    assert np.array_equal(rvs[b, i, :n].view(np.uint32), sv_ref.view(np.uint32)), \
                        f"v scales b{b} kv{kvh}"
                else:
                    got = e4m3_decode(rk[b, i, :n])
                    ref = e4m3_decode(quantize_rows_fp8(kr, sk))
                    step = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 2.0 ** -6))[1] - 4)  # e4m3 spacing
                    d = np.abs(got - ref)
                    assert (d <= step * 1.0000001).all(), f"k codes b{b} kv{kvh}: beyond one e4m3 step"
                    assert float((d > 0).mean()) <= 1e-2, f"k codes b{b} kv{kvh}: too many differ"
                    assert np.array_equal(rv[b, i, :n], quantize_rows_fp8(vn[b, :n, kvh], sv)), \
                        f"v codes b{b} kv{kvh}"
            else:
                mag = pair_magnitude(kn[b, :n, kvh], style)
                for s, p in enumerate(slots):
                    if p >= 0:
                        assert_bf16_near(sk_[b, i, s], kr[p], mag[p], f"sk b{b} kv{kvh} slot{s}", max_frac=1.0 / 16)
                        assert torch.equal(sv_[b, i, s], vb[b, p, kvh]), f"sv b{b} kv{kvh} slot{s}"


def _chunk_inputs(cfg, q, k, v, done, n_new):
    c = max(max(n_new), 1)
    qc = torch.zeros(cfg.batch, c, cfg.num_q_heads, cfg.head_dim, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(cfg.batch, c, cfg.num_kv_heads, cfg.head_dim, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for b in range(cfg.batch):
        qc[b, :n_new[b]] = q[b, done[b]:done[b] + n_new[b]]
        kc[b, :n_new[b]] = k[b, done[b]:done[b] + n_new[b]]
        vc[b, :n_new[b]] = v[b, done[b]:done[b] + n_new[b]]
    return qc, kc, vc


def run_int8(cache, q, k, v, mask, chunks, steps, style, base=BASE):
    """Every call checked against the oracle on the values it sees."""
    cfg = cache.cfg
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    done = [0] * cfg.batch
    for n_new in chunks:
        qc, kc, vc = _chunk_inputs(cfg, q, k, v, done, n_new)
        oc = torch.zeros_like(qc)
        duo.duo_prefill(cache, qc, kc, vc, n_new, oc)
        got = to_np32(oc)
        ref = oracle(duo.DUO_KV_INT8, qn, kn, vn, mask, cfg.sink, cfg.recent,
                     [list(range(done[b], done[b] + n_new[b])) for b in range(cfg.batch)], done, base, style)
        for b, r in ref.items():
            assert_close(got[b, :n_new[b]], r, f"int8 rope prefill call {n_new} b{b}")
        done = [done[b] + n_new[b] for b in range(cfg.batch)]
    for s in range(steps):
        q1 = torch.stack([q[b, done[b]] for b in range(cfg.batch)]).contiguous()
        k1 = torch.stack([k[b, done[b]] for b in range(cfg.batch)]).contiguous()
        v1 = torch.stack([v[b, done[b]] for b in range(cfg.batch)]).contiguous()
        o1 = torch.empty_like(q1)
        duo.duo_decode(cache, q1, k1, v1, o1)
        ref = oracle(duo.DUO_KV_INT8, qn, kn, vn, mask, cfg.sink, cfg.recent, [[done[b]] for b in range(cfg.batch)],
                     done, base, style)
        got = to_np32(o1)
        for b, r in ref.items():
            assert_close(got[b][None], r, f"int8 rope decode step {s} b{b}")
        done = [p + 1 for p in done]
    torch.cuda.synchronize()
    check_cache(cache, duo.DUO_KV_INT8, k, v, mask, done, base, style)


def check_fp8_retrieval(cfg, got, ref, qn_b, kn_b, vn_b, rows, mask, base, style, what):
    """Retrieval heads' prefill of one sequence (got / ref [len(rows), Hq, D]):
    the usual bar for the exact mode; for the fp8-matrix-core mode the
    rounding model, fed the turned q rows and the stored turned K rows."""
    g = cfg.num_q_heads // cfg.num_kv_heads
    retr = [h for h in range(cfg.num_q_heads) if mask[h // g]]
    sk, sv = cfg.kv_scale_k or 1.0, cfg.kv_scale_v or 1.0
    if cfg.fp8_prefill == duo.DUO_FP8_PREFILL_EXACT:
        assert_close(got[:, retr] / sv, ref[:, retr] / sv, f"{what} (exact)")
        return
    sig = np.empty((len(rows), len(retr), cfg.head_dim))
    scale = 1.0 / math.sqrt(cfg.head_dim)
    for i, h in enumerate(retr):
        kvh = h // g
        ks = seen_rows_fp8(rotated_keys(kn_b[:, kvh], base, style), True, sk)
        vs = seen_rows_fp8(vn_b[:, kvh], True, sv)
        qr = apply_rope(qn_b[rows, h], rows, base, style)
        sig[:, i] = mfma_sigma(qr, rows, ks, vs, True, cfg.sink, cfg.recent, scale)
    w = assert_fp8_mfma_close(got[:, retr], ref[:, retr], sig, f"{what} (fp8 mfma)")
    _say(f"{what}: |d|_2/predicted = {w[0]:.3f}, max |d|/sigma = {w[1]:.2f}")


def run_fp8(cache, q, k, v, mask, chunks, steps, style, base=BASE, sk=1.0, sv=1.0):
    cfg = cache.cfg
    outp, outd, done = run_sequence(cache, q, k, v, chunks, steps)
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    b_n = q.shape[0]
    pre = [sum(c[b] for c in chunks) for b in range(b_n)]
    ref = oracle(duo.DUO_KV_FP8, qn, kn, vn, mask, cfg.sink, cfg.recent,
                 {b: list(range(pre[b] + steps)) for b in range(b_n)}, None, base, style, sk, sv)
    g = cfg.num_q_heads // cfg.num_kv_heads
    retr = [h for h in range(cfg.num_q_heads) if mask[h // g]]
    strm = [h for h in range(cfg.num_q_heads) if not mask[h // g]]
    for b in range(b_n):
        if pre[b]:
            got = to_np32(outp[b, :pre[b]])
            r = ref[b][:pre[b]]
            if retr:
                check_fp8_retrieval(cfg, got, r, qn[b], kn[b], vn[b], list(range(pre[b])), mask, base, style,
                                    f"fp8 rope prefill b{b}")
            if strm:
                assert_close(got[:, strm] / sv, r[:, strm] / sv, f"fp8 rope prefill streaming b{b}")
        if steps:
            assert_close(to_np32(outd[:, b]) / sv, ref[b][pre[b]:] / sv, f"fp8 rope decode b{b}")
    check_cache(cache, duo.DUO_KV_FP8, k, v, mask, done, base, style, sk, sv)


CHUNKS = [[100, 50], [64, 1], [1, 63], [65, 0], [0, 130], [130, 100]]


@pytest.mark.parametrize("staged", [False, True], ids=["tiled", "staged"])
@pytest.mark.parametrize("style", [INTERLEAVED, HALF])
@pytest.mark.parametrize("d", [64, 128])
def test_int8_rope_chunked_prefill_and_decode(d, style, staged):
    """Chunks around the window (W=16, S=4): retrieval tiles mix stored int8
    rows with the call's own rows, turned as they are loaded (tiled) or once
    per call into the staging workspace (staged)."""
    require_gpu()
    _say(f"int8 chunked d={d} style={style} staged={staged}")
    mask = [1, 0, 1, 0]
    q, k, v = qkv(2, 430, 8, 4, d, 61, "cuda")
    cache = new_cache(duo.DUO_KV_INT8, 2, 8, 4, d, 430, 4, 16, mask, style, staged=staged)
    run_int8(cache, q, k, v, mask, CHUNKS, 12, style)


@pytest.mark.parametrize("mode", [duo.DUO_FP8_PREFILL_EXACT, duo.DUO_FP8_PREFILL_MFMA], ids=["exact", "mfma"])
@pytest.mark.parametrize("style", [INTERLEAVED, HALF])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_rope_chunked_prefill_and_decode(d, style, mode):
    """The same chunks on an fp8 cache: every retrieval row attended through
    its stored (turned) value; with the fp8 matrix cores q is turned before
    its e4m3 rounding."""
    require_gpu()
    _say(f"fp8 chunked d={d} style={style} mode={mode}")
    mask = [1, 0, 1, 0]
    q, k, v = qkv(2, 430, 8, 4, d, 62, "cuda")
    cache = new_cache(duo.DUO_KV_FP8, 2, 8, 4, d, 430, 4, 16, mask, style, fp8_prefill=mode)
    run_fp8(cache, q, k, v, mask, CHUNKS, 12, style)


@pytest.mark.parametrize("fmt", [duo.DUO_KV_INT8, duo.DUO_KV_FP8])
def test_rope_8bit_group_sizes(fmt):
    """G = 4 and 8 (two head chunks per KV head in 8-bit decode), a Llama-3
    base, one-shot and chunked calls."""
    require_gpu()
    _say(f"groups fmt={fmt}")
    for hq, hkv, mask in [(32, 8, [1, 0, 0, 1, 1, 0, 1, 0]), (16, 2, [1, 0])]:
        q, k, v = qkv(3, 300, hq, hkv, 128, 63, "cuda")
        cache = new_cache(fmt, 3, hq, hkv, 128, 300, 8, 32, mask, HALF, base=500000.0)
        run = run_int8 if fmt == duo.DUO_KV_INT8 else run_fp8
        run(cache, q, k, v, mask, [[200, 3, 77], [50, 140, 0]], 6, HALF, base=500000.0)


@pytest.mark.parametrize("fmt,staged", [(duo.DUO_KV_INT8, False), (duo.DUO_KV_INT8, True), (duo.DUO_KV_FP8, False)],
                         ids=["int8", "int8_staged", "fp8"])
def test_rope_8bit_long_one_shot_then_decode(fmt, staged):
    """A 2100-token one-shot prefill (many tiles, a ragged last one), then
    decode over the stored prefix with several split-K work-groups."""
    require_gpu()
    _say(f"one-shot 2100 fmt={fmt}")
    mask = [1, 0]
    q, k, v = qkv(1, 2104, 4, 2, 128, 64, "cuda")
    cache = new_cache(fmt, 1, 4, 2, 128, 2104, 64, 256, mask, INTERLEAVED, staged=staged)
    run = run_int8 if fmt == duo.DUO_KV_INT8 else run_fp8
    run(cache, q, k, v, mask, [[2100]], 4, INTERLEAVED)


@pytest.mark.parametrize("fmt,staged", [(duo.DUO_KV_INT8, False), (duo.DUO_KV_INT8, True), (duo.DUO_KV_FP8, False)],
                         ids=["int8", "int8_staged", "fp8"])
def test_rope_8bit_paged(fmt, staged):
    """A paged cache (512-position pages): chunked prefill across page
    boundaries, then decode."""
    require_gpu()
    _say(f"paged fmt={fmt}")
    mask = [1, 1, 0, 1]
    q, k, v = qkv(2, 1300, 8, 4, 64, 65, "cuda")
    cache = new_cache(fmt, 2, 8, 4, 64, 1300, 8, 64, mask, HALF, page_tokens=512, num_pages=6, staged=staged)
    run = run_int8 if fmt == duo.DUO_KV_INT8 else run_fp8
    run(cache, q, k, v, mask, [[600, 100], [500, 700], [190, 490]], 5, HALF)


@pytest.mark.parametrize("fmt", [duo.DUO_KV_INT8, duo.DUO_KV_FP8])
def test_rope_8bit_first_token_decode(fmt):
    """Decode into an empty cache: only the new (rotated) token."""
    require_gpu()
    _say(f"decode from empty fmt={fmt}")
    mask = [1, 0]
    q, k, v = qkv(1, 6, 4, 2, 64, 66, "cuda")
    cache = new_cache(fmt, 1, 4, 2, 64, 8, 2, 4, mask, INTERLEAVED)
    run = run_int8 if fmt == duo.DUO_KV_INT8 else run_fp8
    run(cache, q, k, v, mask, [], 6, INTERLEAVED)


@pytest.mark.parametrize("fmt,staged", [(duo.DUO_KV_INT8, False), (duo.DUO_KV_INT8, True), (duo.DUO_KV_FP8, False)],
                         ids=["int8", "int8_staged", "fp8"])
def test_rope_8bit_paged_varlen_equals_padded(fmt, staged):
    """Rotary embedding, an 8-bit paged cache and a stored prefix together:
    a packed (cu_seqlens) prefill gives the padded call's outputs and cache
    bytes bit for bit, and both match the oracle (int8 also through the
    staging workspace, where the packed rows are staged from their packed
    offsets)."""
    require_gpu()
    _say(f"paged varlen == padded fmt={fmt} staged={staged}")
    mask = [1, 0, 1, 1]
    b_n = 3
    pre, lens = [700, 0, 90], [300, 520, 0]
    t = max(p + n for p, n in zip(pre, lens))
    q, k, v = qkv(b_n, t, 8, 4, 64, 67, "cuda")

    def fresh():
        return new_cache(fmt, b_n, 8, 4, 64, t, 8, 32, mask, HALF, page_tokens=512, num_pages=b_n * 2,
                         staged=staged)

    pad, packed = fresh(), fresh()
    for cache in (pad, packed):
        duo.duo_cache_append(cache, k[:, :max(pre)].contiguous(), v[:, :max(pre)].contiguous(), pre)
    c = max(lens)
    qc, kc, vc = (torch.zeros(b_n, c, x.shape[2], 64, dtype=torch.bfloat16, device="cuda") for x in (q, k, v))
    for b in range(b_n):
        qc[b, :lens[b]], kc[b, :lens[b]], vc[b, :lens[b]] = (x[b, pre[b]:pre[b] + lens[b]] for x in (q, k, v))
    out_pad = torch.zeros_like(qc)
    duo.duo_prefill(pad, qc, kc, vc, lens, out_pad)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    qp, kp, vp = (torch.cat([x[b, :lens[b]] for b in range(b_n)]).contiguous() for x in (qc, kc, vc))
    out_p = torch.zeros_like(qp)
    duo.duo_prefill_varlen(packed, qp, kp, vp, cu, out_p)
    torch.cuda.synchronize()
    for b in range(b_n):
        assert torch.equal(out_p[cu[b]:cu[b + 1]].view(torch.int16), out_pad[b, :lens[b]].view(torch.int16)), f"b{b}"
    va, vb_ = duo.cache_views(pad), duo.cache_views(packed)
    names = ("rk", "rv", "sk", "sv") + (("rks", "rvs") if fmt == duo.DUO_KV_INT8 else ())
    for name in names:
        assert torch.equal(va[name].view(torch.uint8), vb_[name].view(torch.uint8)), name
    done = [pre[b] + lens[b] for b in range(b_n)]
    assert pad.lengths() == packed.lengths() == done
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    rows = {b: list(range(pre[b], done[b])) for b in range(b_n)}
    ref = oracle(fmt, qn, kn, vn, mask, 8, 32, rows, pre, BASE, HALF)
    g = 2
    for b in range(b_n):
        if not lens[b]:
            continue
        got = to_np32(out_p[cu[b]:cu[b + 1]])
        if fmt == duo.DUO_KV_INT8:
            assert_close(got, ref[b], f"int8 varlen b{b}")
        else:
            strm = [h for h in range(8) if not mask[h // g]]
            check_fp8_retrieval(packed.cfg, got, ref[b], qn[b], kn[b], vn[b], rows[b], mask, BASE, HALF,
                                f"fp8 varlen b{b}")
            assert_close(got[:, strm], ref[b][:, strm], f"fp8 varlen streaming b{b}")
    check_cache(packed, fmt, k, v, mask, done, BASE, HALF)
