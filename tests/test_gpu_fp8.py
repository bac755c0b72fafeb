"""GPU parity of the fp8 (e4m3) retrieval cache and its two prefill modes.

Bit-exact: every stored retrieval row's codes equal the oracle's encoding
(oracle/fp8_cache.py, readings E2-E3); streaming slots hold the bf16 input.
Decode attends through the stored values in fp32 (q enters as an exact f16
multiple), so it is held to the usual bar against the oracle on those
values (reading E4).

Prefill of retrieval heads:
  * DUO_FP8_PREFILL_EXACT (the default) decodes the stored values exactly to
    bf16 and runs the bf16 tile engine: the usual bar against the oracle,
    and bit for bit the bf16 kernel's output over a bf16 cache that holds the
    stored values;
  * DUO_FP8_PREFILL_MFMA rounds q and the softmax weights to e4m3 on the
    fp8 matrix cores: held to the bar of the rounding model in
    tests/fp8_model.py (L2 error within twice the predicted RMS, every
    element within 6 predicted standard deviations).
Streaming heads keep the bf16 path and the usual bar.  Inputs scaled with
the tensor scales are compared in units of the V scale (the output is
linear in V).  Every cache buffer starts as NaN bytes."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from fp8_model import assert_fp8_mfma_close, mfma_sigma
from oracle import attend_rows, streaming_slot_positions
from oracle.fp8_cache import quantize_rows_fp8, seen_rows_fp8
from parity_util import assert_close, require_gpu, run_sequence, staging_workspace, to_np32
from workloads import qkv

pytestmark = pytest.mark.gpu

EXACT, MFMA = duo.DUO_FP8_PREFILL_EXACT, duo.DUO_FP8_PREFILL_MFMA
MODES = [EXACT, MFMA]
MODE_IDS = ["exact", "mfma"]


def _say(msg):
    print(f"[gpu-fp8] {msg}", flush=True)


def new_cache_fp8(batch, hq, hkv, d, max_len, sink, recent, mask, sk=1.0, sv=1.0, mode=EXACT, **kw):
    cfg = duo.Config(batch, hq, hkv, d, max_len, sink, recent, [int(x) for x in mask], kv_format=duo.DUO_KV_FP8,
                     kv_scale_k=sk, kv_scale_v=sv, fp8_prefill=mode, **kw)
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


def sample_rows(n, cap=384):
    """Rows of a prefill compared under the fp8-MFMA model: all of them up
    to `cap`, else the first and last 64 and an even spread between."""
    if n <= cap:
        return list(range(n))
    mid = np.linspace(64, n - 65, cap - 128).astype(np.int64).tolist()
    return sorted(set(list(range(64)) + mid + list(range(n - 64, n))))


def mfma_sigmas(qn_rows, rows, kn, vn, mask, heads, g, sink, recent, sk, sv, scale):
    """Model sigma [len(rows), len(heads), D] of one sequence's rows.
    qn_rows [len(rows), Hq, D] as the kernel rounds them; kn, vn [T, Hkv, D]
    un-encoded (the stored values are taken here)."""
    out = np.empty((len(rows), len(heads), qn_rows.shape[-1]))
    seen = {}
    for i, h in enumerate(heads):
        kvh = h // g
        if kvh not in seen:
            seen[kvh] = (seen_rows_fp8(kn[:, kvh], True, sk), seen_rows_fp8(vn[:, kvh], True, sv))
        out[:, i] = mfma_sigma(qn_rows[:, h], rows, seen[kvh][0], seen[kvh][1], bool(mask[kvh]), sink, recent,
                               scale)
    return out


def check_retrieval_prefill(cache, got, ref, qn_b, kn_b, vn_b, rows, mask, what):
    """got / ref [len(rows), Hq, D] of one sequence; the bar of the cache's
    prefill mode for its retrieval heads (module docstring)."""
    cfg = cache.cfg
    g = cfg.num_q_heads // cfg.num_kv_heads
    retr = [h for h in range(cfg.num_q_heads) if mask[h // g]]
    if not retr:
        return None
    sv = cfg.kv_scale_v or 1.0
    if cfg.fp8_prefill == EXACT:
        assert_close(got[:, retr] / sv, ref[:, retr] / sv, f"{what} (exact)")
        return None
    sel = sample_rows(len(rows))
    rr = [rows[i] for i in sel]
    sig = mfma_sigmas(qn_b[rr], rr, kn_b, vn_b, mask, retr, g, cfg.sink, cfg.recent, cfg.kv_scale_k or 1.0, sv,
                      1.0 / math.sqrt(cfg.head_dim))
    return assert_fp8_mfma_close(got[sel][:, retr], ref[sel][:, retr], sig, f"{what} (fp8 mfma)")


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
            strm = [h for h in range(cfg.num_q_heads) if not mask[h // g]]
            w = check_retrieval_prefill(cache, got, r, qn[b], kn[b], vn[b], list(range(pre[b])), mask,
                                        f"{what} prefill b{b}")
            if w is not None:
                worst = (max(worst[0], w[0]), max(worst[1], w[1]))
            if strm:  # the output is linear in V: compare in units of the V scale
                assert_close(got[:, strm] / sv, r[:, strm] / sv, f"{what} prefill streaming b{b}")
        if steps:
            assert_close(to_np32(outd[:, b]) / sv, ref[b][pre[b]:] / sv, f"{what} decode b{b}")
    if cfg.fp8_prefill == MFMA:
        _say(f"{what}: fp8-mfma prefill worst |d|_2/predicted = {worst[0]:.3f}, max |d|/sigma = {worst[1]:.2f}")
    check_cache_fp8(cache, kn, vn, k, v, mask, done, sk, sv)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_chunked_prefill_and_decode(d, mode):
    require_gpu()
    _say(f"chunked d={d} mode={mode}")
    mask = [1, 0, 1, 0]
    q, k, v = qkv(2, 430, 8, 4, d, 91, "cuda")
    cache = new_cache_fp8(2, 8, 4, d, 430, 4, 16, mask, mode=mode)
    run_fp8(cache, q, k, v, mask, [[100, 50], [64, 1], [1, 63], [65, 0], [0, 130], [130, 100]], 12, 1.0, 1.0,
            f"d{d}")


@pytest.mark.parametrize("hq,hkv,mask,sk,sv", [(32, 8, [1, 0, 0, 1, 1, 0, 1, 0], 0.5, 4.0),
                                               (16, 2, [1, 0], 2.0, 0.25), (24, 3, [0, 1, 1], 1.0, 1.0)])
@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_fp8_groups_and_scales(hq, hkv, mask, sk, sv, mode):
    """G = 4, 8, 8 with tensor scales other than 1 (inputs scaled to match)."""
    require_gpu()
    _say(f"groups Hq={hq} Hkv={hkv} scales {sk} {sv} mode={mode}")
    q, k, v = qkv(3, 300, hq, hkv, 128, 92, "cuda")
    k, v = (k.float() * sk).to(torch.bfloat16), (v.float() * sv).to(torch.bfloat16)
    cache = new_cache_fp8(3, hq, hkv, 128, 300, 8, 32, mask, sk, sv, mode=mode)
    run_fp8(cache, q, k, v, mask, [[200, 3, 77], [50, 140, 0]], 6, sk, sv, f"G{hq // hkv}")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_fp8_long_one_shot_prefill_then_decode(mode):
    """A 4096-token one-shot prefill (64 key tiles per late query tile, the
    reference moving as maxima grow) and decode steps with many splits."""
    require_gpu()
    _say(f"one-shot 4096 mode={mode}")
    mask = [1, 0, 0, 1]
    q, k, v = qkv(1, 4100, 4, 4, 128, 93, "cuda")
    cache = new_cache_fp8(1, 4, 4, 128, 4100, 64, 256, mask, mode=mode)
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


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_fp8_paged_chunked_prefill_and_decode(mode):
    """fp8 rows in pages (P = 512): chunked prefill across page boundaries (the
    prefill looks up the page of every 64-row tile), then decode steps that
    open new pages; codes read back through the page table."""
    require_gpu()
    _say(f"paged chunked mode={mode}")
    mask = [1, 0, 1, 1]
    t = 1700
    q, k, v = qkv(2, t, 8, 4, 128, 96, "cuda")
    cache = new_cache_fp8(2, 8, 4, 128, t, 4, 64, mask, page_tokens=512, num_pages=8, mode=mode)
    run_fp8(cache, q, k, v, mask, [[700, 300], [600, 1000], [380, 390]], 6, 1.0, 1.0, "paged")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_fp8_paged_equals_contiguous(mode):
    """The same calls into a paged and a contiguous fp8 cache give bitwise
    equal prefill outputs and stored codes."""
    require_gpu()
    _say(f"paged == contiguous mode={mode}")
    mask = [1, 1, 0, 1]
    t = 2600
    q, k, v = qkv(2, t, 16, 4, 128, 97, "cuda")
    chunks = [[1500, 900], [1100, 1700]]
    paged = new_cache_fp8(2, 16, 4, 128, t, 64, 256, mask, page_tokens=1024, num_pages=6, mode=mode)
    flat = new_cache_fp8(2, 16, 4, 128, t, 64, 256, mask, mode=mode)
    op, _, _ = run_sequence(paged, q, k, v, chunks, 0)
    fp, _, _ = run_sequence(flat, q, k, v, chunks, 0)
    assert torch.equal(op.view(torch.int16), fp.view(torch.int16))
    a, b = duo.cache_views(paged), duo.cache_views(flat)
    for name in ("rk", "rv"):  # the paged view holds whole pages: compare the stored rows
        assert torch.equal(a[name][:, :, :t], b[name][:, :, :t]), name


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_fp8_varlen_equals_padded(mode):
    """Packed rows with cu_seqlens into an fp8 cache give the padded call's
    prefill outputs and cache bit for bit (including an empty sequence)."""
    require_gpu()
    _say(f"varlen == padded mode={mode}")
    mask = [0, 1, 1, 0]
    lens = [300, 0, 1029, 64]
    b_n, c = 4, max(lens)
    q, k, v = qkv(b_n, c, 8, 4, 128, 98, "cuda")
    pad = new_cache_fp8(b_n, 8, 4, 128, 2048, 8, 32, mask, mode=mode)
    packed = new_cache_fp8(b_n, 8, 4, 128, 2048, 8, 32, mask, mode=mode)
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
            strm = [h for h in range(8) if not mask[h // g]]
            check_retrieval_prefill(packed, got, ref[b], qn[b], kn[b], vn[b], list(range(lens[b])), mask,
                                    f"varlen b{b}")
            assert_close(got[:, strm], ref[b][:, strm], f"varlen streaming b{b}")


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_fp8_exact_prefill_is_bf16_engine_on_stored_values(paged):
    """DUO_FP8_PREFILL_EXACT gives, bit for bit, what the bf16 tile engine
    gives over a bf16 cache holding the stored values (the oracle's e4m3
    view of the retrieval heads' K and V, the streaming heads' inputs as
    given), in one-shot and chunked calls, with tensor scales other than 1
    (folded into q's pre-multiplication and the final normalisation; exact
    because they are powers of two)."""
    require_gpu()
    _say(f"exact == bf16 over stored values paged={paged}")
    mask = [1, 0, 1, 1]
    b_n, hq, hkv, d, t = 2, 16, 4, 128, 1500
    sk, sv = 2.0, 0.25
    q, k, v = qkv(b_n, t, hq, hkv, d, 99, "cuda")
    k, v = (k.float() * sk).to(torch.bfloat16), (v.float() * sv).to(torch.bfloat16)
    kn, vn = to_np32(k), to_np32(v)
    ks, vs = k.clone(), v.clone()
    for kvh in range(hkv):
        if mask[kvh]:
            for b in range(b_n):
                ks[b, :, kvh] = torch.from_numpy(seen_rows_fp8(kn[b, :, kvh], True, sk)).to(torch.bfloat16)
                vs[b, :, kvh] = torch.from_numpy(seen_rows_fp8(vn[b, :, kvh], True, sv)).to(torch.bfloat16)
    extra = dict(page_tokens=512, num_pages=b_n * 3) if paged else {}
    for chunks in ([[t, t - 100]], [[900, 1200], [600, 300]]):
        f8 = new_cache_fp8(b_n, hq, hkv, d, t, 16, 64, mask, sk, sv, **extra)
        cfg = duo.Config(b_n, hq, hkv, d, t, 16, 64, mask, **extra)
        bf = duo.duo_cache_init(cfg, torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8,
                                                device="cuda"))
        out8, _, _ = run_sequence(f8, q, k, v, chunks, 0)
        outb, _, _ = run_sequence(bf, q, ks, vs, chunks, 0)
        assert torch.equal(out8.view(torch.int16), outb.view(torch.int16)), \
            (len(chunks), (out8.float() - outb.float()).abs().max().item())


@pytest.mark.parametrize("variant", ["contiguous", "paged", "rope", "rope_paged"])
def test_fp8_staged_exact_prefill_equals_tiled(variant):
    """Exact prefill with the staging workspace (every retrieval row the call
    reads decoded once, exactly, to bf16 code * scale, then the bf16 tile
    engine) and without it (e4m3 tiles decoded in every work-group, scales
    folded into q and the normalisation): outputs and caches equal bit for
    bit, with tensor scales 2 and 1/4, also when a workspace too small for
    the later calls makes them fall back to the tiles.  The chunk plan mixes
    sequences with and without new rows, prefixes that end inside a tile,
    and chunks of one row."""
    require_gpu()
    _say(f"fp8 staged == tiled, {variant}")
    mask = [1, 0, 1, 1]
    b_n, hq, hkv, d, t = 3, 8, 4, 128, 1500
    sk, sv = 2.0, 0.25
    kw = {}
    if "paged" in variant:
        kw.update(page_tokens=512, num_pages=b_n * 3)
    if "rope" in variant:
        kw.update(rope_base=10000.0, rope_style=duo.DUO_ROPE_HALF)
    q, k, v = qkv(b_n, t, hq, hkv, d, 46, "cuda")
    k, v = (k.float() * sk).to(torch.bfloat16), (v.float() * sv).to(torch.bfloat16)
    plan = [[300, 0, 130], [1, 700, 64], [500, 1, 0], [0, 300, 900], [699, 499, 1]]
    cfg0 = duo.Config(b_n, hq, hkv, d, t, 8, 64, mask, kv_format=duo.DUO_KV_FP8, kv_scale_k=sk, kv_scale_v=sv,
                      **kw)
    n_r = sum(mask)
    # enough for rows up to 830 (the first three calls), not for the last two
    small = 4 * b_n * n_r * d * 830
    outs, caches = {}, {}
    for mode, nbytes in (("tiled", None), ("staged", duo.prefill_staging_bytes(cfg0)), ("small", small)):
        cfg = duo.Config(**{**cfg0.__dict__})
        if nbytes is not None:
            staging_workspace(cfg, nbytes)
        cache = duo.duo_cache_init(cfg, torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8,
                                                   device="cuda"))
        outs[mode], _, _ = run_sequence(cache, q, k, v, plan, 0)
        caches[mode] = cache
        torch.cuda.synchronize()
        assert torch.isfinite(outs[mode].float()).all(), mode
    for mode in ("staged", "small"):
        assert torch.equal(outs["tiled"].view(torch.int16), outs[mode].view(torch.int16)), \
            (mode, (outs["tiled"].float() - outs[mode].float()).abs().max().item())
        for name in ("rk", "rv", "sk", "sv"):
            va = duo.cache_views(caches["tiled"])[name]
            vb = duo.cache_views(caches[mode])[name]
            assert torch.equal(va.view(torch.uint8), vb.view(torch.uint8)), f"{mode} {name}"
