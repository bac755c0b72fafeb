"""GPU parity of the paged retrieval cache and of packed (variable-length)
inputs.

Paging and packing change where rows live, never what is computed: the
oracle is the same positional definition.  Checked here: outputs against the
oracle, the stored rows read back through each sequence's pages (bit for
bit), page accounting (every sequence holds ceil(len / P) distinct pages,
released pages return to the pool and are reused), and equality with the
contiguous cache and padded inputs (prefill outputs bitwise: the same
kernels in the same order).  Every cache buffer starts as NaN bytes."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from parity_util import assert_close, check_cache_bits, oracle_rows, require_gpu, run_sequence, to_np32
from test_gpu_int8 import check_cache_q8, oracle_q8
from test_gpu_rope import check_cache_rope, oracle_rope
from workloads import qkv

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-paged] {msg}", flush=True)


def new_cache_paged(batch, hq, hkv, d, max_len, sink, recent, mask, page_tokens, num_pages, **kw):
    cfg = duo.Config(batch, hq, hkv, d, max_len, sink, recent, [int(x) for x in mask], page_tokens=page_tokens,
                     num_pages=num_pages, **kw)
    buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
    return duo.duo_cache_init(cfg, buf)


def check_pages(cache, lengths):
    p = cache.cfg.page_tokens
    seen = set()
    for b, n in enumerate(lengths):
        pages, free = cache.pages(b)
        assert len(pages) == (n + p - 1) // p, f"sequence {b}: {len(pages)} pages for {n} tokens"
        assert not seen.intersection(pages), "a page is held by two sequences"
        seen.update(pages)
    assert free == cache.cfg.num_pages - len(seen)
    table = duo.cache_views(cache)["page_table"].cpu()
    for b in range(cache.cfg.batch):
        pages, _ = cache.pages(b)
        assert table[b, :len(pages)].tolist() == pages, f"device page table of sequence {b}"


def full_check(cache, q, k, v, mask, chunks, steps, what):
    cfg = cache.cfg
    outp, outd, done = run_sequence(cache, q, k, v, chunks, steps)
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    pre = [sum(c[b] for c in chunks) for b in range(cfg.batch)]
    ref = oracle_rows(qn, kn, vn, mask, cfg.sink, cfg.recent, {b: list(range(pre[b] + steps)) for b in range(cfg.batch)})
    for b in range(cfg.batch):
        if pre[b]:
            assert_close(to_np32(outp[b, :pre[b]]), ref[b][:pre[b]], f"{what} prefill b{b}")
        if steps:
            assert_close(to_np32(outd[:, b]), ref[b][pre[b]:], f"{what} decode b{b}")
    check_cache_bits(cache, k, v, mask, done)
    check_pages(cache, done)
    return outp, outd, done


@pytest.mark.parametrize("d", [64, 128])
def test_paged_chunked_prefill_and_decode(d):
    """Three sequences growing across page boundaries (P = 512) in chunks,
    then decode steps that open new pages."""
    require_gpu()
    _say(f"paged d={d}")
    mask = [1, 0, 1, 0]
    t = 2100
    q, k, v = qkv(3, t, 8, 4, d, 61, "cuda")
    cache = new_cache_paged(3, 8, 4, d, t, 4, 64, mask, 512, 14)
    full_check(cache, q, k, v, mask, [[700, 1, 1300], [600, 1000, 5], [2, 500, 300]], 8, f"paged d{d}")


def test_paged_equals_contiguous():
    """Same inputs into a paged and a contiguous cache: prefill outputs
    equal bit for bit, decode within the usual bar of each other."""
    require_gpu()
    _say("paged == contiguous")
    mask = [1, 1, 0, 1]
    t = 3000
    q, k, v = qkv(2, t, 16, 4, 128, 62, "cuda")
    chunks = [[1500, 900], [1400, 2000]]
    paged = new_cache_paged(2, 16, 4, 128, t, 64, 256, mask, 1024, 7)
    cfg = duo.Config(2, 16, 4, 128, t, 64, 256, mask)
    flat = duo.duo_cache_init(cfg, torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda"))
    op, od, _ = run_sequence(paged, q, k, v, chunks, 4)
    fp, fd, _ = run_sequence(flat, q, k, v, chunks, 4)
    assert torch.equal(op.view(torch.int16), fp.view(torch.int16))
    assert_close(to_np32(od), to_np32(fd).astype(np.float64), "decode paged vs contiguous")


def test_release_and_reuse():
    """Sequence 1 ends, its pages return to the pool, and a new sequence in
    its slot takes pages (some of them the old ones) and is attended
    correctly; sequence 0 is untouched."""
    require_gpu()
    _say("release + reuse")
    mask = [1, 0]
    q, k, v = qkv(2, 1600, 4, 2, 128, 63, "cuda")
    q2, k2, v2 = qkv(2, 1600, 4, 2, 128, 64, "cuda")
    cache = new_cache_paged(2, 4, 2, 128, 1600, 4, 64, mask, 512, 6)
    run_sequence(cache, q, k, v, [[1000, 1500]], 0)
    assert cache.pages(1)[1] == 1  # 2 + 3 pages held
    old = cache.pages(1)[0]
    duo.duo_cache_release(cache, 1)
    assert cache.lengths() == [1000, 0] and cache.pages(1) == ([], 4)
    assert duo.cache_views(cache)["lengths"].cpu().tolist() == [1000, 0]
    # slot 1 restarts from the second set of inputs; slot 0 continues
    b_n, c = 2, 600
    qc = torch.zeros(b_n, c, 4, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(b_n, c, 2, 128, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    qc[0], kc[0], vc[0] = q[0, 1000:1000 + c], k[0, 1000:1000 + c], v[0, 1000:1000 + c]
    qc[1], kc[1], vc[1] = q2[1, :c], k2[1, :c], v2[1, :c]
    oc = torch.zeros_like(qc)
    duo.duo_prefill(cache, qc, kc, vc, [c, c], oc)
    torch.cuda.synchronize()
    assert set(cache.pages(1)[0]) <= set(old) | set(range(6))
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    r0 = oracle_rows(qn[:1], kn[:1], vn[:1], mask, 4, 64, {0: list(range(1000, 1000 + c))})[0]
    assert_close(to_np32(oc[0]), r0, "continuing sequence")
    qn2, kn2, vn2 = to_np32(q2[1:]), to_np32(k2[1:]), to_np32(v2[1:])
    r1 = oracle_rows(qn2, kn2, vn2, mask, 4, 64, {0: list(range(c))})[0]
    assert_close(to_np32(oc[1]), r1, "new sequence in a released slot")
    kall = torch.stack([k[0], torch.cat([k2[1, :c], k2[1, c:]])])
    vall = torch.stack([v[0], torch.cat([v2[1, :c], v2[1, c:]])])
    check_cache_bits(cache, kall, vall, mask, [1000 + c, c])
    check_pages(cache, [1000 + c, c])


def test_varlen_equals_padded():
    """Packed rows with cu_seqlens give the padded call's outputs and cache
    bit for bit (prefill) and continue identically."""
    require_gpu()
    _say("varlen == padded")
    mask = [0, 1, 1, 0]
    lens = [300, 0, 1029, 64]
    b_n, c = 4, max(lens)
    q, k, v = qkv(b_n, c, 8, 4, 128, 65, "cuda")
    cfg = duo.Config(b_n, 8, 4, 128, 2048, 8, 32, mask)

    def fresh():
        return duo.duo_cache_init(cfg, torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda"))

    pad, packed = fresh(), fresh()
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
    # a second packed call through append_varlen and the padded append
    more = [5, 7, 0, 100]
    k2, v2 = qkv(b_n, 100, 8, 4, 128, 66, "cuda")[1:]
    duo.duo_cache_append(pad, k2, v2, more)
    cu2 = [0]
    for n in more:
        cu2.append(cu2[-1] + n)
    duo.duo_cache_append_varlen(packed, torch.cat([k2[b, :more[b]] for b in range(b_n)]).contiguous(),
                                torch.cat([v2[b, :more[b]] for b in range(b_n)]).contiguous(), cu2)
    torch.cuda.synchronize()
    for b in range(b_n):
        assert torch.equal(out_p[cu[b]:cu[b + 1]].view(torch.int16), out_pad[b, :lens[b]].view(torch.int16)), f"b{b}"
    vp_views, vq_views = duo.cache_views(pad), duo.cache_views(packed)
    for name in ("rk", "rv", "sk", "sv"):
        a16, b16 = vp_views[name].view(torch.int16), vq_views[name].view(torch.int16)
        assert torch.equal(a16, b16), name
    assert pad.lengths() == packed.lengths() == [lens[b] + more[b] for b in range(b_n)]
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    ref = oracle_rows(qn, kn, vn, mask, 8, 32, {b: list(range(lens[b])) for b in range(b_n)})
    for b in range(b_n):
        if lens[b]:
            assert_close(to_np32(out_p[cu[b]:cu[b + 1]]), ref[b], f"varlen b{b}")


def test_paged_int8():
    """int8 retrieval rows in pages: codes and scales read back through the
    page table bit for bit, outputs against the quantized-cache oracle."""
    require_gpu()
    _say("paged int8")
    mask = [1, 0, 0, 1]
    q, k, v = qkv(2, 1300, 8, 4, 128, 67, "cuda")
    cache = new_cache_paged(2, 8, 4, 128, 1300, 4, 64, mask, 512, 6, kv_format=duo.DUO_KV_INT8)
    from test_gpu_int8 import run_q8
    done = run_q8(cache, q, k, v, [[600, 1000], [500, 200]], 5, mask)
    check_pages(cache, done)


def test_paged_rope():
    """Rotary embedding with a paged cache (retrieval keys read through the
    pages after their rotated store)."""
    require_gpu()
    _say("paged rope")
    mask = [1, 0]
    q, k, v = qkv(2, 1400, 4, 2, 128, 68, "cuda")
    cache = new_cache_paged(2, 4, 2, 128, 1400, 4, 64, mask, 512, 6, rope_base=10000.0, rope_style=duo.DUO_ROPE_HALF)
    from test_gpu_rope import run_and_check
    run_and_check(cache, q, k, v, mask, [[1000, 700], [300, 600]], 6, 10000.0, duo.DUO_ROPE_HALF, "paged rope")
    check_pages(cache, [1306, 1306])


def test_mixed_batch_paged_varlen():
    """The mixed-length batch served the paged way: 8 sequences of 1000..9000
    tokens, prefilled in packed chunks of up to 2048 rows, then decoded; the
    pool holds only the pages the lengths need (sum of ceil(len / P)) where
    a contiguous cache reserves B * max_len rows."""
    require_gpu()
    rng = np.random.default_rng(69)
    lens = [int(x) for x in rng.integers(1000, 9001, size=8)]
    _say(f"mixed batch {lens}")
    mask = [1, 0, 1, 0, 0, 1, 0, 0]
    p, steps = 512, 3
    pages = sum((n + steps + p - 1) // p for n in lens)
    t = max(lens) + steps
    q, k, v = qkv(8, t, 32, 8, 128, 70, "cuda")
    cache = new_cache_paged(8, 32, 8, 128, 16384, 64, 256, mask, p, pages)
    flat = duo.Config(8, 32, 8, 128, 16384, 64, 256, mask)
    assert duo.required_bytes(cache.cfg) < 0.75 * duo.required_bytes(flat)
    done = [0] * 8
    outs = {b: [] for b in range(8)}
    while any(done[b] < lens[b] for b in range(8)):
        n = [min(2048, lens[b] - done[b]) for b in range(8)]
        cu = [0]
        for x in n:
            cu.append(cu[-1] + x)
        qp = torch.cat([q[b, done[b]:done[b] + n[b]] for b in range(8)]).contiguous()
        kp = torch.cat([k[b, done[b]:done[b] + n[b]] for b in range(8)]).contiguous()
        vp = torch.cat([v[b, done[b]:done[b] + n[b]] for b in range(8)]).contiguous()
        op = torch.zeros_like(qp)
        duo.duo_prefill_varlen(cache, qp, kp, vp, cu, op)
        for b in range(8):
            outs[b].append(op[cu[b]:cu[b + 1]])
        done = [done[b] + n[b] for b in range(8)]
    for s in range(steps):
        q1 = torch.stack([q[b, done[b]] for b in range(8)]).contiguous()
        k1 = torch.stack([k[b, done[b]] for b in range(8)]).contiguous()
        v1 = torch.stack([v[b, done[b]] for b in range(8)]).contiguous()
        o1 = torch.empty_like(q1)
        duo.duo_decode(cache, q1, k1, v1, o1)
        for b in range(8):
            outs[b].append(o1[b:b + 1])
        done = [x + 1 for x in done]
    torch.cuda.synchronize()
    assert cache.pages(0)[1] == 0  # the pool is exactly used up
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    # sampled rows of every sequence: chunk edges, the last prefill row, every decode step
    rows = {b: sorted({0, 1, 2047, 2048, lens[b] - 1} | {lens[b] + s for s in range(steps)}) for b in range(8)}
    rows = {b: [r for r in rs if r < lens[b] + steps] for b, rs in rows.items()}
    ref = oracle_rows(qn, kn, vn, mask, 64, 256, rows)
    for b in range(8):
        got = torch.cat(outs[b])
        assert_close(to_np32(got[rows[b]]), ref[b], f"mixed b{b}")
    check_pages(cache, done)
