"""GPU parity at the limits of the boundary: the largest batch (128
sequences), the largest number of KV heads (256), calls that add nothing,
a cache filled to exactly max_len, caches one position longer than a
1024-position row block, and decode at the split count where the merge's
arrival counting changes.  All through the C ABI against the fp64 oracle;
cache buffers start as NaN bytes."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from parity_util import assert_close, check_cache_bits, new_cache, oracle_rows, require_gpu, run_sequence, to_np32
from workloads import qkv

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-edges] {msg}", flush=True)


def test_max_batch_packed():
    """128 sequences of 0..300 tokens in one packed prefill call, then two
    decode steps; every 9th sequence checked against the oracle and read back."""
    require_gpu()
    _say("batch 128")
    b_n = duo.DUO_MAX_BATCH if hasattr(duo, "DUO_MAX_BATCH") else 128
    rng = np.random.default_rng(81)
    lens = [int(x) for x in rng.integers(0, 301, size=b_n)]
    lens[0], lens[1] = 0, 300
    mask = [1, 0]
    t = max(lens) + 2
    q, k, v = qkv(b_n, t, 4, 2, 64, 82, "cuda")
    cache = new_cache(b_n, 4, 2, 64, t, 4, 32, mask)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    qp = torch.cat([q[b, :lens[b]] for b in range(b_n)]).contiguous()
    kp = torch.cat([k[b, :lens[b]] for b in range(b_n)]).contiguous()
    vp = torch.cat([v[b, :lens[b]] for b in range(b_n)]).contiguous()
    op = torch.zeros_like(qp)
    duo.duo_prefill_varlen(cache, qp, kp, vp, cu, op)
    outd = []
    done = list(lens)
    for s in range(2):
        q1 = torch.stack([q[b, done[b]] for b in range(b_n)]).contiguous()
        k1 = torch.stack([k[b, done[b]] for b in range(b_n)]).contiguous()
        v1 = torch.stack([v[b, done[b]] for b in range(b_n)]).contiguous()
        o1 = torch.empty_like(q1)
        duo.duo_decode(cache, q1, k1, v1, o1)
        outd.append(o1)
        done = [x + 1 for x in done]
    torch.cuda.synchronize()
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    picked = list(range(0, b_n, 9)) + [1]
    ref = oracle_rows(qn, kn, vn, mask, 4, 32, {b: list(range(lens[b] + 2)) if b in picked else [] for b in range(b_n)})
    for b in picked:
        got = np.concatenate([to_np32(op[cu[b]:cu[b + 1]]), np.stack([to_np32(o[b]) for o in outd])])
        assert_close(got, ref[b], f"sequence {b} ({lens[b]} tokens)")
    check_cache_bits(cache, k, v, mask, done)


def test_max_kv_heads():
    """256 KV heads (the largest number a head map holds), MHA, every other
    one a retrieval head: 100-token prefill and 2 decode steps."""
    require_gpu()
    _say("256 KV heads")
    h = 256
    mask = [1 if i % 2 == 0 else 0 for i in range(h)]
    mask[255] = 1
    q, k, v = qkv(1, 102, h, h, 64, 83, "cuda")
    cache = new_cache(1, h, h, 64, 102, 4, 16, mask)
    qc, kc, vc = q[:, :100].contiguous(), k[:, :100].contiguous(), v[:, :100].contiguous()
    oc = torch.zeros_like(qc)
    duo.duo_prefill(cache, qc, kc, vc, [100], oc)
    outd = []
    for s in range(2):
        o1 = torch.empty(1, h, 64, dtype=torch.bfloat16, device="cuda")
        duo.duo_decode(cache, q[:, 100 + s].contiguous(), k[:, 100 + s].contiguous(), v[:, 100 + s].contiguous(), o1)
        outd.append(o1)
    torch.cuda.synchronize()
    ref = oracle_rows(to_np32(q), to_np32(k), to_np32(v), mask, 4, 16, {0: list(range(102))})[0]
    got = np.concatenate([to_np32(oc[0]), np.stack([to_np32(o[0]) for o in outd])])
    assert_close(got, ref, "256 KV heads")
    check_cache_bits(cache, k, v, mask, [102])


def test_calls_that_add_nothing():
    """A prefill and an append with n_new = 0 everywhere, and a packed call
    with no rows, leave outputs, lengths and cache bytes as they were."""
    require_gpu()
    _say("empty calls")
    mask = [1, 0]
    q, k, v = qkv(2, 50, 4, 2, 128, 84, "cuda")
    cache = new_cache(2, 4, 2, 128, 64, 4, 16, mask)
    duo.duo_prefill(cache, q, k, v, [50, 20], torch.zeros_like(q))
    torch.cuda.synchronize()
    before = cache.buf.clone()
    out = torch.full_like(q, 7.0)
    duo.duo_prefill(cache, q, k, v, [0, 0], out)
    duo.duo_cache_append(cache, k, v, [0, 0])
    duo.duo_prefill_varlen(cache, q[0, :0].contiguous(), k[0, :0].contiguous(), v[0, :0].contiguous(), [0, 0, 0],
                           out[0, :0].contiguous())
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    assert cache.lengths() == [50, 20]
    views = duo.cache_views(cache)
    # the split-K records are scratch; every other byte is unchanged
    lay = cache.layout()
    keep = torch.ones_like(before, dtype=torch.bool)
    keep[lay.work_offset:lay.work_offset + lay.work_bytes] = False
    assert torch.equal(cache.buf[keep], before[keep])
    assert views["lengths"].cpu().tolist() == [50, 20]


def test_exactly_full_cache():
    """Prefill to max_len - 1, one decode step to exactly max_len, then every
    call that would add a token fails with CAPACITY and changes nothing."""
    require_gpu()
    _say("full cache")
    mask = [1, 0]
    n = 300
    q, k, v = qkv(1, n, 4, 2, 128, 85, "cuda")
    cache = new_cache(1, 4, 2, 128, n, 4, 64, mask)
    outp = torch.zeros(1, n - 1, 4, 128, dtype=torch.bfloat16, device="cuda")
    duo.duo_prefill(cache, q[:, :n - 1].contiguous(), k[:, :n - 1].contiguous(), v[:, :n - 1].contiguous(), [n - 1],
                    outp)
    o1 = torch.empty(1, 4, 128, dtype=torch.bfloat16, device="cuda")
    duo.duo_decode(cache, q[:, n - 1].contiguous(), k[:, n - 1].contiguous(), v[:, n - 1].contiguous(), o1)
    torch.cuda.synchronize()
    ref = oracle_rows(to_np32(q), to_np32(k), to_np32(v), mask, 4, 64, {0: list(range(n))})[0]
    assert_close(np.concatenate([to_np32(outp[0]), to_np32(o1)]), ref, "up to max_len")
    before = cache.buf.clone()
    for call in (lambda: duo.duo_decode(cache, q[:, 0].contiguous(), k[:, 0].contiguous(), v[:, 0].contiguous(), o1),
                 lambda: duo.duo_prefill(cache, q[:, :1].contiguous(), k[:, :1].contiguous(), v[:, :1].contiguous(),
                                         [1], torch.zeros_like(q[:, :1])),
                 lambda: duo.duo_cache_append(cache, k[:, :1].contiguous(), v[:, :1].contiguous(), [1])):
        with pytest.raises(duo.DuoError) as e:
            call()
        assert e.value.status == duo.DUO_ERR_CAPACITY
    torch.cuda.synchronize()
    assert cache.lengths() == [n] and torch.equal(cache.buf, before)
    check_cache_bits(cache, k, v, mask, [n])


@pytest.mark.parametrize("fmt", ["bf16", "int8", "fp8"])
def test_block_boundary(fmt):
    """A contiguous cache one position longer than a 1024-position block (two
    blocks, the second nearly empty): chunked prefill to 1020 rows, then
    decode steps that cross into the second block; outputs against each
    format's oracle, cache read back through the reordered views."""
    require_gpu()
    _say(f"block boundary {fmt}")
    mask = [1, 0, 1, 1]
    t, pre, steps = 1025, 1020, 5
    q, k, v = qkv(2, t, 8, 4, 128, 86, "cuda")
    kw = {"bf16": {}, "int8": dict(kv_format=duo.DUO_KV_INT8), "fp8": dict(kv_format=duo.DUO_KV_FP8)}[fmt]
    cfg = duo.Config(2, 8, 4, 128, t, 4, 32, mask, **kw)
    cache = duo.duo_cache_init(cfg, torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda"))
    assert cache.layout().block_tokens == 1024
    chunks = [[700, 1000], [320, 20]]
    if fmt == "bf16":
        outp, outd, done = run_sequence(cache, q, k, v, chunks, steps)
        qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
        ref = oracle_rows(qn, kn, vn, mask, 4, 32, {b: list(range(pre + steps)) for b in range(2)})
        for b in range(2):
            assert_close(to_np32(outp[b, :pre]), ref[b][:pre], f"prefill b{b}")
            assert_close(to_np32(outd[:, b]), ref[b][pre:], f"decode b{b}")
        check_cache_bits(cache, k, v, mask, done)
    elif fmt == "int8":
        from test_gpu_int8 import run_q8
        run_q8(cache, q, k, v, chunks, steps, mask)
    else:
        from test_gpu_fp8 import run_fp8
        run_fp8(cache, q, k, v, mask, chunks, steps, 1.0, 1.0, "block boundary")


@pytest.mark.parametrize("stored", [12287, 12288])
def test_decode_split_count_boundary(stored):
    """One retrieval and one streaming KV head: decode splits a unit's rows
    into ~384-row pieces, so 12288 and 12289 rows give 32 and 33 work-groups
    on a 256-CU device: the last arrival counts on the unit's counter alone
    at 32, through the group counters at 33.  Three steps cross from one
    side to the other and back into a fresh call."""
    require_gpu()
    _say(f"split-count boundary, {stored} stored rows")
    mask = [1, 0]
    steps = 3
    t = stored + steps
    q, k, v = qkv(1, t, 2, 2, 128, 83, "cuda")
    cache = new_cache(1, 2, 2, 128, t, 64, 256, mask)
    duo.duo_cache_append(cache, k[:, :stored].contiguous(), v[:, :stored].contiguous(), [stored])
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    for s in range(steps):
        p = stored + s
        o1 = torch.empty(1, 2, 128, dtype=torch.bfloat16, device="cuda")
        duo.duo_decode(cache, q[:, p].contiguous(), k[:, p].contiguous(), v[:, p].contiguous(), o1)
        ref = oracle_rows(qn, kn, vn, mask, 64, 256, {0: [p]})[0]
        assert_close(to_np32(o1), ref, f"decode at {p}")
    torch.cuda.synchronize()
    check_cache_bits(cache, k, v, mask, [t])
