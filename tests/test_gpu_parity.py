"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

All inputs are seeded N(0,1) rounded to bf16 (plus the stress inputs of the
oracle pins); every cache buffer is poisoned with NaN bytes first, so a read
of any slot the method must not use shows up as a non-finite output.
"""

import math

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from parity_util import (assert_close, check_cache_bits, decode_steps_poisoned, new_cache, oracle_rows, require_gpu,
                         run_sequence, to_np32)
from workloads import WORKLOADS, qkv, randn_bf16, workload_mask

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)


def _full_check(cache, q, k, v, mask, sink, recent, chunks, steps, what):
    outp, outd, done = run_sequence(cache, q, k, v, chunks, steps)
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    b_n = q.shape[0]
    pre = [sum(c[b] for c in chunks) for b in range(b_n)]
    rows = {b: list(range(pre[b] + steps)) for b in range(b_n)}
    ref = oracle_rows(qn, kn, vn, mask, sink, recent, rows)
    for b in range(b_n):
        if pre[b]:
            assert_close(to_np32(outp[b, :pre[b]]), ref[b][:pre[b]], f"{what} prefill b{b}")
        if steps:
            assert_close(to_np32(outd[:, b]), ref[b][pre[b]:], f"{what} decode b{b}")
    check_cache_bits(cache, k, v, mask, done)
    return outp, outd


def test_tiny_mha_full_parity():
    """4 heads (2 retrieval, 2 streaming), D=64, prefill 512 + 16 decode steps, S=4, W=64."""
    require_gpu()
    w = WORKLOADS["tiny_mha_512"]
    _say(w.name)
    mask = workload_mask(w)
    t = w.prefill + w.decode_steps
    q, k, v = qkv(w.batch, t, w.num_q_heads, w.num_kv_heads, w.head_dim, w.seed, "cuda")
    cache = new_cache(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, t, w.sink, w.recent, mask)
    _full_check(cache, q, k, v, mask, w.sink, w.recent, [[w.prefill]], w.decode_steps, w.name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chunk", [1, 3, 63, 64, 65, 100, 300])
def test_chunked_prefill_matches_oracle(d, chunk):
    """Chunk sizes around the window (W=64) exercise the ring overwrite order."""
    require_gpu()
    _say(f"chunked d={d} chunk={chunk}")
    total, steps, sink, recent = 300, 5, 4, 64
    mask = [1, 0, 0, 1]
    q, k, v = qkv(1, total + steps, 4, 4, d, 100 + chunk, "cuda")
    cache = new_cache(1, 4, 4, d, total + steps, sink, recent, mask)
    plan, left = [], total
    while left:
        n = min(chunk, left)
        plan.append([n])
        left -= n
    _full_check(cache, q, k, v, mask, sink, recent, plan, steps, f"chunk{chunk}")


def test_gqa_mixed_lengths_and_empty_rows():
    """G=4, three sequences of different lengths, n_b = 0 in some calls."""
    require_gpu()
    _say("gqa mixed lengths")
    mask = [1, 0]
    sink, recent = 8, 40
    chunks = [[200, 0, 77], [50, 130, 0], [0, 1, 129]]
    steps = 4
    t = 300
    q, k, v = qkv(3, t, 8, 2, 128, 7, "cuda")
    cache = new_cache(3, 8, 2, 128, t, sink, recent, mask)
    _full_check(cache, q, k, v, mask, sink, recent, chunks, steps, "gqa-mixed")


def test_many_units_mixed_lengths():
    """16 sequences of different lengths, 2 retrieval KV heads each (32
    retrieval units, G = 4): the first two calls are balanced enough for the
    prefill's snake deal of units to the 8 XCDs (one-shot rows of 120..600
    tokens, then 48 rows over those prefixes), the last two are not (skipped
    sequences, ragged rows) and take the t-major order."""
    require_gpu()
    _say("many units, mixed lengths")
    b_n, mask = 16, [1, 0, 1, 0]
    sink, recent = 16, 64
    chunks = [[120 + 32 * i for i in range(b_n)], [48] * b_n,
              [0 if i % 3 == 0 else 60 + 19 * i for i in range(b_n)], [180 - 10 * i for i in range(b_n)]]
    steps = 2
    t = max(sum(c[b] for c in chunks) for b in range(b_n)) + steps
    q, k, v = qkv(b_n, t, 16, 4, 128, 77, "cuda")
    cache = new_cache(b_n, 16, 4, 128, t, sink, recent, mask)
    _full_check(cache, q, k, v, mask, sink, recent, chunks, steps, "many-units")


@pytest.mark.parametrize("hq,hkv,mask", [(24, 3, [0, 1, 0]), (6, 2, [1, 0]), (16, 8, [1, 0, 0, 1, 1, 0, 1, 0])])
def test_group_sizes(hq, hkv, mask):
    """G = 8, 3 and 2: head chunking in prefill and decode."""
    require_gpu()
    _say(f"group hq={hq} hkv={hkv}")
    sink, recent, n, steps = 4, 32, 150, 3
    q, k, v = qkv(2, n + steps, hq, hkv, 128, 11 + hq, "cuda")
    cache = new_cache(2, hq, hkv, 128, n + steps, sink, recent, mask)
    _full_check(cache, q, k, v, mask, sink, recent, [[n, n - 17]], steps, f"g{hq // hkv}")


@pytest.mark.parametrize("sink,recent,mask", [
    (0, 16, [0, 0]),        # pure sliding window (StreamingLLM without sinks)
    (5, 1, [0, 1]),         # window of one: sinks + self
    (64, 200, [0, 0]),      # window + sinks cover the whole sequence: no eviction
    (4, 32, [1, 1]),        # full attention for every head
    (3, 7, [0, 0]),         # every head streaming (StreamingLLM)
])
def test_edge_windows(sink, recent, mask):
    require_gpu()
    _say(f"edge sink={sink} recent={recent} mask={mask}")
    n, steps = 190, 6
    q, k, v = qkv(1, n + steps, 4, 2, 64, 5 + sink + recent, "cuda")
    cache = new_cache(1, 4, 2, 64, n + steps, sink, recent, mask)
    _full_check(cache, q, k, v, mask, sink, recent, [[n]], steps, "edge")


def test_stress_inputs():
    """Peaky softmax, monotone scores (max rises every tile), planted sink."""
    require_gpu()
    _say("stress")
    n, d, sink, recent = 400, 128, 4, 64
    mask = [1, 0]
    g = torch.Generator(device="cpu").manual_seed(9)
    base = torch.randn(d, generator=g)
    q = (torch.randn(1, n, 2, d, generator=g) * 8)
    q[:, :, 1] = base / base.norm() * 6
    k = torch.randn(1, n, 2, d, generator=g)
    k[0, :, 0] = torch.outer(torch.arange(n) / 40.0, base) + 0.05 * torch.randn(n, d, generator=g)
    k[0, 0, 1] = base * 4  # planted sink for the streaming head
    v = torch.randn(1, n, 2, d, generator=g)
    q, k, v = (x.to(torch.bfloat16).cuda() for x in (q, k, v))
    cache = new_cache(1, 2, 2, d, n, sink, recent, mask)
    _full_check(cache, q, k, v, mask, sink, recent, [[n - 8]], 8, "stress")


# (name, B, Hq, Hkv, D, mask, prefill lengths, decode steps, kv_format):
# a few splits per head chunk (G = 4); one query head per work-group with
# ~80 splits (direct arrivals, single-pass merge); ~200 splits (grouped
# arrivals and the two-level merge); an int8 cache.
DETERMINISM_CASES = [
    ("gqa_700", 2, 16, 4, 128, [1, 0, 1, 0], [600, 650], 40, 0),
    ("mha_20k", 1, 8, 8, 128, [1, 0, 0, 1, 0, 0, 0, 0], [20000], 4, 0),
    ("single_100k", 1, 2, 2, 128, [1, 0], [100000], 3, 0),
    ("int8_gqa_9k", 2, 16, 4, 128, [0, 1, 1, 0], [9000, 7000], 4, 1),
]


@pytest.mark.parametrize("case", DETERMINISM_CASES, ids=[c[0] for c in DETERMINISM_CASES])
def test_deterministic(case):
    """Two runs on the same inputs give bitwise equal prefill outputs, cache
    bytes and decode outputs (the default static decode split: fixed rows
    per work-group, records merged in work-group order).  The split records
    are filled with NaN bytes before every decode call, so a record read
    before its store in that call would show as a non-finite output."""
    require_gpu()
    name, b_n, hq, hkv, d, mask, lens, steps, fmt = case
    _say(f"determinism {name}")
    t = max(lens) + steps
    q, k, v = qkv(b_n, t, hq, hkv, d, 21, "cuda")
    outs, caches = [], []
    for _ in range(2):
        cfg = duo.Config(b_n, hq, hkv, d, t, 16, 64, mask, kv_format=fmt)
        buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
        cache = duo.duo_cache_init(cfg, buf)
        if max(lens) > 20000:  # long context: fill by append, prefill only the last 64 tokens
            pre = [n - 64 for n in lens]
            duo.duo_cache_append(cache, k[:, :max(pre)].contiguous(), v[:, :max(pre)].contiguous(), pre)
            c = 64
            qc = torch.stack([q[i, pre[i]:pre[i] + c] for i in range(b_n)]).contiguous()
            kc = torch.stack([k[i, pre[i]:pre[i] + c] for i in range(b_n)]).contiguous()
            vc = torch.stack([v[i, pre[i]:pre[i] + c] for i in range(b_n)]).contiguous()
            outp = torch.empty_like(qc)
            duo.duo_prefill(cache, qc, kc, vc, [c] * b_n, outp)
        else:
            outp, _, _ = run_sequence(cache, q, k, v, [lens], 0)
        outd = decode_steps_poisoned(cache, q, k, v, lens, steps)
        outs.append((outp, outd))
        caches.append(cache)
    assert torch.isfinite(outs[0][1].float()).all(), "decode read a record before writing it"
    assert torch.equal(outs[0][0], outs[1][0]), "prefill outputs differ"
    assert torch.equal(outs[0][1], outs[1][1]), "decode outputs differ"
    views = [duo.cache_views(c) for c in caches]
    for vname in views[0]:  # raw bits: unused rows hold the NaN poison
        x, y = views[0][vname], views[1][vname]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        elif x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), vname


def test_dynamic_split_within_summation_order_bound():
    """DUO_DECODE_DYNAMIC: work-groups claim rows at run time, so the fp32
    sums of a decode output may associate differently between runs.  Two
    recursive fp32 sums of the same n terms in different orders differ by at
    most about 2 (n - 1) u sum|terms| (u = 2^-24, the standard bound for
    recursive summation).  The output is sum(p_j v_j) / sum(p_j) with
    p_j >= 0, so the two fp32 results differ by at most
    4 (n - 1) u max|v| + 2 (n - 1) u |o|, and their bf16 roundings by that
    plus one bf16 ulp of the larger (<= 2^-7 |o|).  Both runs also meet the
    oracle bar and stay finite with poisoned records."""
    require_gpu()
    _say("dynamic split")
    mask = [1, 0]
    n, steps = 9000, 3
    q, k, v = qkv(2, n + steps, 8, 2, 128, 31, "cuda")
    outs = []
    for _ in range(2):
        cfg = duo.Config(2, 8, 2, 128, n + steps, 64, 256, mask, decode_split=duo.DUO_DECODE_DYNAMIC)
        buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
        cache = duo.duo_cache_init(cfg, buf)
        duo.duo_cache_append(cache, k[:, :n].contiguous(), v[:, :n].contiguous(), [n, n - 4000])
        outs.append(decode_steps_poisoned(cache, q, k, v, [n, n - 4000], steps))
    a, b = outs[0].double(), outs[1].double()
    assert torch.isfinite(a).all() and torch.isfinite(b).all()
    u = 2.0 ** -24
    vmax = v.float().abs().max().item()
    big = torch.maximum(a.abs(), b.abs())
    bound = 4 * (n + steps) * u * vmax + (2 * (n + steps) * u + 2.0 ** -7) * big
    assert ((a - b).abs() <= bound).all(), ((a - b).abs() - bound).max().item()
    kn, vn, qn = to_np32(k), to_np32(v), to_np32(q)
    pos = [n, n - 4000]
    ref = oracle_rows(qn, kn, vn, mask, 64, 256, {i: [pos[i] + s for s in range(steps)] for i in range(2)})
    for i in range(2):
        assert_close(to_np32(outs[0][:, i]), ref[i], f"dynamic b{i}")


def test_decode_many_splits():
    """Long retrieval context so decode uses many split-K work-groups (and
    the last-work-group merge), checked at several lengths."""
    require_gpu()
    _say("decode splits")
    mask = [1, 0]
    n, steps = 9000, 3
    q, k, v = qkv(2, n + steps, 8, 2, 128, 31, "cuda")
    cache = new_cache(2, 8, 2, 128, n + steps, 64, 256, mask)
    # fill by append (no attention), then decode
    duo.duo_cache_append(cache, k[:, :n].contiguous(), v[:, :n].contiguous(), [n, n - 4000])
    outd = []
    pos = [n, n - 4000]
    for s in range(steps):
        q1 = torch.stack([q[b, pos[b] + s] for b in range(2)]).contiguous()
        k1 = torch.stack([k[b, pos[b] + s] for b in range(2)]).contiguous()
        v1 = torch.stack([v[b, pos[b] + s] for b in range(2)]).contiguous()
        o1 = torch.empty_like(q1)
        duo.duo_decode(cache, q1, k1, v1, o1)
        outd.append(o1)
    torch.cuda.synchronize()
    outd = torch.stack(outd)
    kn, vn, qn = to_np32(k), to_np32(v), to_np32(q)
    ref = oracle_rows(qn, kn, vn, mask, 64, 256, {b: [pos[b] + s for s in range(steps)] for b in range(2)})
    for b in range(2):
        assert_close(to_np32(outd[:, b]), ref[b], f"decode-splits b{b}")
    check_cache_bits(cache, k, v, mask, [p + steps for p in pos])


def test_llama2_mha_32k_full_size_sampled():
    """Full-size Llama-2-7B-shaped MHA layer as the benchmark runs it:
    one-shot prefill of 32768 tokens, then 256 decode steps; sampled rows of
    every head against the oracle."""
    require_gpu()
    w = WORKLOADS["llama2_7b_mha_32k"]
    _say(w.name)
    mask = workload_mask(w)
    t = w.prefill + w.decode_steps
    q, k, v = qkv(1, t, w.num_q_heads, w.num_kv_heads, w.head_dim, w.seed, "cuda")
    cache = new_cache(1, w.num_q_heads, w.num_kv_heads, w.head_dim, t, w.sink, w.recent, mask)
    outp, outd, done = run_sequence(cache, q, k, v, [[w.prefill]], w.decode_steps)
    rng = np.random.default_rng(0)
    s, wd = w.sink, w.recent
    rows = sorted(set([0, 1, s - 1, s, s + wd - 1, s + wd, 4095, 4096, w.prefill - 1] +
                      rng.integers(0, w.prefill, 12).tolist()))
    steps = [0, 1, 127, 255]
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    ref = oracle_rows(qn, kn, vn, mask, s, wd, {0: rows + [w.prefill + x for x in steps]})[0]
    assert_close(to_np32(outp[0, rows]), ref[:len(rows)], "32k prefill")
    assert_close(to_np32(outd[steps, 0]), ref[len(rows):], "32k decode")
    check_cache_bits(cache, k, v, mask, done)
