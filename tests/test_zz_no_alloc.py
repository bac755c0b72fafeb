"""duo_decode_static_scratch, the decode entry point that allocates nothing,
against duo_decode through the C ABI: two calls in a row (the second on a
smaller cache), outputs bit for bit equal to duo_decode's on an identical
cache and within the usual bar of the oracle.  The static-scratch cache's
own work region is filled with 0xFF bytes (NaN records, counters far from
zero) before its calls, so a call that touched it instead of the library's
array would merge garbage."""

import pytest
import torch

import kv_cache_duo_amd as duo
from parity_util import assert_close, check_cache_bits, oracle_rows, require_gpu, to_np32
from workloads import qkv

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, D, mask, prefix lengths, decode steps): many splits per
# head first, then a smaller cache (fewer units, fewer splits)
CASES = [(2, 16, 4, 128, [1, 0, 1, 1], [9000, 5000], 3), (1, 8, 2, 64, [1, 0], [700], 2)]


def _say(msg):
    print(f"[gpu-no-alloc] {msg}", flush=True)


def _cache(b, hq, hkv, d, mask, t):
    cfg = duo.Config(b, hq, hkv, d, t, 16, 64, mask)
    buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
    return duo.duo_cache_init(cfg, buf)


def test_static_scratch_decode_equals_duo_decode():
    require_gpu()
    for case in CASES:
        b_n, hq, hkv, d, mask, pre, steps = case
        _say(f"B={b_n} Hq={hq} Hkv={hkv} D={d} prefix={pre}")
        t = max(pre) + steps
        q, k, v = qkv(b_n, t, hq, hkv, d, 77, "cuda")
        ref_cache, st_cache = _cache(b_n, hq, hkv, d, mask, t), _cache(b_n, hq, hkv, d, mask, t)
        for c in (ref_cache, st_cache):
            duo.duo_cache_append(c, k[:, :max(pre)].contiguous(), v[:, :max(pre)].contiguous(), pre)
        lay = st_cache.layout()
        torch.cuda.synchronize()
        st_cache.buf[lay.work_offset:lay.work_offset + lay.work_bytes].fill_(0xFF)
        outs = []
        for s in range(steps):
            q1 = torch.stack([q[i, pre[i] + s] for i in range(b_n)]).contiguous()
            k1 = torch.stack([k[i, pre[i] + s] for i in range(b_n)]).contiguous()
            v1 = torch.stack([v[i, pre[i] + s] for i in range(b_n)]).contiguous()
            o_ref, o_st = torch.empty_like(q1), torch.empty_like(q1)
            duo.duo_decode(ref_cache, q1, k1, v1, o_ref)
            duo.duo_decode_static_scratch(st_cache, q1, k1, v1, o_st)
            outs.append((o_ref, o_st))
        torch.cuda.synchronize()
        for s, (o_ref, o_st) in enumerate(outs):
            assert torch.equal(o_ref.view(torch.int16), o_st.view(torch.int16)), f"step {s}"
        qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
        ref = oracle_rows(qn, kn, vn, mask, 16, 64, {i: [pre[i] + s for s in range(steps)] for i in range(b_n)})
        got = torch.stack([o for _, o in outs])
        for i in range(b_n):
            assert_close(to_np32(got[:, i]), ref[i], f"static scratch b{i}")
        check_cache_bits(st_cache, k, v, mask, [p + steps for p in pre])
        del ref_cache, st_cache


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_static_scratch_decode_8bit_equals_duo_decode(fmt):
    """The same two calls in a row over an int8 or fp8 retrieval cache (the
    8-bit decode kernels write the same split records): outputs and stored
    rows bit for bit equal to duo_decode's on an identical cache."""
    require_gpu()
    kv_format = duo.DUO_KV_INT8 if fmt == "int8" else duo.DUO_KV_FP8
    for case in CASES:
        b_n, hq, hkv, d, mask, pre, steps = case
        _say(f"{fmt} B={b_n} Hq={hq} Hkv={hkv} D={d} prefix={pre}")
        t = max(pre) + steps
        q, k, v = qkv(b_n, t, hq, hkv, d, 78, "cuda")
        caches = []
        for _ in range(2):
            cfg = duo.Config(b_n, hq, hkv, d, t, 16, 64, mask, kv_format=kv_format)
            caches.append(duo.duo_cache_init(cfg, torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8,
                                                             device="cuda")))
        ref_cache, st_cache = caches
        for c in caches:
            duo.duo_cache_append(c, k[:, :max(pre)].contiguous(), v[:, :max(pre)].contiguous(), pre)
        lay = st_cache.layout()
        torch.cuda.synchronize()
        st_cache.buf[lay.work_offset:lay.work_offset + lay.work_bytes].fill_(0xFF)
        outs = []
        for s in range(steps):
            q1 = torch.stack([q[i, pre[i] + s] for i in range(b_n)]).contiguous()
            k1 = torch.stack([k[i, pre[i] + s] for i in range(b_n)]).contiguous()
            v1 = torch.stack([v[i, pre[i] + s] for i in range(b_n)]).contiguous()
            o_ref, o_st = torch.empty_like(q1), torch.empty_like(q1)
            duo.duo_decode(ref_cache, q1, k1, v1, o_ref)
            duo.duo_decode_static_scratch(st_cache, q1, k1, v1, o_st)
            outs.append((o_ref, o_st))
        torch.cuda.synchronize()
        for s, (o_ref, o_st) in enumerate(outs):
            assert torch.isfinite(o_st.float()).all(), f"{fmt} step {s}"
            assert torch.equal(o_ref.view(torch.int16), o_st.view(torch.int16)), f"{fmt} step {s}"
        va, vb = duo.cache_views(ref_cache), duo.cache_views(st_cache)
        for name in ("rk", "rv", "sk", "sv") + (("rks", "rvs") if fmt == "int8" else ()):
            assert torch.equal(va[name].contiguous().view(torch.uint8), vb[name].contiguous().view(torch.uint8)), name
        del ref_cache, st_cache, caches
