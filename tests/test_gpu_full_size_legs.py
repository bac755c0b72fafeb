"""GPU parity of the benchmark's variant legs at full size: the
llama2_7b_mha_32k layer (32 heads, D = 128, 8 retrieval heads, one-shot
32768-token prefill, 256 decode steps) exactly as the benchmark launches it,
with

  * an int8 retrieval cache (DUO_KV_INT8),
  * rotary position embedding (base 10000, half-split pairs),
  * a paged retrieval cache (1024-position pages, a pool just large enough),
  * an fp8 (e4m3) retrieval cache with unit tensor scales (DUO_KV_FP8).

Sampled prefill rows and decode steps of every query head are compared with
the oracle of each format at the bar its own tests state; the cache is read
back (bit for bit, or for rotated keys within the rotation tolerance)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from parity_util import assert_close, check_cache_bits, oracle_rows, require_gpu, run_sequence, to_np32
from test_gpu_fp8 import assert_fp8_close, check_cache_fp8, oracle_fp8
from test_gpu_int8 import check_cache_q8, oracle_q8
from test_gpu_rope import check_cache_rope, oracle_rope
from workloads import WORKLOADS, qkv, workload_mask

pytestmark = pytest.mark.gpu

W = WORKLOADS["llama2_7b_mha_32k"]
STEPS = [0, 1, 127, 255]


def _say(msg):
    print(f"[gpu-legs] {msg}", flush=True)


def _sampled_rows():
    rng = np.random.default_rng(0)
    s, wd = W.sink, W.recent
    return sorted(set([0, 1, s - 1, s, s + wd - 1, s + wd, 4095, 4096, W.prefill - 1] +
                      rng.integers(0, W.prefill, 8).tolist()))


def _cache(leg, mask, t):
    kw = {}
    if leg == "int8":
        kw = dict(kv_format=duo.DUO_KV_INT8)
    elif leg == "rope":
        kw = dict(rope_base=10000.0, rope_style=duo.DUO_ROPE_HALF)
    elif leg == "paged":
        kw = dict(page_tokens=1024, num_pages=(t + 1023) // 1024)
    elif leg == "fp8":
        kw = dict(kv_format=duo.DUO_KV_FP8)
    cfg = duo.Config(W.batch, W.num_q_heads, W.num_kv_heads, W.head_dim, t, W.sink, W.recent,
                     [int(x) for x in mask], **kw)
    buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
    return duo.duo_cache_init(cfg, buf)


@pytest.mark.parametrize("leg", ["int8", "rope", "paged", "fp8"])
def test_bench_layer_leg(leg):
    require_gpu()
    _say(f"{W.name} {leg}")
    mask = workload_mask(W)
    t = W.prefill + W.decode_steps
    q, k, v = qkv(1, t, W.num_q_heads, W.num_kv_heads, W.head_dim, W.seed, "cuda")
    cache = _cache(leg, mask, t)
    outp, outd, done = run_sequence(cache, q, k, v, [[W.prefill]], W.decode_steps)
    rows = _sampled_rows()
    dec = [W.prefill + x for x in STEPS]
    qn, kn, vn = to_np32(q), to_np32(k), to_np32(v)
    got_p, got_d = to_np32(outp[0, rows]), to_np32(outd[STEPS, 0])
    s, wd = W.sink, W.recent
    if leg == "int8":
        ref_p = oracle_q8(qn, kn, vn, mask, s, wd, {0: rows}, [0])[0]
        assert_close(got_p, ref_p, "int8 prefill")
        for i, p in enumerate(dec):
            ref = oracle_q8(qn, kn, vn, mask, s, wd, {0: [p]}, [p])[0]
            assert_close(got_d[i:i + 1], ref, f"int8 decode step {STEPS[i]}")
        check_cache_q8(cache, kn, vn, k, v, mask, done)
    elif leg == "rope":
        ref = oracle_rope(qn, kn, vn, mask, s, wd, {0: rows + dec}, 10000.0, duo.DUO_ROPE_HALF)[0]
        assert_close(got_p, ref[:len(rows)], "rope prefill")
        assert_close(got_d, ref[len(rows):], "rope decode")
        check_cache_rope(cache, k, v, mask, done, 10000.0, duo.DUO_ROPE_HALF)
    elif leg == "paged":
        ref = oracle_rows(qn, kn, vn, mask, s, wd, {0: rows + dec})[0]
        assert_close(got_p, ref[:len(rows)], "paged prefill")
        assert_close(got_d, ref[len(rows):], "paged decode")
        check_cache_bits(cache, k, v, mask, done)
    else:
        ref = oracle_fp8(qn, kn, vn, mask, s, wd, {0: rows + dec}, 1.0, 1.0)[0]
        g = W.num_q_heads // W.num_kv_heads
        retr = [h for h in range(W.num_q_heads) if mask[h // g]]
        strm = [h for h in range(W.num_q_heads) if not mask[h // g]]
        from oracle.fp8_cache import seen_rows_fp8
        vmax = [np.abs(seen_rows_fp8(vn[0, :W.prefill, h // g], True, 1.0)).max() for h in retr]
        worst = assert_fp8_close(got_p[:, retr], ref[:len(rows)][:, retr], vmax, "fp8 prefill")
        _say(f"fp8 prefill worst max|d|/max|V| = {worst[0]:.3e}, relL2 = {worst[1]:.3e}")
        assert_close(got_p[:, strm], ref[:len(rows)][:, strm], "fp8 prefill streaming")
        assert_close(got_d, ref[len(rows):], "fp8 decode")
        check_cache_fp8(cache, kn, vn, k, v, mask, done, 1.0, 1.0)
    del cache, q, k, v, outp, outd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
