"""GPU parity of the benchmark's variant legs at full size: the
llama3_8b_gqa_b8_128k layer (32 query / 8 KV heads, D = 128, 4 retrieval KV
heads, 8 sequences, one-shot 131072-token prefill, 128 decode steps) exactly
as the benchmark launches it, with

  * an int8 retrieval cache (DUO_KV_INT8),
  * rotary position embedding (base 10000, half-split pairs),
  * a paged retrieval cache (1024-position pages, a pool just large enough),
  * an fp8 (e4m3) retrieval cache with unit tensor scales, exact prefill
    (the default) and prefill on the fp8 matrix cores,
  * the dynamic decode split,
  * an int8 retrieval cache with rotary embedding,

the rotary and fp8 legs with the prefill staging workspace (the chunk's K
rows turned, the fp8 rows decoded, once per call), as the benchmark runs
them.

Sequences 0 and 7 are compared at sampled prefill rows and decode steps, in
every query head, with the oracle of each format at the bar its own tests
state; stored rows at sampled positions are read back (codes and scales bit
for bit, bf16 rows bitwise)."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from fp8_model import assert_fp8_mfma_close, mfma_sigma
from oracle.fp8_cache import quantize_rows_fp8, seen_rows_fp8
from oracle.quantized_cache import quantize_rows
from parity_util import assert_close, oracle_rows, require_gpu, run_sequence, staging_workspace, to_np32
from test_gpu_fp8 import oracle_fp8
from test_gpu_int8 import oracle_q8
from test_gpu_rope import oracle_rope
from test_gpu_rope_8bit import oracle as oracle_8bit
from workloads import WORKLOADS, qkv, workload_mask

pytestmark = pytest.mark.gpu

W = WORKLOADS["llama3_8b_gqa_b8_128k"]
SEQS = [0, 7]
STEPS = [0, W.decode_steps - 1]
LEGS = ["int8", "rope", "paged", "fp8", "fp8mfma", "dynamic", "int8rope"]


def _say(msg):
    print(f"[gpu-legs] {msg}", flush=True)


def _sampled_rows():
    s, wd = W.sink, W.recent
    return [0, s - 1, s + wd, 4095, 65535, W.prefill - 1]


def _cache(leg, mask, t):
    kw = {}
    if leg == "int8":
        kw = dict(kv_format=duo.DUO_KV_INT8)
    elif leg == "rope":
        kw = dict(rope_base=10000.0, rope_style=duo.DUO_ROPE_HALF)
    elif leg == "paged":
        kw = dict(page_tokens=1024, num_pages=W.batch * ((t + 1023) // 1024))
    elif leg == "fp8":
        kw = dict(kv_format=duo.DUO_KV_FP8)
    elif leg == "fp8mfma":
        kw = dict(kv_format=duo.DUO_KV_FP8, fp8_prefill=duo.DUO_FP8_PREFILL_MFMA)
    elif leg == "dynamic":
        kw = dict(decode_split=duo.DUO_DECODE_DYNAMIC)
    elif leg == "int8rope":
        kw = dict(kv_format=duo.DUO_KV_INT8, rope_base=10000.0, rope_style=duo.DUO_ROPE_HALF)
    cfg = duo.Config(W.batch, W.num_q_heads, W.num_kv_heads, W.head_dim, t, W.sink, W.recent,
                     [int(x) for x in mask], **kw)
    if leg in ("int8rope", "rope", "fp8"):  # as the benchmark runs these legs
        staging_workspace(cfg)
    buf = torch.full((duo.required_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
    return duo.duo_cache_init(cfg, buf)


def _readback(cache, leg, mask, kn, vn, k, v, positions):
    """Stored retrieval rows of sequences SEQS at `positions`, against the
    inputs (bf16 bitwise) or the oracle's encoding (codes and scales)."""
    views = duo.cache_views(cache)
    hidx = cache.head_index()
    for i, b in enumerate(SEQS):
        for kvh in range(W.num_kv_heads):
            if not mask[kvh]:
                continue
            j = hidx[kvh]
            if leg in ("int8", "int8rope"):
                # (int8rope: V only -- a turned K may sit one code from the
                # oracle's at a rounding tie, which the rotary tests bound)
                for name, x, sname in ((("rk", kn, "rks"),) if leg == "int8" else ()) + (("rv", vn, "rvs"),):
                    codes, scales = quantize_rows(x[i, positions, kvh])
                    assert np.array_equal(views[name][b, j, positions].cpu().numpy(), codes), f"{name} b{b} kv{kvh}"
                    got_s = views[sname][b, j, positions].cpu().numpy()
                    assert np.array_equal(got_s.view(np.uint32), scales.view(np.uint32)), f"{sname} b{b} kv{kvh}"
            elif leg in ("fp8", "fp8mfma"):
                for name, x in (("rk", kn), ("rv", vn)):
                    got = views[name][b, j, positions].cpu().numpy()
                    assert np.array_equal(got, quantize_rows_fp8(x[i, positions, kvh], 1.0)), f"{name} b{b} kv{kvh}"
            elif leg != "rope":
                for name, x in (("rk", k), ("rv", v)):
                    got = views[name][b, j, positions].view(torch.int16).cpu()
                    assert torch.equal(got, x[b, positions, kvh].view(torch.int16).cpu()), f"{name} b{b} kv{kvh}"


@pytest.mark.parametrize("leg", LEGS)
def test_bench_headline_leg(leg):
    require_gpu()
    _say(f"{W.name} {leg}")
    mask = workload_mask(W)
    t = W.prefill + W.decode_steps
    q, k, v = qkv(W.batch, t, W.num_q_heads, W.num_kv_heads, W.head_dim, W.seed * 100, "cuda")
    cache = _cache(leg, mask, t)
    outp, outd, done = run_sequence(cache, q, k, v, [[W.prefill] * W.batch], W.decode_steps)
    assert cache.lengths() == [t] * W.batch
    rows = _sampled_rows()
    dec = [W.prefill + x for x in STEPS]
    sub = lambda x: to_np32(x[SEQS])  # noqa: E731  (host copies of the checked sequences only)
    qn, kn, vn = sub(q), sub(k), sub(v)
    got_p = to_np32(outp[SEQS][:, rows])
    got_d = to_np32(outd[STEPS][:, SEQS]).transpose(1, 0, 2, 3)
    s, wd = W.sink, W.recent
    g = W.group
    retr = [h for h in range(W.num_q_heads) if mask[h // g]]
    strm = [h for h in range(W.num_q_heads) if not mask[h // g]]
    for i, b in enumerate(SEQS):
        if leg == "int8":  # one call: stored rows are the earlier ones, the call's own at input precision
            ref_p = oracle_q8(qn[i:i + 1], kn[i:i + 1], vn[i:i + 1], mask, s, wd, {0: rows}, [0])[0]
            ref_d = np.concatenate([oracle_q8(qn[i:i + 1], kn[i:i + 1], vn[i:i + 1], mask, s, wd, {0: [p]}, [p])[0]
                                    for p in dec])
        elif leg == "int8rope":  # one call: the chunk's own rows at input precision (turned)
            ref_p = oracle_8bit(duo.DUO_KV_INT8, qn[i:i + 1], kn[i:i + 1], vn[i:i + 1], mask, s, wd, {0: rows}, [0],
                                10000.0, duo.DUO_ROPE_HALF)[0]
            ref_d = np.concatenate([oracle_8bit(duo.DUO_KV_INT8, qn[i:i + 1], kn[i:i + 1], vn[i:i + 1], mask, s, wd,
                                                {0: [p]}, [p], 10000.0, duo.DUO_ROPE_HALF)[0] for p in dec])
        elif leg == "rope":
            ref = oracle_rope(qn[i:i + 1], kn[i:i + 1], vn[i:i + 1], mask, s, wd, {0: rows + dec}, 10000.0,
                              duo.DUO_ROPE_HALF)[0]
            ref_p, ref_d = ref[:len(rows)], ref[len(rows):]
        elif leg in ("fp8", "fp8mfma"):
            ref = oracle_fp8(qn[i:i + 1], kn[i:i + 1], vn[i:i + 1], mask, s, wd, {0: rows + dec}, 1.0, 1.0)[0]
            ref_p, ref_d = ref[:len(rows)], ref[len(rows):]
        else:
            ref = oracle_rows(qn[i:i + 1], kn[i:i + 1], vn[i:i + 1], mask, s, wd, {0: rows + dec})[0]
            ref_p, ref_d = ref[:len(rows)], ref[len(rows):]
        if leg == "fp8mfma":
            scale = 1.0 / math.sqrt(W.head_dim)
            sig = np.empty((len(rows), len(retr), W.head_dim))
            for j, h in enumerate(retr):
                kvh = h // g
                ks = seen_rows_fp8(kn[i, :, kvh], True, 1.0)
                vs = seen_rows_fp8(vn[i, :, kvh], True, 1.0)
                sig[:, j] = mfma_sigma(qn[i, rows, h], rows, ks, vs, True, s, wd, scale)
            w = assert_fp8_mfma_close(got_p[i][:, retr], ref_p[:, retr], sig, f"{leg} prefill b{b}")
            _say(f"fp8 mfma b{b}: |d|_2/predicted = {w[0]:.3f}, max |d|/sigma = {w[1]:.2f}")
            assert_close(got_p[i][:, strm], ref_p[:, strm], f"{leg} prefill streaming b{b}")
        else:
            assert_close(got_p[i], ref_p, f"{leg} prefill b{b}")
        assert_close(got_d[i], ref_d, f"{leg} decode b{b}")
    _readback(cache, leg, mask, kn, vn, k, v, [0, 1, 4095, 65535, t - 1])
    del cache, q, k, v, outp, outd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
