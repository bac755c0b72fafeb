"""GPU parity at the full sizes of the GQA and mixed-length workloads, on
sampled outputs the fp64 oracle computes one by one.

Only the rows the oracle needs are copied to the host; K/V of one
(sequence, KV head) at a time are converted to fp64.  The oracle never reads
the GPU cache: every input is the seeded tensor the GPU was given (or is
regenerated from its seed).
"""

import math

import numpy as np
import pytest
import torch

import kv_cache_duo_amd as duo
from oracle import attend_rows, seen_rows, streaming_slot_positions
from parity_util import assert_close, new_cache, require_gpu, staging_workspace
from workloads import WORKLOADS, randn_bf16, sequence_lengths, workload_mask

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-full] {msg}", flush=True)


def _kv64(k_seq, v_seq):
    """fp64 host copies of one KV head's keys/values [T, D] (torch, any device)."""
    return (k_seq.float().cpu().numpy().astype(np.float64), v_seq.float().cpu().numpy().astype(np.float64))


def _oracle(qrows, kv, pos, retrieval, w):
    """qrows: torch [R, D] of one query head; kv: its KV head from _kv64;
    pos: [R] positions."""
    scale = 1.0 / math.sqrt(w.head_dim)
    return attend_rows(qrows.float().cpu().numpy(), pos, kv[0], kv[1], retrieval, w.sink, w.recent, scale)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_llama3_gqa_batch8_128k():
    """B=8 x 131072 context, 32/8 heads, 4 of 8 KV heads retrieval; one-shot
    prefill then 128 decode steps; sampled rows of every query head."""
    require_gpu()
    w = WORKLOADS["llama3_8b_gqa_b8_128k"]
    _say(w.name)
    mask = workload_mask(w)
    dev = torch.device("cuda", 0)
    t_all = w.prefill + w.decode_steps
    q = randn_bf16((w.batch, t_all, w.num_q_heads, w.head_dim), 3 * w.seed + 1, dev)
    k = randn_bf16((w.batch, t_all, w.num_kv_heads, w.head_dim), 3 * w.seed + 2, dev)
    v = randn_bf16((w.batch, t_all, w.num_kv_heads, w.head_dim), 3 * w.seed + 3, dev)
    cache = new_cache(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, t_all, w.sink, w.recent, mask,
                      poison=False)
    outp = torch.empty(w.batch, w.prefill, w.num_q_heads, w.head_dim, dtype=torch.bfloat16, device=dev)
    duo.duo_prefill(cache, q[:, :w.prefill].contiguous(), k[:, :w.prefill].contiguous(),
                    v[:, :w.prefill].contiguous(), [w.prefill] * w.batch, outp)
    steps = [0, 63, 127]
    outd = {}
    for s in range(w.decode_steps):
        p = w.prefill + s
        o = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.bfloat16, device=dev)
        duo.duo_decode(cache, q[:, p].contiguous(), k[:, p].contiguous(), v[:, p].contiguous(), o)
        if s in steps:
            outd[s] = o
    torch.cuda.synchronize()
    assert cache.lengths() == [t_all] * w.batch
    rng = np.random.default_rng(3)
    rows = sorted(set([0, w.sink - 1, w.sink + w.recent, 65535, w.prefill - 1] +
                      rng.integers(0, w.prefill, 3).tolist()))
    g = w.group
    for b in [0, 3, 7]:
        for kvh in range(w.num_kv_heads):
            retrieval = bool(mask[kvh])
            pos = rows + [w.prefill + s for s in steps]
            kv = _kv64(k[b, :, kvh], v[b, :, kvh])
            for h in range(kvh * g, (kvh + 1) * g):
                ref = _oracle(q[b, pos, h], kv, pos, retrieval, w)
                got = torch.cat([outp[b, rows, h], torch.stack([outd[s][b, h] for s in steps])])
                assert_close(got.float().cpu().numpy()[:, None, :], ref[:, None, :], f"gqa b{b} h{h}")
    del q, k, v, outp, cache, outd
    _free()


@pytest.mark.parametrize("n_retrieval,fmt", [(2, "bf16"), (4, "bf16"), (6, "bf16"), (4, "int8_staged")])
def test_mixed_gqa_batch32_chunked(n_retrieval, fmt):
    """32 sequences of lengths U[4096, 65536], chunked prefill in 4096-token
    calls (finished sequences pass 0), then 64 decode steps; retrieval ratio
    25/50/75%, and at 50% over an int8 retrieval cache with the prefill
    staging workspace (as the benchmark's int8 leg of this workload runs it:
    every call after the first attends a stored int8 prefix, decoded once per
    call).  Four sequences (shortest, longest, two others) are checked; for
    int8 against the oracle's view of each call (rows stored by earlier
    calls through their codes, the call's own rows as given)."""
    require_gpu()
    w = WORKLOADS["mixed_gqa_b32"]
    _say(f"{w.name} nR={n_retrieval} {fmt}")
    from workloads import retrieval_mask
    mask = retrieval_mask(w.num_kv_heads, n_retrieval, w.seed + n_retrieval)
    dev = torch.device("cuda", 0)
    lens = sequence_lengths(w.batch, w.length_range[0], w.length_range[1], w.seed)
    order = np.argsort(lens)
    check = sorted({int(order[0]), int(order[-1]), int(order[5]), int(order[20])})
    max_len = int(lens.max()) + w.decode_steps
    int8 = fmt == "int8_staged"
    if int8:
        cfg = duo.Config(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, max_len, w.sink, w.recent,
                         [int(x) for x in mask], kv_format=duo.DUO_KV_INT8)
        staging_workspace(cfg)
        cache = duo.duo_cache_init(cfg, torch.empty(duo.required_bytes(cfg), dtype=torch.uint8, device=dev))
    else:
        cache = new_cache(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, max_len, w.sink, w.recent, mask,
                          poison=False)
    hq, hkv, d, c = w.num_q_heads, w.num_kv_heads, w.head_dim, w.chunk
    # host copies (bf16) of the checked sequences' tokens, and of outputs at sampled rows
    seq_q = {b: [] for b in check}
    seq_k = {b: [] for b in check}
    seq_v = {b: [] for b in check}
    seq_o = {b: [] for b in check}
    done = np.zeros(w.batch, dtype=np.int64)
    call = 0
    while (done < lens).any():
        n_new = [int(min(c, lens[b] - done[b])) for b in range(w.batch)]
        seed = 1000 * (w.seed + n_retrieval) + call
        q = randn_bf16((w.batch, c, hq, d), 3 * seed + 1, dev)
        k = randn_bf16((w.batch, c, hkv, d), 3 * seed + 2, dev)
        v = randn_bf16((w.batch, c, hkv, d), 3 * seed + 3, dev)
        out = torch.zeros_like(q)
        duo.duo_prefill(cache, q, k, v, n_new, out)
        for b in check:
            n = n_new[b]
            if n:
                seq_q[b].append(q[b, :n].cpu())
                seq_k[b].append(k[b, :n].cpu())
                seq_v[b].append(v[b, :n].cpu())
                seq_o[b].append(out[b, :n].cpu())
        done += np.array(n_new)
        call += 1
    for s in range(w.decode_steps):
        seed = 1000 * (w.seed + n_retrieval) + 500 + s
        q = randn_bf16((w.batch, hq, d), 3 * seed + 1, dev)
        k = randn_bf16((w.batch, hkv, d), 3 * seed + 2, dev)
        v = randn_bf16((w.batch, hkv, d), 3 * seed + 3, dev)
        o = torch.empty_like(q)
        duo.duo_decode(cache, q, k, v, o)
        for b in check:
            seq_q[b].append(q[b][None].cpu())
            seq_k[b].append(k[b][None].cpu())
            seq_v[b].append(v[b][None].cpu())
            seq_o[b].append(o[b][None].cpu())
    torch.cuda.synchronize()
    assert cache.lengths() == [int(x) + w.decode_steps for x in lens]
    g = w.group
    rng = np.random.default_rng(n_retrieval)
    for b in check:
        qs, ks, vs, os_ = (torch.cat(x) for x in (seq_q[b], seq_k[b], seq_v[b], seq_o[b]))
        n = int(lens[b])
        pos = sorted(set([0, c - 1, c, n - 1, n, n + w.decode_steps - 1] +
                         rng.integers(0, n, 3).tolist()))
        for kvh in range(hkv):
            kv = _kv64(ks[:, kvh], vs[:, kvh])
            for h in range(kvh * g, (kvh + 1) * g):
                if not int8:
                    ref = _oracle(qs[pos, h], kv, pos, bool(mask[kvh]), w)
                else:  # rows grouped by the call that computed them: stored rows before it
                    ref = np.empty((len(pos), w.head_dim))
                    before = [(p // c) * c if p < n else p for p in pos]
                    for sb in sorted(set(before)):
                        idx = [i for i, x in enumerate(before) if x == sb]
                        seen = (seen_rows(kv[0], bool(mask[kvh]), sb), seen_rows(kv[1], bool(mask[kvh]), sb))
                        ref[idx] = _oracle(qs[[pos[i] for i in idx], h], seen, [pos[i] for i in idx],
                                           bool(mask[kvh]), w)
                assert_close(os_[pos, h].float().numpy()[:, None, :], ref[:, None, :],
                             f"mixed nR={n_retrieval} {fmt} b{b} h{h}")
    del cache
    _free()


def test_llama3_gqa_stack_1m_decode():
    """32 layers of the GQA layer at 1,048,576 tokens (B=1), caches filled by
    duo_cache_append in 65536-token chunks, then 64 decode steps through all
    layers.  Layers 0 and 31 are checked at steps 0 and 63, every query head,
    with the K/V regenerated from their seeds for the oracle; streaming slots
    of those layers are read back bit-exactly against the regenerated rows."""
    require_gpu()
    w = WORKLOADS["llama3_8b_gqa_stack_1m"]
    _say(w.name)
    dev = torch.device("cuda", 0)
    n_ctx, steps, ck = w.prefill, w.decode_steps, 65536
    hq, hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    t_all = n_ctx + steps

    def kv_chunk(layer, i):
        s = 100000 * (layer + 1) + i
        return (randn_bf16((1, ck, hkv, d), 2 * s, dev), randn_bf16((1, ck, hkv, d), 2 * s + 1, dev))

    def dec_inputs(layer, s):
        z = 100000 * (layer + 1) + 50000 + s
        return (randn_bf16((1, hq, d), 3 * z, dev), randn_bf16((1, hkv, d), 3 * z + 1, dev),
                randn_bf16((1, hkv, d), 3 * z + 2, dev))

    caches, masks = [], []
    for layer in range(w.layers):
        mask = workload_mask(w, layer)
        masks.append(mask)
        cache = new_cache(1, hq, hkv, d, t_all, w.sink, w.recent, mask, poison=False)
        for i in range(n_ctx // ck):
            kc, vc = kv_chunk(layer, i)
            duo.duo_cache_append(cache, kc, vc, [ck])
        caches.append(cache)
        if layer % 8 == 7:
            _say(f"filled {layer + 1} layers")
    check_steps = [0, steps - 1]
    outs = {}
    for s in range(steps):
        for layer in range(w.layers):
            qd, kd, vd = dec_inputs(layer, s)
            o = torch.empty_like(qd)
            duo.duo_decode(caches[layer], qd, kd, vd, o)
            if layer in (0, w.layers - 1) and s in check_steps:
                outs[(layer, s)] = o
    torch.cuda.synchronize()
    g = w.group
    for layer in (0, w.layers - 1):
        mask = masks[layer]
        assert caches[layer].lengths() == [t_all]
        # regenerate this layer's K/V (bf16, host) for the oracle
        kh = torch.empty(t_all, hkv, d, dtype=torch.bfloat16)
        vh = torch.empty(t_all, hkv, d, dtype=torch.bfloat16)
        for i in range(n_ctx // ck):
            kc, vc = kv_chunk(layer, i)
            kh[i * ck:(i + 1) * ck] = kc[0].cpu()
            vh[i * ck:(i + 1) * ck] = vc[0].cpu()
        qsteps = {}
        for s in range(steps):
            qd, kd, vd = dec_inputs(layer, s)
            kh[n_ctx + s] = kd[0].cpu()
            vh[n_ctx + s] = vd[0].cpu()
            if s in check_steps:
                qsteps[s] = qd[0].cpu()
        views = duo.cache_views(caches[layer])
        hidx = caches[layer].head_index()
        slots = streaming_slot_positions(t_all, w.sink, w.recent)
        sk = views["sk"].view(torch.int16).cpu()
        for kvh in range(hkv):
            if not mask[kvh]:
                assert torch.equal(sk[0, hidx[kvh]], kh[torch.from_numpy(slots), kvh].view(torch.int16))
            pos = [n_ctx + s for s in check_steps]
            kv = _kv64(kh[:, kvh], vh[:, kvh])
            for h in range(kvh * g, (kvh + 1) * g):
                qrows = torch.stack([qsteps[s][h] for s in check_steps])
                ref = _oracle(qrows, kv, pos, bool(mask[kvh]), w)
                got = torch.stack([outs[(layer, s)][0, h].cpu() for s in check_steps])
                assert_close(got.float().numpy()[:, None, :], ref[:, None, :], f"stack L{layer} h{h}")
        _say(f"layer {layer} checked")
    del caches, outs
    _free()
