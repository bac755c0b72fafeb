"""Helpers shared by the GPU parity tests: run the HIP path through the C
ABI, evaluate the oracle on the same bf16 inputs, compare.

Tolerance (the bar stated for this path): per (sequence, query head) slice,
max |gpu - ref| <= 2e-2 AND ||gpu - ref||_2 / ||ref||_2 <= 1e-2, where ref is
the fp64 oracle on the bf16 inputs the GPU saw.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import kv_cache_duo_amd as duo
from oracle import attend_rows, streaming_slot_positions

MAX_ABS = 2e-2
REL_L2 = 1e-2


def require_gpu():
    assert torch.cuda.is_available(), "GPU test needs a visible MI355X"
    duo.load_library()


def new_cache(batch, hq, hkv, d, max_len, sink, recent, mask, poison=True):
    cfg = duo.Config(batch, hq, hkv, d, max_len, sink, recent, [int(x) for x in mask])
    nbytes = duo.required_bytes(cfg)
    fill = 0xFF if poison else 0  # 0xFFFF bf16 = NaN: catches reads of unwritten slots
    buf = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
    return duo.duo_cache_init(cfg, buf)


def staging_workspace(cfg, nbytes=None):
    """Attach a prefill staging workspace to cfg (all of
    prefill_staging_bytes(cfg) by default), filled with 0xFF bytes: a staged row
    read before it is written would be a bf16 NaN and poison the output."""
    n = duo.prefill_staging_bytes(cfg) if nbytes is None else nbytes
    cfg.prefill_staging = torch.full((max(n, 16),), 0xFF, dtype=torch.uint8, device="cuda")[:n] if n else None
    return cfg


def to_np32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def oracle_rows(q, k, v, mask, sink, recent, rows_by_b, scale=None):
    """fp64 oracle for selected positions.  q [B,T,Hq,D], k/v [B,T,Hkv,D]
    (numpy, any float dtype); rows_by_b[b] = positions.  Returns
    {b: [len(rows), Hq, D]} float64."""
    b_n, _t, hq, d = q.shape
    hkv = k.shape[2]
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = {}
    for b in range(b_n):
        rows = np.asarray(rows_by_b[b], dtype=np.int64)
        if len(rows) == 0:
            continue
        tmax = int(rows.max()) + 1
        res = np.empty((len(rows), hq, d))
        for kvh in range(hkv):
            ks = np.ascontiguousarray(k[b, :tmax, kvh, :], dtype=np.float64)
            vs = np.ascontiguousarray(v[b, :tmax, kvh, :], dtype=np.float64)
            for h in range(kvh * g, (kvh + 1) * g):
                res[:, h, :] = attend_rows(q[b, rows, h, :], rows, ks, vs, bool(mask[kvh]), sink, recent, scale)
        out[b] = res
    return out


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    """got/ref [..., H, D]: compare per head slice over all leading rows."""
    got = got.astype(np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    h = got.shape[-2]
    g2 = got.reshape(-1, h, got.shape[-1])
    r2 = ref.reshape(-1, h, ref.shape[-1])
    for hh in range(h):
        diff = g2[:, hh] - r2[:, hh]
        mx = np.abs(diff).max()
        rel = np.linalg.norm(diff) / max(np.linalg.norm(r2[:, hh]), 1e-30)
        assert mx <= MAX_ABS and rel <= REL_L2, f"{what} head {hh}: max|d|={mx:.3e} relL2={rel:.3e}"


def check_cache_bits(cache, k_all, v_all, mask, n_tokens):
    """Bit-exact readback: retrieval rows hold positions 0..n-1; streaming slot
    s holds the position the oracle's closed-form slot map assigns to it.
    k_all/v_all: torch bf16 [B,T,Hkv,D] on any device; n_tokens[b]."""
    views = duo.cache_views(cache)
    cfg = cache.cfg
    hidx = cache.head_index()
    assert views["lengths"].cpu().tolist() == list(n_tokens)
    assert cache.lengths() == list(n_tokens)
    kb = k_all.view(torch.int16).cpu()
    vb = v_all.view(torch.int16).cpu()
    rk, rv = views["rk"].view(torch.int16).cpu(), views["rv"].view(torch.int16).cpu()
    sk, sv = views["sk"].view(torch.int16).cpu(), views["sv"].view(torch.int16).cpu()
    for b in range(cfg.batch):
        n = n_tokens[b]
        slots = streaming_slot_positions(n, cfg.sink, cfg.recent)
        for kvh in range(cfg.num_kv_heads):
            i = hidx[kvh]
            if mask[kvh]:
                assert torch.equal(rk[b, i, :n], kb[b, :n, kvh]), f"rk b{b} kv{kvh}"
                assert torch.equal(rv[b, i, :n], vb[b, :n, kvh]), f"rv b{b} kv{kvh}"
            else:
                for s, p in enumerate(slots):
                    if p >= 0:
                        assert torch.equal(sk[b, i, s], kb[b, p, kvh]), f"sk b{b} kv{kvh} slot{s}"
                        assert torch.equal(sv[b, i, s], vb[b, p, kvh]), f"sv b{b} kv{kvh} slot{s}"


def run_sequence(cache, q, k, v, chunks, decode_steps, out_fill=0.0):
    """Prefill in the given chunk plan, then decode.

    q [B,T,Hq,D], k/v [B,T,Hkv,D] bf16 on cuda holding every token (prefill
    tokens first, then one per decode step).  chunks: list of per-call n_new
    lists; each call's chunk length C = max(n_new).  Returns (prefill out
    [B,T,Hq,D] with untouched rows = out_fill, decode out [steps,B,Hq,D])."""
    cfg = cache.cfg
    b_n = cfg.batch
    outp = torch.full_like(q, out_fill)
    done = [0] * b_n
    for n_new in chunks:
        c = max(max(n_new), 1)
        qc = torch.zeros(b_n, c, cfg.num_q_heads, cfg.head_dim, dtype=torch.bfloat16, device="cuda")
        kc = torch.zeros(b_n, c, cfg.num_kv_heads, cfg.head_dim, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        oc = torch.full_like(qc, out_fill)
        for b in range(b_n):
            n = n_new[b]
            qc[b, :n] = q[b, done[b]:done[b] + n]
            kc[b, :n] = k[b, done[b]:done[b] + n]
            vc[b, :n] = v[b, done[b]:done[b] + n]
        duo.duo_prefill(cache, qc, kc, vc, n_new, oc)
        for b in range(b_n):
            outp[b, done[b]:done[b] + n_new[b]] = oc[b, :n_new[b]]
            # rows past n_new must be untouched
            if n_new[b] < c:
                assert torch.all(oc[b, n_new[b]:] == out_fill), "prefill wrote rows past n_new"
            done[b] += n_new[b]
    outd = []
    for s in range(decode_steps):
        pos = done
        q1 = torch.stack([q[b, pos[b]] for b in range(b_n)]).contiguous()
        k1 = torch.stack([k[b, pos[b]] for b in range(b_n)]).contiguous()
        v1 = torch.stack([v[b, pos[b]] for b in range(b_n)]).contiguous()
        o1 = torch.empty_like(q1)
        duo.duo_decode(cache, q1, k1, v1, o1)
        outd.append(o1)
        done = [p + 1 for p in pos]
    torch.cuda.synchronize()
    return outp, (torch.stack(outd) if outd else None), done


def poison_decode_records(cache):
    """Fill the cache's decode split records with NaN bytes (0xFF): a decode
    call that read a record before writing it in the same call would produce
    a non-finite output."""
    lay = cache.layout()
    cache.buf[lay.work_records_offset:lay.work_offset + lay.work_bytes].fill_(0xFF)


def decode_steps_poisoned(cache, q, k, v, start, steps):
    """`steps` decode calls of tokens start[b] + s of q/k/v [B,T,H,D] (bf16,
    cuda), with the split records poisoned before each call.  Returns
    [steps, B, Hq, D]."""
    b_n = cache.cfg.batch
    outs = []
    for s in range(steps):
        q1 = torch.stack([q[b, start[b] + s] for b in range(b_n)]).contiguous()
        k1 = torch.stack([k[b, start[b] + s] for b in range(b_n)]).contiguous()
        v1 = torch.stack([v[b, start[b] + s] for b in range(b_n)]).contiguous()
        o1 = torch.empty_like(q1)
        poison_decode_records(cache)
        duo.duo_decode(cache, q1, k1, v1, o1)
        outs.append(o1)
    torch.cuda.synchronize()
    return torch.stack(outs)
