"""Benchmark of the DuoAttention hot path on one MI355X.

Headline step (`--workload`, default the Llama-3-8B-shaped GQA batch: 32
query / 8 KV heads, D = 128, 4 of 8 KV heads retrieval, 8 sequences of
131072 tokens, 128 decode steps, 64 sink + 256 recent):
    cache init -> one-shot prefill of every sequence -> `decode_steps`
    decode calls.
Inputs are resident in HBM before the timed region.  Reported:
  value      decode attention: algorithmic HBM bytes / decode-phase time
  prefill    algorithmic flops / prefill-phase time
  roofline   decode kernel: algorithmic bytes per launch / mean launch time
             (one decode call is one launch; HIP events on the launch
             stream around the decode phase), against 8 TB/s
  roofline_prefill  the prefill call (prefill kernel + append kernel)
  full_attention    the same step with every KV head a retrieval head (the
             method's full-attention reference on the same kernels): times,
             cache bytes and the Duo/full ratios
Legs (--legs, each with its own fixed repetitions):
  mha32k     the Llama-2-7B-shaped MHA layer (32 heads, 8 retrieval, 32768
             prefill, 256 decode) rotated over 8 layer caches, and its
             full-attention reference
  stack1m    32 GQA layers at 1,048,576 tokens, caches filled by
             duo_cache_append outside the timed region, 64 decode steps
             through every layer; full attention on 4 of the layers
  mixed      32 sequences of lengths U[4096, 65536], chunked prefill in
             4096-token calls then 64 decode steps, 2/4/6 of 8 KV heads
             retrieval and the full-attention reference (8 of 8)
             (and, at 4 of 8, over an int8 retrieval cache: prefill over the
             stored int8 prefix decoded per tile or staged once per call)
  int8, int8rope, fp8, fp8mfma, rope, paged, dynamic
             the headline step over an int8 / fp8 retrieval cache (int8rope:
             int8 with rotary embedding; fp8mfma: retrieval prefill on fp8
             matrix cores), with rotary embedding, over a paged cache, and
             with the dynamic decode split; the rotary and fp8 legs run
             with the prefill staging workspace and once without it (tiled)
  cpu_baseline  the fp64 oracle on a bounded sample of the headline
             workload (decode and prefill rows), with all host cores and
             with one, and the full workload's oracle time extrapolated
Algorithmic counts: each K/V byte once per (sequence, KV head) plus q, out
and the appended token; flops = 4*D per allowed (query, key) pair per query
head.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_traffic.json")
ALL_LEGS = "mha32k,stack1m,mixed,int8,int8rope,fp8,fp8mfma,rope,paged,dynamic"


def say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(path: str) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode launch of `workload` from the committed rocprofv3
    counter record, or None when the kernel source changed since."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    src = os.path.join(ROOT, "kv_cache_duo_amd", "csrc", "decode.hip")
    ent = rec.get("workloads", {}).get(workload)
    if not ent or ent.get("decode_hip_sha256_16") != source_digest(src):
        return None
    return ent.get("bytes_per_launch")


def measured_ceilings(decode_mib: int, extra_mib=()):
    """Streaming-read (launches of the decode call's size -- and of each
    size in extra_mib -- over 8 buffers in turn, and 4 GiB) and MFMA-loop
    ceilings from kv_cache_duo_amd/ceiling, run as a child process."""
    import subprocess
    exe = os.path.join(ROOT, "kv_cache_duo_amd", "ceiling")
    out = {}
    sizes = [decode_mib] + [m for m in extra_mib if m != decode_mib]
    for args in ([["stream_read_rotating", str(m), "8"] for m in sizes] +
                 [["stream_read", "4096"], ["mfma"], ["mfma_random"], ["mfma_fp8_random"], ["lds_read"]]):
        r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=120)
        if r.returncode != 0:
            raise RuntimeError(f"{exe} {' '.join(args)} failed: {r.stderr}")
        rec = json.loads(r.stdout.strip().splitlines()[-1])
        key = rec["ceiling"] + ("_%dMiB" % rec["mib"] if "mib" in rec else "")
        out[key] = {k: v for k, v in rec.items() if k != "ceiling"}
    return out


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--workload", default="llama3_8b_gqa_b8_128k")
    p.add_argument("--layers", type=int, default=0,
                   help="layer caches rotated in the headline step (0: 1, or 8 for a cache under 1 GB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceilings", action="store_true")
    p.add_argument("--no-full", action="store_true", help="skip the full-attention reference of the headline")
    p.add_argument("--legs", default=ALL_LEGS, help=f"comma list of {ALL_LEGS} (empty for none)")
    return p.parse_args()


# ---- algorithmic counts -------------------------------------------------

def allowed(t: int, retrieval: bool, sink: int, recent: int) -> int:
    """Keys a query at position t attends to."""
    return t + 1 if retrieval else min(t + 1, sink + recent)


def sum_allowed(lo: int, hi: int, retrieval: bool, sink: int, recent: int) -> int:
    """Sum of allowed(t) for t in [lo, hi)."""
    if hi <= lo:
        return 0
    if retrieval:
        return (hi * (hi + 1) - lo * (lo + 1)) // 2
    cap = sink + recent
    a = min(hi, cap)
    below = (a * (a + 1) - lo * (lo + 1)) // 2 if lo < a else 0
    return below + max(hi - max(lo, cap), 0) * cap


def prefill_flops(w, mask, spans) -> float:
    """4*D per allowed pair per query head over the query positions
    [lo, hi) of every sequence (spans: list of (lo, hi))."""
    g = w.group
    tot = 0
    for kv in mask:
        for lo, hi in spans:
            tot += sum_allowed(lo, hi, bool(kv), w.sink, w.recent)
    return 4.0 * w.head_dim * g * tot


def decode_bytes(w, mask, ctxs, row_r=None) -> float:
    """Algorithmic bytes of one decode call when sequence b holds ctxs[b]
    tokens.  row_r: bytes of a stored retrieval K or V row (default bf16; the
    new retrieval token is read as bf16 and stored as row_r bytes)."""
    row = 2 * w.head_dim
    row_r = row if row_r is None else row_r
    nr = int(sum(mask))
    ns = w.num_kv_heads - nr
    tot = 0
    for c in ctxs:
        tot += 2 * (nr * (c * row_r + row + row_r) + ns * row * min(c + 1, w.sink + w.recent) + ns * row)
        tot += 2 * row * w.num_q_heads
    return float(tot)


def int8_row(w):
    return w.head_dim + 4


def fp8_row(w):
    return w.head_dim


# ---- running the path ---------------------------------------------------

class Runner:
    def __init__(self, torch, duo, lib, dev, stream):
        self.torch, self.duo, self.lib, self.dev, self.stream = torch, duo, lib, dev, stream
        self.sp = ctypes.c_void_p(stream.cuda_stream)

    @staticmethod
    def ptr(t):
        return ctypes.c_void_p(t.data_ptr())

    def check(self, st, where):
        if st != 0:
            raise RuntimeError(f"{where}: {self.duo.status_string(st)}")

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def buffers(self, cfgs, old=None):
        """Device buffers for caches of cfgs (reusing `old` where large enough)."""
        out = []
        for i, c in enumerate(cfgs):
            need = self.duo.required_bytes(c)
            if old is not None and i < len(old) and old[i].numel() >= need:
                out.append(old[i])
            else:
                out.append(self.torch.empty(need, dtype=self.torch.uint8, device=self.dev))
        return out


def layer_inputs(torch, w, nl, dev):
    """Per layer l: prefill q/k/v [B, prefill, H, D] and decode q/k/v per step
    [B, H, D], all contiguous; seeded as the full-size parity tests seed them
    (qkv over prefill + decode tokens, seed w.seed * 100 + l)."""
    from workloads import qkv
    t_all = w.prefill + w.decode_steps
    ins = []
    for layer in range(nl):
        q, k, v = qkv(w.batch, t_all, w.num_q_heads, w.num_kv_heads, w.head_dim, w.seed * 100 + layer, dev)
        pre = tuple(x[:, :w.prefill].contiguous() for x in (q, k, v))
        dec = [tuple(x[:, w.prefill + s].contiguous() for x in (q, k, v)) for s in range(w.decode_steps)]
        ins.append((pre, dec))
        del q, k, v
    return ins


def time_layer_step(R, w, cfgs, bufs, ins, reps, warmup):
    """`warmup` untimed then `reps` timed repetitions of: init every layer's
    cache, one-shot prefill of each layer, decode steps visiting every layer.
    Returns (prefill ms, decode ms) summed over the timed repetitions, and
    the total timed wall ms between the first and last event."""
    torch, lib = R.torch, R.lib
    nl = len(cfgs)
    n_new = (ctypes.c_int32 * w.batch)(*([w.prefill] * w.batch))
    outp = torch.empty(w.batch, w.prefill, w.num_q_heads, w.head_dim, dtype=torch.bfloat16, device=R.dev)
    outd = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.bfloat16, device=R.dev)
    op, od = R.ptr(outp), R.ptr(outd)
    pre_p = [tuple(R.ptr(x) for x in ins[l][0]) for l in range(nl)]
    dec_p = [[tuple(R.ptr(x) for x in st) for st in ins[l][1]] for l in range(nl)]
    ev = [R.event() for _ in range(3)]
    t0, t1 = R.event(), R.event()
    pre_ms = dec_ms = 0.0
    for it in range(warmup + reps):
        if it == warmup:
            torch.cuda.synchronize()
            t0.record(R.stream)
        caches = [R.duo.duo_cache_init(cfgs[l], bufs[l]) for l in range(nl)]
        hs = [c.handle for c in caches]
        ev[0].record(R.stream)
        for l in range(nl):
            R.check(lib.duo_prefill(hs[l], *pre_p[l], n_new, w.prefill, op, R.sp), "prefill")
        ev[1].record(R.stream)
        for s in range(w.decode_steps):
            for l in range(nl):
                R.check(lib.duo_decode(hs[l], *dec_p[l][s], od, R.sp), "decode")
        ev[2].record(R.stream)
        torch.cuda.synchronize()
        if it >= warmup:
            pre_ms += ev[0].elapsed_time(ev[1])
            dec_ms += ev[1].elapsed_time(ev[2])
        del caches
    t1.record(R.stream)
    torch.cuda.synchronize()
    return pre_ms, dec_ms, t0.elapsed_time(t1)


def layer_counts(w, masks, row_r=None):
    flops = sum(prefill_flops(w, m, [(0, w.prefill)] * w.batch) for m in masks)
    byts = sum(decode_bytes(w, m, [w.prefill + s] * w.batch, row_r) for m in masks for s in range(w.decode_steps))
    return flops, byts


def summarize(w, masks, pre_ms, dec_ms, reps, row_r=None, mfma_peak=BF16_MFMA_PEAK_TFLOPS):
    nl = len(masks)
    flops, byts = layer_counts(w, masks, row_r)
    n_dec = w.decode_steps * nl
    dec_call_ms = dec_ms / (reps * n_dec)
    pre_call_ms = pre_ms / (reps * nl)
    gbs = byts * reps / (dec_ms * 1e-3) / 1e9
    tfl = flops * reps / (pre_ms * 1e-3) / 1e12
    return {
        "decode_gbs": round(gbs, 1), "decode_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "decode_us_per_call": round(dec_call_ms * 1e3, 3), "decode_bytes_per_call": byts / n_dec,
        "prefill_tflops": round(tfl, 1), "prefill_frac_of_mfma_peak": round(tfl / mfma_peak, 4),
        "prefill_ms_per_call": round(pre_call_ms, 4), "prefill_flops_per_call": flops / nl,
    }


def full_mask(w):
    return [1] * w.num_kv_heads


def make_cfgs(duo, w, masks, t_all, **kw):
    return [duo.Config(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, t_all, w.sink, w.recent,
                       [int(x) for x in m], **kw) for m in masks]


def ratio(a, b):
    return round(a / b, 4) if b else None


# ---- legs ---------------------------------------------------------------

def leg_layer(R, w, nl, reps, warmup, full: bool):
    """A single-layer workload rotated over nl layer caches, and (full) its
    full-attention reference."""
    from workloads import workload_mask
    masks = [workload_mask(w, l) for l in range(nl)]
    t_all = w.prefill + w.decode_steps
    ins = layer_inputs(R.torch, w, nl, R.dev)
    cfgs = make_cfgs(R.duo, w, masks, t_all)
    bufs = R.buffers(cfgs)
    pre, dec, _ = time_layer_step(R, w, cfgs, bufs, ins, reps, warmup)
    out = {"workload": w.name, "layers_rotated": nl, "reps": reps, **summarize(w, masks, pre, dec, reps),
           "cache_bytes_per_layer": R.duo.required_bytes(cfgs[0])}
    if full:
        fm = [full_mask(w)] * nl
        cfgf = make_cfgs(R.duo, w, fm, t_all)
        del bufs
        bufs = R.buffers(cfgf)
        pre_f, dec_f, _ = time_layer_step(R, w, cfgf, bufs, ins, reps, warmup)
        s = summarize(w, fm, pre_f, dec_f, reps)
        out["full_attention"] = {
            **s, "cache_bytes_per_layer": R.duo.required_bytes(cfgf[0]),
            "decode_speedup": ratio(dec_f, dec), "prefill_speedup": ratio(pre_f, pre),
            "memory_reduction": ratio(R.duo.required_bytes(cfgf[0]), out["cache_bytes_per_layer"])}
    del bufs, ins
    R.torch.cuda.synchronize()
    R.torch.cuda.empty_cache()
    return out


def leg_stack(R, reps_full_layers=4):
    """32 GQA layers at 1,048,576 tokens: fill by append (untimed), then 64
    decode steps through every layer, timed; full attention on the first
    reps_full_layers layers (the same decode, every KV head retrieval)."""
    from workloads import WORKLOADS, randn_bf16, workload_mask
    torch, duo, lib = R.torch, R.duo, R.lib
    w = WORKLOADS["llama3_8b_gqa_stack_1m"]
    n_ctx, steps, ck = w.prefill, w.decode_steps, 65536
    hq, hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    warm = 2
    t_all = n_ctx + steps + warm

    def kv_chunk(layer, i):  # the full-size parity test's seeds
        s = 100000 * (layer + 1) + i
        return (randn_bf16((1, ck, hkv, d), 2 * s, R.dev), randn_bf16((1, ck, hkv, d), 2 * s + 1, R.dev))

    def run(layers, masks):
        cfgs = [duo.Config(1, hq, hkv, d, t_all, w.sink, w.recent, [int(x) for x in m]) for m in masks]
        bufs = [torch.empty(duo.required_bytes(c), dtype=torch.uint8, device=R.dev) for c in cfgs]
        caches = [duo.duo_cache_init(c, b) for c, b in zip(cfgs, bufs)]
        n1 = (ctypes.c_int32 * 1)(ck)
        for li, layer in enumerate(layers):
            for i in range(n_ctx // ck):
                kc, vc = kv_chunk(layer, i)
                R.check(lib.duo_cache_append(caches[li].handle, R.ptr(kc), R.ptr(vc), n1, ck, R.sp), "append")
            if li % 8 == 7:
                say(f"stack: filled {li + 1} layers")
        dq = [randn_bf16((steps + warm, 1, hq, d), 7 * (layer + 1), R.dev) for layer in layers]
        dk = [randn_bf16((steps + warm, 1, hkv, d), 7 * (layer + 1) + 1, R.dev) for layer in layers]
        dv = [randn_bf16((steps + warm, 1, hkv, d), 7 * (layer + 1) + 2, R.dev) for layer in layers]
        od = torch.empty(1, hq, d, dtype=torch.bfloat16, device=R.dev)
        e0, e1 = R.event(), R.event()
        for s in range(steps + warm):
            if s == warm:
                torch.cuda.synchronize()
                e0.record(R.stream)
            for li in range(len(layers)):
                R.check(lib.duo_decode(caches[li].handle, R.ptr(dq[li][s]), R.ptr(dk[li][s]), R.ptr(dv[li][s]),
                                       R.ptr(od), R.sp), "decode")
        e1.record(R.stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        byts = sum(decode_bytes(w, m, [n_ctx + warm + s]) for m in masks for s in range(steps))
        cache_bytes = sum(duo.required_bytes(c) for c in cfgs)
        del caches, bufs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return ms, byts, cache_bytes

    layers = list(range(w.layers))
    masks = [workload_mask(w, l) for l in layers]
    ms, byts, cb = run(layers, masks)
    gbs = byts / (ms * 1e-3) / 1e9
    out = {"workload": w.name, "layers": w.layers, "context": n_ctx, "decode_steps": steps,
           "decode_ms_per_step": round(ms / steps, 3), "decode_gbs": round(gbs, 1),
           "decode_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "decode_bytes_per_step": byts / steps,
           "cache_gib": round(cb / 2**30, 2)}
    sub = layers[:reps_full_layers]
    ms_d, byts_d, cb_d = run(sub, [masks[l] for l in sub])
    ms_f, byts_f, cb_f = run(sub, [full_mask(w)] * len(sub))
    out["full_attention"] = {"layers_compared": len(sub), "duo_decode_ms_per_step": round(ms_d / steps, 3),
                             "full_decode_ms_per_step": round(ms_f / steps, 3),
                             "full_decode_gbs": round(byts_f / (ms_f * 1e-3) / 1e9, 1),
                             "decode_speedup": ratio(ms_f, ms_d), "memory_reduction": ratio(cb_f, cb_d)}
    return out


def leg_mixed(R, reps, warmup):
    """32 sequences of lengths U[4096, 65536]: chunked prefill (4096-token
    calls; finished sequences pass 0) then 64 decode steps, at 2, 4 and 6 of
    8 KV heads retrieval and with all 8 (full attention)."""
    from workloads import WORKLOADS, randn_bf16, retrieval_mask, sequence_lengths
    torch, duo, lib = R.torch, R.duo, R.lib
    w = WORKLOADS["mixed_gqa_b32"]
    lens = [int(x) for x in sequence_lengths(w.batch, w.length_range[0], w.length_range[1], w.seed)]
    ck, hq, hkv, d = w.chunk, w.num_q_heads, w.num_kv_heads, w.head_dim
    ncalls = -(-max(lens) // ck)
    t_all = max(lens) + w.decode_steps
    # two distinct seeded chunks of inputs, used by calls in turn (the
    # values do not change what the kernels do)
    pool = [tuple(randn_bf16((w.batch, ck, h, d), 11 * (i + 1) + j, R.dev) for j, h in enumerate((hq, hkv, hkv)))
            for i in range(2)]
    dq = randn_bf16((w.decode_steps, w.batch, hq, d), 901, R.dev)
    dk = randn_bf16((w.decode_steps, w.batch, hkv, d), 902, R.dev)
    dv = randn_bf16((w.decode_steps, w.batch, hkv, d), 903, R.dev)
    outp = torch.empty(w.batch, ck, hq, d, dtype=torch.bfloat16, device=R.dev)
    outd = torch.empty(w.batch, hq, d, dtype=torch.bfloat16, device=R.dev)
    n_calls = [(ctypes.c_int32 * w.batch)(*[max(0, min(ck, L - c * ck)) for L in lens]) for c in range(ncalls)]
    res = {"workload": w.name, "batch": w.batch, "mean_length": round(sum(lens) / len(lens), 1),
           "prefill_calls": ncalls, "reps": reps, "ratios": {}}
    buf = None

    def run(cfg):
        """(prefill ms, decode ms) summed over the timed repetitions."""
        nonlocal buf
        need = duo.required_bytes(cfg)
        if buf is None or buf.numel() < need:
            buf = None
            torch.cuda.empty_cache()
            buf = torch.empty(need, dtype=torch.uint8, device=R.dev)
        ev = [R.event() for _ in range(3)]
        pre_ms = dec_ms = 0.0
        for it in range(warmup + reps):
            cache = duo.duo_cache_init(cfg, buf)
            ev[0].record(R.stream)
            for c in range(ncalls):
                q, k, v = pool[c % 2]
                R.check(lib.duo_prefill(cache.handle, R.ptr(q), R.ptr(k), R.ptr(v), n_calls[c], ck, R.ptr(outp),
                                        R.sp), "prefill")
            ev[1].record(R.stream)
            for s in range(w.decode_steps):
                R.check(lib.duo_decode(cache.handle, R.ptr(dq[s]), R.ptr(dk[s]), R.ptr(dv[s]), R.ptr(outd), R.sp),
                        "decode")
            ev[2].record(R.stream)
            torch.cuda.synchronize()
            if it >= warmup:
                pre_ms += ev[0].elapsed_time(ev[1])
                dec_ms += ev[1].elapsed_time(ev[2])
            del cache
        return pre_ms, dec_ms, need

    for nr in list(w.extra["ratio_sweep"]) + [hkv]:
        mask = retrieval_mask(hkv, nr, w.seed + nr) if nr < hkv else full_mask(w)  # the parity test's masks
        cfg = duo.Config(w.batch, hq, hkv, d, t_all, w.sink, w.recent, [int(x) for x in mask])
        pre_ms, dec_ms, need = run(cfg)
        flops = prefill_flops(w, mask, [(0, L) for L in lens])
        byts = sum(decode_bytes(w, mask, [L + s for L in lens]) for s in range(w.decode_steps))
        gbs = byts * reps / (dec_ms * 1e-3) / 1e9
        tfl = flops * reps / (pre_ms * 1e-3) / 1e12
        key = f"{100 * nr // hkv}%"
        res["ratios"][key] = {"retrieval_kv_heads": nr, "prefill_ms": round(pre_ms / reps, 3),
                              "prefill_tflops": round(tfl, 1),
                              "prefill_frac_of_mfma_peak": round(tfl / BF16_MFMA_PEAK_TFLOPS, 4),
                              "decode_us_per_call": round(dec_ms / reps / w.decode_steps * 1e3, 2),
                              "decode_gbs": round(gbs, 1), "decode_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                              "cache_bytes": need}
    full = res["ratios"]["100%"]
    for key, r in res["ratios"].items():
        if key != "100%":
            r["decode_speedup_vs_full"] = ratio(full["decode_us_per_call"], r["decode_us_per_call"])
            r["prefill_speedup_vs_full"] = ratio(full["prefill_ms"], r["prefill_ms"])
            r["memory_reduction_vs_full"] = ratio(full["cache_bytes"], r["cache_bytes"])
    # an int8 retrieval cache at 4 of 8 retrieval KV heads: every chunk after
    # the first attends a stored int8 prefix, decoded in every tile (tiled)
    # or once per call into the staging workspace (staged)
    nr = hkv // 2
    mask = retrieval_mask(hkv, nr, w.seed + nr)
    base = res["ratios"][f"{100 * nr // hkv}%"]
    res["int8_prefix"] = {"retrieval_kv_heads": nr}
    for mode in ("tiled", "staged"):
        cfg = duo.Config(w.batch, hq, hkv, d, t_all, w.sink, w.recent, [int(x) for x in mask],
                         kv_format=duo.DUO_KV_INT8)
        if mode == "staged":
            cfg.prefill_staging = torch.empty(duo.prefill_staging_bytes(cfg), dtype=torch.uint8, device=R.dev)
        pre_ms, dec_ms, need = run(cfg)
        res["int8_prefix"][mode] = {
            "prefill_ms": round(pre_ms / reps, 3), "prefill_time_vs_bf16": ratio(pre_ms / reps, base["prefill_ms"]),
            "decode_us_per_call": round(dec_ms / reps / w.decode_steps * 1e3, 2),
            "cache_bytes": need, "staging_bytes": duo.prefill_staging_bytes(cfg) if mode == "staged" else 0}
        del cfg
    del pool, buf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# ---- CPU baseline -------------------------------------------------------

def cpu_baseline(w, mask, ins_l0, budget_s=12.0):
    """The fp64 oracle as it stands, on a bounded sample of the headline
    workload (sequence 0, every query head): decode steps from step 0 on,
    then prefill rows from the end of the context, each for about budget_s
    seconds with all host cores and a shorter slice with one thread.
    Reported in the decode metric's unit (decode bytes the oracle covers per
    second) and as oracle flops per second, with the full workload's oracle
    time extrapolated from those rates (labelled as such)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attend_rows
    (pq, pk, pv), dec = ins_l0
    cores = len(os.sched_getaffinity(0))
    g = w.group
    scale = 1.0 / math.sqrt(w.head_dim)
    b = 0
    t_all = w.prefill + w.decode_steps
    # fp64 copies of sequence 0's K/V per KV head, outside the timed region
    k64 = [np.empty((t_all, w.head_dim)) for _ in range(w.num_kv_heads)]
    v64 = [np.empty((t_all, w.head_dim)) for _ in range(w.num_kv_heads)]
    pk0, pv0 = pk[b].float().cpu().numpy(), pv[b].float().cpu().numpy()
    for h in range(w.num_kv_heads):
        k64[h][:w.prefill] = pk0[:, h]
        v64[h][:w.prefill] = pv0[:, h]
    for s, (q, k, v) in enumerate(dec):
        kk, vv = k[b].float().cpu().numpy(), v[b].float().cpu().numpy()
        for h in range(w.num_kv_heads):
            k64[h][w.prefill + s] = kk[h]
            v64[h][w.prefill + s] = vv[h]
    dq = [x[0][b].float().cpu().numpy() for x in dec]
    pq0 = pq[b].float().cpu().numpy()

    def decode_sample(limit_s):
        t0 = time.perf_counter()
        byts, steps = 0.0, 0
        for s in range(w.decode_steps):
            t = w.prefill + s
            for h in range(w.num_q_heads):
                kvh = h // g
                attend_rows(dq[s][h][None], [t], k64[kvh], v64[kvh], bool(mask[kvh]), w.sink, w.recent, scale)
            byts += decode_bytes(w, mask, [t]) / 1.0
            steps += 1
            if time.perf_counter() - t0 > limit_s:
                break
        return byts, steps, time.perf_counter() - t0

    def prefill_sample(limit_s):
        t0 = time.perf_counter()
        flops, rows = 0.0, 0
        for i in range(w.prefill - 1, -1, -1):
            for h in range(w.num_q_heads):
                kvh = h // g
                attend_rows(pq0[i, h][None], [i], k64[kvh], v64[kvh], bool(mask[kvh]), w.sink, w.recent, scale)
                flops += 4.0 * w.head_dim * allowed(i, bool(mask[kvh]), w.sink, w.recent)
            rows += 1
            if time.perf_counter() - t0 > limit_s:
                break
        return flops, rows, time.perf_counter() - t0

    with threadpool_limits(limits=cores):
        db, ds, dt = decode_sample(budget_s)
        pf, pr, pt = prefill_sample(budget_s)
    with threadpool_limits(limits=1):
        db1, ds1, dt1 = decode_sample(budget_s / 3)
        pf1, pr1, pt1 = prefill_sample(budget_s / 3)
    flops_all, bytes_all = layer_counts(w, [mask])
    dec_rate, pre_rate = db / dt, pf / pt
    dec_rate1, pre_rate1 = db1 / dt1, pf1 / pt1
    return {
        "value": round(dec_rate / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": (f"numpy fp64 oracle, sequence 0 of {w.name}, all {w.num_q_heads} query heads: {ds} decode steps "
                   f"at context {w.prefill}+ ({dt:.2f} s) and {pr} prefill rows from position {w.prefill - 1} "
                   f"down ({pt:.2f} s), BLAS threads = os.sched_getaffinity = {cores}"),
        "seconds": round(dt + pt, 3),
        "prefill_tflops": round(pre_rate / 1e12, 6),
        "one_thread": {"decode_gbs": round(dec_rate1 / 1e9, 4), "prefill_tflops": round(pre_rate1 / 1e12, 6),
                       "decode_steps": ds1, "prefill_rows": pr1, "seconds": round(dt1 + pt1, 3)},
        "extrapolated_full_workload": {
            "label": "EXTRAPOLATED from the sampled rates (oracle cost per byte / per flop is flat in the row)",
            "decode_s": round(bytes_all / dec_rate, 1), "prefill_s": round(flops_all / pre_rate, 1),
            "decode_s_one_thread": round(bytes_all / dec_rate1, 1),
            "prefill_s_one_thread": round(flops_all / pre_rate1, 1)},
    }


# ---- main ---------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path, and a figure at more than one "
              "GPU is not produced (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import kv_cache_duo_amd as duo
    from workloads import WORKLOADS, workload_mask

    w = WORKLOADS[args.workload]
    if w.length_range is not None or w.layers > 1:
        print(f"workload {w.name} is a leg of the benchmark, not a headline step", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lib = duo.load_library()
    stream = torch.cuda.current_stream()
    R = Runner(torch, duo, lib, dev, stream)
    legs = [x for x in args.legs.split(",") if x]
    unknown = set(legs) - set(ALL_LEGS.split(","))
    if unknown:
        print(f"unknown legs: {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)

    # ---- headline step
    t_all = w.prefill + w.decode_steps
    per_layer = 4 * w.head_dim * w.batch * w.n_retrieval * t_all
    nl = args.layers or (8 if per_layer < (1 << 30) else 1)
    say(f"{w.name}: {nl} layer cache(s), generating inputs")
    masks = [workload_mask(w, l) for l in range(nl)]
    ins = layer_inputs(torch, w, nl, dev)
    cfgs = make_cfgs(duo, w, masks, t_all)
    bufs = R.buffers(cfgs)
    say("headline step")
    wall0 = time.perf_counter()
    pre_ms, dec_ms, timed_ms = time_layer_step(R, w, cfgs, bufs, ins, args.steps, args.warmup)
    wall = time.perf_counter() - wall0
    head = summarize(w, masks, pre_ms, dec_ms, args.steps)
    bytes_launch = head["decode_bytes_per_call"]
    achieved = bytes_launch / (head["decode_us_per_call"] * 1e-6) / 1e9
    flops_call = head["prefill_flops_per_call"]
    pre_achieved = flops_call / (head["prefill_ms_per_call"] * 1e-3) / 1e12
    result = {
        "metric": "decode attn HBM GB/s (% of peak) + prefill TFLOP/s (% MFMA peak), 1 MI355X",
        "value": head["decode_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(timed_ms / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "retrieval_kv_heads": w.n_retrieval, "prefill_tokens": w.prefill,
            "decode_steps": w.decode_steps, "sink": w.sink, "recent": w.recent, "layers_rotated": nl,
        },
        "decode": {"gbs": head["decode_gbs"], "frac_of_hbm_peak": head["decode_frac_of_hbm_peak"],
                   "phase_ms_per_step": round(dec_ms / args.steps, 3), "calls_per_step": w.decode_steps * nl},
        "prefill": {"tflops": head["prefill_tflops"], "frac_of_mfma_peak": head["prefill_frac_of_mfma_peak"],
                    "phase_ms_per_step": round(pre_ms / args.steps, 3), "flops_per_step": flops_call * nl},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name),
                     "kernel": "decode_kernel (one launch per decode call)",
                     "mean_launch_us": head["decode_us_per_call"], "bytes_per_launch": bytes_launch},
        "roofline_prefill": {"bound": "mfma", "achieved": round(pre_achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(pre_achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                             "kernel": "prefill_kernel + append_kernel (one prefill call)",
                             "mean_launch_ms": head["prefill_ms_per_call"], "flops_per_launch": flops_call},
        "wall_s": round(wall, 3),
    }
    reps, warm = 2, 1  # the legs' own repetitions
    if not args.no_full:
        say("full-attention reference")
        fm = [full_mask(w)] * nl
        cfgf = make_cfgs(duo, w, fm, t_all)
        bf = R.buffers(cfgf, None)
        pre_f, dec_f, _ = time_layer_step(R, w, cfgf, bf, ins, reps, warm)
        s = summarize(w, fm, pre_f, dec_f, reps)
        duo_pre, duo_dec = pre_ms / args.steps, dec_ms / args.steps
        result["full_attention"] = {
            "prefill_ms_per_call": s["prefill_ms_per_call"], "prefill_tflops": s["prefill_tflops"],
            "decode_us_per_call": s["decode_us_per_call"], "decode_gbs": s["decode_gbs"],
            "cache_bytes_per_layer": duo.required_bytes(cfgf[0]),
            "duo_cache_bytes_per_layer": duo.required_bytes(cfgs[0]),
            "decode_speedup": ratio(dec_f / reps, duo_dec), "prefill_speedup": ratio(pre_f / reps, duo_pre),
            "memory_reduction": ratio(duo.required_bytes(cfgf[0]), duo.required_bytes(cfgs[0]))}
        del bf
        torch.cuda.empty_cache()

    def variant(name, row_r=None, mfma_peak=BF16_MFMA_PEAK_TFLOPS, **kw):
        say(f"leg {name}")
        cv = [dataclasses.replace(c, **kw) for c in cfgs]
        bv = R.buffers(cv, bufs)
        p, d, _ = time_layer_step(R, w, cv, bv, ins, reps, warm)
        s = summarize(w, masks, p, d, reps, row_r, mfma_peak)
        s["decode_time_vs_bf16"] = ratio(d / reps, dec_ms / args.steps)
        s["prefill_time_vs_bf16"] = ratio(p / reps, pre_ms / args.steps)
        return s

    if "int8" in legs:
        result["int8"] = {**variant("int8", int8_row(w), kv_format=duo.DUO_KV_INT8),
                          "cache": "retrieval K/V as int8 codes + fp32 row scales (DUO_KV_INT8)"}
    if "int8rope" in legs:
        # int8 cache with rotary embedding: the one-shot prefill attends the
        # chunk's own rows turned; staged once per call into the workspace
        # (the default here) or in every tile (tiled_prefill_ms)
        stg = torch.empty(duo.prefill_staging_bytes(dataclasses.replace(cfgs[0], kv_format=duo.DUO_KV_INT8,
                                                                        rope_base=10000.0)),
                          dtype=torch.uint8, device=R.dev)
        result["int8rope"] = {**variant("int8rope", int8_row(w), kv_format=duo.DUO_KV_INT8, rope_base=10000.0,
                                        rope_style=duo.DUO_ROPE_HALF, prefill_staging=stg),
                              "staging_bytes": stg.numel()}
        del stg
        tiled = variant("int8rope_tiled", int8_row(w), kv_format=duo.DUO_KV_INT8, rope_base=10000.0,
                        rope_style=duo.DUO_ROPE_HALF)
        result["int8rope"]["tiled_prefill_ms"] = tiled["prefill_ms_per_call"]
        result["int8rope"]["tiled_prefill_time_vs_bf16"] = tiled["prefill_time_vs_bf16"]
        torch.cuda.empty_cache()
    if "fp8" in legs:
        # exact prefill: the stored rows decoded once per call into the
        # staging workspace (the default here), or in every tile
        # (tiled_prefill_ms)
        stg = torch.empty(duo.prefill_staging_bytes(dataclasses.replace(cfgs[0], kv_format=duo.DUO_KV_FP8)),
                          dtype=torch.uint8, device=R.dev)
        result["fp8"] = {**variant("fp8", fp8_row(w), kv_format=duo.DUO_KV_FP8, prefill_staging=stg),
                         "cache": "retrieval K/V as e4m3 codes, one power-of-two scale per tensor (DUO_KV_FP8)",
                         "staging_bytes": stg.numel()}
        del stg
        tiled = variant("fp8_tiled", fp8_row(w), kv_format=duo.DUO_KV_FP8)
        result["fp8"]["tiled_prefill_ms"] = tiled["prefill_ms_per_call"]
        result["fp8"]["tiled_prefill_time_vs_bf16"] = tiled["prefill_time_vs_bf16"]
        torch.cuda.empty_cache()
    if "fp8mfma" in legs and hasattr(duo, "DUO_FP8_PREFILL_MFMA"):
        result["fp8mfma"] = {**variant("fp8mfma", fp8_row(w), FP8_MFMA_PEAK_TFLOPS, kv_format=duo.DUO_KV_FP8,
                                       fp8_prefill=duo.DUO_FP8_PREFILL_MFMA),
                             "cache": "DUO_KV_FP8, retrieval prefill on fp8 matrix cores (priced at 5 PFLOP/s)"}
    if "rope" in legs:
        # the streaming heads' chunk K rows turned once per call into the
        # staging workspace (the default here), or in every tile that holds
        # them (tiled_prefill_ms)
        stg = torch.empty(duo.prefill_staging_bytes(dataclasses.replace(cfgs[0], rope_base=10000.0)),
                          dtype=torch.uint8, device=R.dev)
        result["rope"] = {**variant("rope", rope_base=10000.0, rope_style=duo.DUO_ROPE_HALF, prefill_staging=stg),
                          "embedding": "rotary, base 10000, pairs (i, i + D/2), applied inside the library",
                          "staging_bytes": stg.numel()}
        del stg
        tiled = variant("rope_tiled", rope_base=10000.0, rope_style=duo.DUO_ROPE_HALF)
        result["rope"]["tiled_prefill_ms"] = tiled["prefill_ms_per_call"]
        result["rope"]["tiled_prefill_time_vs_bf16"] = tiled["prefill_time_vs_bf16"]
        torch.cuda.empty_cache()
    if "paged" in legs:
        result["paged"] = {**variant("paged", page_tokens=1024, num_pages=w.batch * (-(-t_all // 1024))),
                           "page_tokens": 1024}
    if "dynamic" in legs and hasattr(duo, "DUO_DECODE_DYNAMIC"):
        result["dynamic"] = {**variant("dynamic", decode_split=duo.DUO_DECODE_DYNAMIC),
                             "decode": "dynamic row claiming (not bitwise reproducible)"}
    cpu_ins = ins[0]
    del bufs
    torch.cuda.empty_cache()
    if "mha32k" in legs:
        say("leg mha32k")
        result["mha32k"] = leg_layer(R, WORKLOADS["llama2_7b_mha_32k"], 8, 3, 1, True)
    if "mixed" in legs:
        say("leg mixed")
        result["mixed"] = leg_mixed(R, reps, warm)
    if not args.no_cpu_baseline:
        say("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(w, masks[0], cpu_ins)
    del ins, cpu_ins
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if "stack1m" in legs:
        say("leg stack1m")
        result["stack1m"] = leg_stack(R)
    if not args.no_ceilings:
        say("ceilings")
        mib = lambda b: max(1, int(round(b / 2**20)))  # noqa: E731
        legs8 = [k for k in ("int8", "fp8") if k in result]
        result["measured_ceilings"] = measured_ceilings(mib(bytes_launch),
                                                        [mib(result[k]["decode_bytes_per_call"]) for k in legs8])
        # the decode calls against a measured single-launch read of their own size
        rec = result["measured_ceilings"].get(f"stream_read_rotating_{mib(bytes_launch)}MiB")
        if rec:
            result["decode"]["frac_of_measured_read"] = round(result["decode"]["gbs"] / rec["nontemporal_gbs"], 4)
        for k in legs8:
            rec = result["measured_ceilings"].get(f"stream_read_rotating_{mib(result[k]['decode_bytes_per_call'])}MiB")
            if rec:
                result[k]["decode_frac_of_measured_read"] = round(result[k]["decode_gbs"] / rec["nontemporal_gbs"], 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
