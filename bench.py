"""Benchmark of the DuoAttention hot path on one MI355X.

One step = the whole path over one batch of synthetic input, for each of
`--layers` independently seeded layer caches (a model's layer loop; it also
keeps the decode working set far above the 256 MB Infinity Cache, so decode
bandwidth is HBM bandwidth):
  cache init -> one-shot prefill of the context -> `decode_steps` decode
  steps (each step visits every layer).
Inputs are resident in HBM before the timed region.  Reported:
  value      decode attention, algorithmic HBM bytes / decode-phase wall time
  prefill    algorithmic flops / prefill-phase wall time
  roofline   decode kernel: algorithmic bytes per launch / mean launch time,
             against 8 TB/s; one decode call is one kernel launch, and the
             mean launch time is the decode phase (HIP events on the launch
             stream) divided by the number of launches
  decode_int8  the same decode phase over an int8 retrieval cache
             (DUO_KV_INT8: codes + fp32 row scales), filled by the same
             prefill; its algorithmic bytes count D + 4 per stored K or V row
  rope       the same step with rotary position embedding applied inside the
             library (same algorithmic counts; rotation work is overhead)
  paged      the same step over a paged retrieval cache (1024-position pages)
  fp8        the same step over an fp8 (e4m3) retrieval cache: retrieval
             heads' prefill on fp8 matrix cores (priced against the 5 PF
             dense fp8 peak), decode over D-byte rows
  cpu_baseline  the fp64 oracle on a bounded sample of the same decode work
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


def source_digest(path: str) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter
    record, or None when the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    src = os.path.join(ROOT, "kv_cache_duo_amd", "csrc", "decode.hip")
    if rec.get("decode_hip_sha256_16") != source_digest(src):
        return None
    return rec.get("bytes_per_launch")


def measured_ceilings(decode_mib: int):
    """Streaming-read (launches of the decode call's size over 8 buffers in
    turn, and 4 GiB) and bf16 MFMA-loop ceilings (constant operands, and
    changing random operands: the sustained MFMA rate is power-limited and
    depends on the data) from kv_cache_duo_amd/ceiling, run as a child."""
    import subprocess
    exe = os.path.join(ROOT, "kv_cache_duo_amd", "ceiling")
    out = {}
    for args in (["stream_read_rotating", str(decode_mib), "8"], ["stream_read", "4096"], ["mfma"], ["mfma_random"],
                 ["mfma_fp8_random"]):
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
    p.add_argument("--workload", default="llama2_7b_mha_32k")
    p.add_argument("--layers", type=int, default=8)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-steps", type=int, default=128)
    p.add_argument("--no-ceilings", action="store_true")
    p.add_argument("--legs", default="int8,rope,paged,fp8",
                   help="variant legs to run after the plain step (comma list of int8, rope, paged, fp8; "
                        "empty for none)")
    return p.parse_args()


def prefill_flops(w, mask) -> float:
    g = w.group
    nr = int(sum(mask))
    ns = w.num_kv_heads - nr
    n = w.prefill
    retr = n * (n + 1) // 2
    cap = w.sink + w.recent
    stream = (min(n, cap) * (min(n, cap) + 1)) // 2 + max(n - cap, 0) * cap
    return 4.0 * w.head_dim * w.batch * g * (nr * retr + ns * stream)


def decode_bytes(w, mask, ctx: int) -> float:
    """Algorithmic bytes of one decode call when each sequence holds ctx tokens."""
    nr = int(sum(mask))
    ns = w.num_kv_heads - nr
    row = 2 * w.head_dim  # bf16 row
    kv = 2 * row * w.batch * (nr * (ctx + 1) + ns * min(ctx + 1, w.sink + w.recent))
    qo = 2 * row * w.batch * w.num_q_heads
    append = 2 * row * w.batch * w.num_kv_heads
    return float(kv + qo + append)


def decode_bytes_int8(w, mask, ctx: int) -> float:
    """Algorithmic bytes of one decode call with an int8 retrieval cache: each
    stored retrieval row once as D codes + a 4-byte scale for K and for V, the
    new token read (bf16) and stored (int8), streaming rows as bf16, q/out."""
    nr = int(sum(mask))
    ns = w.num_kv_heads - nr
    row = 2 * w.head_dim
    row8 = w.head_dim + 4
    kv = 2 * w.batch * (nr * (ctx * row8 + row + row8) + ns * row * min(ctx + 1, w.sink + w.recent))
    qo = 2 * row * w.batch * w.num_q_heads
    append = 2 * row * w.batch * ns  # streaming heads' new token stored as bf16
    return float(kv + qo + append)


def decode_bytes_fp8(w, mask, ctx: int) -> float:
    """Algorithmic bytes of one decode call with an fp8 retrieval cache: each
    stored retrieval row once as D codes for K and for V (one scale per
    tensor, a kernel argument), the new token read (bf16) and stored (fp8),
    streaming rows as bf16, q/out."""
    nr = int(sum(mask))
    ns = w.num_kv_heads - nr
    row = 2 * w.head_dim
    row8 = w.head_dim
    kv = 2 * w.batch * (nr * (ctx * row8 + row + row8) + ns * row * min(ctx + 1, w.sink + w.recent))
    qo = 2 * row * w.batch * w.num_q_heads
    append = 2 * row * w.batch * ns
    return float(kv + qo + append)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import kv_cache_duo_amd as duo
    from workloads import WORKLOADS, qkv, workload_mask

    w = WORKLOADS[args.workload]
    if w.length_range is not None or w.layers > 1:
        print(f"workload {w.name} is a parity case, not a bench line", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lib = duo.load_library()
    nl = args.layers
    t_all = w.prefill + w.decode_steps
    masks = [workload_mask(w, layer) for layer in range(nl)]
    cfgs = [duo.Config(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, t_all, w.sink, w.recent,
                       [int(x) for x in m]) for m in masks]
    bufs = [torch.empty(duo.required_bytes(c), dtype=torch.uint8, device=dev) for c in cfgs]
    ins = [qkv(w.batch, t_all, w.num_q_heads, w.num_kv_heads, w.head_dim, w.seed * 100 + layer, dev)
           for layer in range(nl)]
    outp = torch.empty(w.batch, w.prefill, w.num_q_heads, w.head_dim, dtype=torch.bfloat16, device=dev)
    outd = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.bfloat16, device=dev)
    # decode inputs per (layer, step), contiguous [B,H,D]
    dq = [[ins[l][0][:, w.prefill + s].contiguous() for s in range(w.decode_steps)] for l in range(nl)]
    dk = [[ins[l][1][:, w.prefill + s].contiguous() for s in range(w.decode_steps)] for l in range(nl)]
    dv = [[ins[l][2][:, w.prefill + s].contiguous() for s in range(w.decode_steps)] for l in range(nl)]
    pq = [ins[l][0][:, :w.prefill].contiguous() for l in range(nl)]
    pk = [ins[l][1][:, :w.prefill].contiguous() for l in range(nl)]
    pv = [ins[l][2][:, :w.prefill].contiguous() for l in range(nl)]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    n_new = (ctypes.c_int32 * w.batch)(*([w.prefill] * w.batch))
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    dq_p = [[ptr(x) for x in row] for row in dq]
    dk_p = [[ptr(x) for x in row] for row in dk]
    dv_p = [[ptr(x) for x in row] for row in dv]
    od_p = ptr(outd)
    op_p = ptr(outp)
    n_dec = w.decode_steps * nl
    ph = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def check(st, where):
        if st != 0:
            raise RuntimeError(f"{where}: {duo.status_string(st)}")

    def one_step():
        caches = [duo.duo_cache_init(cfgs[l], bufs[l]) for l in range(nl)]
        hs = [c.handle for c in caches]
        ph[0].record(stream)
        for l in range(nl):
            check(lib.duo_prefill(hs[l], ptr(pq[l]), ptr(pk[l]), ptr(pv[l]), n_new, w.prefill, op_p, sp),
                  "prefill")
        ph[1].record(stream)
        for s in range(w.decode_steps):
            for l in range(nl):
                check(lib.duo_decode(hs[l], dq_p[l][s], dk_p[l][s], dv_p[l][s], od_p, sp), "decode")
        ph[2].record(stream)
        return caches

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    pre_ms = dec_ms = 0.0
    t0.record(stream)
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        caches = one_step()
        torch.cuda.synchronize()
        pre_ms += ph[0].elapsed_time(ph[1])
        dec_ms += ph[1].elapsed_time(ph[2])
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t0.elapsed_time(t1) / args.steps
    del caches

    # algorithmic work
    flops_step = sum(prefill_flops(w, m) for m in masks)
    bytes_step = sum(decode_bytes(w, m, w.prefill + s) for m in masks for s in range(w.decode_steps))
    dec_gbs = bytes_step * args.steps / (dec_ms * 1e-3) / 1e9
    pre_tflops = flops_step * args.steps / (pre_ms * 1e-3) / 1e12
    mean_dec_launch = dec_ms / (args.steps * n_dec)  # ms per decode launch
    bytes_per_launch = bytes_step / n_dec
    achieved = bytes_per_launch / (mean_dec_launch * 1e-3) / 1e9
    mean_pre_launch = pre_ms / (args.steps * nl)     # ms per prefill call (prefill + append kernels)
    pre_achieved = (flops_step / nl) / (mean_pre_launch * 1e-3) / 1e12

    def variant_phases(cfgs_v, what):
        """Prefill and decode phase times (ms, summed over the timed steps)
        of the same step on caches of another configuration (the buffers of
        the main run are reused where they are large enough)."""
        bv = [bufs[l] if duo.required_bytes(cfgs_v[l]) <= bufs[l].numel() else
              torch.empty(duo.required_bytes(cfgs_v[l]), dtype=torch.uint8, device=dev) for l in range(nl)]
        pre_v = dec_v = 0.0
        for it in range(args.warmup + args.steps):
            cv = [duo.duo_cache_init(cfgs_v[l], bv[l]) for l in range(nl)]
            hv = [c.handle for c in cv]
            ph[0].record(stream)
            for l in range(nl):
                check(lib.duo_prefill(hv[l], ptr(pq[l]), ptr(pk[l]), ptr(pv[l]), n_new, w.prefill, op_p, sp),
                      f"prefill {what}")
            ph[1].record(stream)
            for s in range(w.decode_steps):
                for l in range(nl):
                    check(lib.duo_decode(hv[l], dq_p[l][s], dk_p[l][s], dv_p[l][s], od_p, sp), f"decode {what}")
            ph[2].record(stream)
            torch.cuda.synchronize()
            if it >= args.warmup:
                pre_v += ph[0].elapsed_time(ph[1])
                dec_v += ph[1].elapsed_time(ph[2])
        return pre_v, dec_v

    # the same step with an int8 retrieval cache (DUO_KV_INT8: smaller, so
    # the bf16 buffers hold it), and with rotary position embedding applied
    # inside the library (base 10000, half-split pairs)
    variants = {}
    legs = [x for x in args.legs.split(",") if x]
    if "int8" in legs:
        variants["int8"] = variant_phases([dataclasses.replace(c, kv_format=duo.DUO_KV_INT8) for c in cfgs], "int8")
    if "rope" in legs:
        variants["rope"] = variant_phases(
            [dataclasses.replace(c, rope_base=10000.0, rope_style=duo.DUO_ROPE_HALF) for c in cfgs], "rope")
    # and with a paged retrieval cache (pages of 1024 positions, a pool just
    # large enough)
    page = 1024
    if "fp8" in legs:
        variants["fp8"] = variant_phases([dataclasses.replace(c, kv_format=duo.DUO_KV_FP8) for c in cfgs], "fp8")
    if "paged" in legs:
        variants["paged"] = variant_phases(
            [dataclasses.replace(c, page_tokens=page, num_pages=(t_all + page - 1) // page) for c in cfgs], "paged")

    result = {
        "metric": "decode attn HBM GB/s (% of peak) + prefill TFLOP/s (% MFMA peak), 1 MI355X",
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
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
        "decode": {"gbs": round(dec_gbs, 1), "frac_of_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "phase_ms_per_step": round(dec_ms / args.steps, 3),
                   "calls_per_step": n_dec},
        "prefill": {"tflops": round(pre_tflops, 1),
                    "frac_of_mfma_peak": round(pre_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                    "phase_ms_per_step": round(pre_ms / args.steps, 3),
                    "flops_per_step": flops_step},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "decode_kernel (one launch per decode call)",
                     "mean_launch_us": round(mean_dec_launch * 1e3, 3),
                     "bytes_per_launch": bytes_per_launch},
        "roofline_prefill": {"bound": "mfma", "achieved": round(pre_achieved, 1),
                             "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(pre_achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                             "kernel": "prefill_kernel + append_kernel (one prefill call)",
                             "mean_launch_ms": round(mean_pre_launch, 4)},
        "wall_s": round(wall, 3),
    }
    if "int8" in variants:
        dec8_ms = variants["int8"][1]
        bytes8_step = sum(decode_bytes_int8(w, m, w.prefill + s) for m in masks for s in range(w.decode_steps))
        dec8_gbs = bytes8_step * args.steps / (dec8_ms * 1e-3) / 1e9
        result["decode_int8"] = {"gbs": round(dec8_gbs, 1), "frac_of_hbm_peak": round(dec8_gbs / HBM_PEAK_GBS, 4),
                                 "phase_ms_per_step": round(dec8_ms / args.steps, 3),
                                 "bytes_per_launch": bytes8_step / n_dec,
                                 "decode_time_vs_bf16": round(dec8_ms / dec_ms, 4),
                                 "cache": "retrieval K/V as int8 codes + fp32 row scales (DUO_KV_INT8)"}
    if "rope" in variants:
        pre_r_ms, dec_r_ms = variants["rope"]
        result["rope"] = {"decode_gbs": round(bytes_step * args.steps / (dec_r_ms * 1e-3) / 1e9, 1),
                          "prefill_tflops": round(flops_step * args.steps / (pre_r_ms * 1e-3) / 1e12, 1),
                          "decode_time_vs_plain": round(dec_r_ms / dec_ms, 4),
                          "prefill_time_vs_plain": round(pre_r_ms / pre_ms, 4),
                          "embedding": "rotary, base 10000, pairs (i, i + D/2), applied to q and k inside the library"}
    if "paged" in variants:
        pre_p_ms, dec_p_ms = variants["paged"]
        result["paged"] = {"decode_gbs": round(bytes_step * args.steps / (dec_p_ms * 1e-3) / 1e9, 1),
                           "prefill_tflops": round(flops_step * args.steps / (pre_p_ms * 1e-3) / 1e12, 1),
                           "decode_time_vs_contiguous": round(dec_p_ms / dec_ms, 4),
                           "prefill_time_vs_contiguous": round(pre_p_ms / pre_ms, 4),
                           "page_tokens": page}
    if "fp8" in variants:
        pre_f_ms, dec_f_ms = variants["fp8"]
        bytesf_step = sum(decode_bytes_fp8(w, m, w.prefill + s) for m in masks for s in range(w.decode_steps))
        decf_gbs = bytesf_step * args.steps / (dec_f_ms * 1e-3) / 1e9
        pref_tflops = flops_step * args.steps / (pre_f_ms * 1e-3) / 1e12
        result["fp8"] = {"decode_gbs": round(decf_gbs, 1), "decode_frac_of_hbm_peak": round(decf_gbs / HBM_PEAK_GBS, 4),
                         "decode_bytes_per_launch": bytesf_step / n_dec,
                         "decode_time_vs_bf16": round(dec_f_ms / dec_ms, 4),
                         "prefill_tflops": round(pref_tflops, 1),
                         "prefill_frac_of_fp8_mfma_peak": round(pref_tflops / FP8_MFMA_PEAK_TFLOPS, 4),
                         "prefill_phase_ms_per_step": round(pre_f_ms / args.steps, 3),
                         "prefill_time_vs_bf16": round(pre_f_ms / pre_ms, 4),
                         "cache": "retrieval K/V as e4m3 codes, one power-of-two scale per tensor (DUO_KV_FP8)"}
    if not args.no_ceilings:
        result["measured_ceilings"] = measured_ceilings(max(1, int(round(bytes_per_launch / 2**20))))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, masks[0], ins[0], args.cpu_sample_steps)
    print(json.dumps(result), flush=True)


def cpu_baseline(w, mask, qkv_l0, sample_steps):
    """Oracle timed on a bounded sample: the first `sample_steps` decode steps
    of layer 0 (every query head), in the decode metric's unit."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attend_rows
    q, k, v = (x.float().cpu().numpy() for x in qkv_l0)
    g = w.group
    scale = 1.0 / math.sqrt(w.head_dim)
    b = 0
    # fp64 copies per KV head, outside the timed region
    ks = [np.ascontiguousarray(k[b, :, h, :], dtype=np.float64) for h in range(w.num_kv_heads)]
    vs = [np.ascontiguousarray(v[b, :, h, :], dtype=np.float64) for h in range(w.num_kv_heads)]
    t0 = time.perf_counter()
    done_bytes = 0.0
    steps = 0
    for s in range(sample_steps):
        t = w.prefill + s
        for h in range(w.num_q_heads):
            kvh = h // g
            attend_rows(q[b, [t], h, :], [t], ks[kvh], vs[kvh], bool(mask[kvh]), w.sink, w.recent, scale)
        done_bytes += decode_bytes(w, mask, t) / w.batch
        steps += 1
        if time.perf_counter() - t0 > 30.0:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} decode steps of layer 0, sequence 0, all {w.num_q_heads} query heads, "
                      f"context {w.prefill}+ ({dt:.2f} s)",
            "seconds": round(dt, 3)}


if __name__ == "__main__":
    main()
