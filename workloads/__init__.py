"""Seeded synthetic workloads shared by the tests and the benchmark.

This module only describes shapes and draws seeded random inputs.  It holds
none of the attention arithmetic: the oracle (``oracle/``) and the HIP
library (``kv_cache_duo_amd``) both consume what it produces and neither is
imported here.

The shapes stand in for the models the DuoAttention pages evaluate (an MHA
Llama-2-7B-32K-shaped layer and a GQA Llama-3-8B-shaped layer; retrieval
ratios of 25% for MHA and 50% for GQA per the sourcepulse card, "Limitations
& Caveats").  No model weights or datasets are used: activations are N(0,1).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    n_retrieval: int            # retrieval KV heads
    prefill: int                # tokens per sequence filled by prefill (or append)
    decode_steps: int
    sink: int
    recent: int
    seed: int = 0
    layers: int = 1
    fixed_mask: tuple | None = None  # explicit retrieval mask instead of a seeded one
    length_range: tuple | None = None  # per-sequence prefill lengths drawn uniformly
    chunk: int | None = None    # chunked prefill size
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    # Tiny single-layer MHA used for full parity: 4 heads, two retrieval
    # (heads 0 and 1), two streaming; fp32 N(0,1) rounded to bf16.
    "tiny_mha_512": Workload(
        "tiny_mha_512", batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64,
        n_retrieval=2, prefill=512, decode_steps=16, sink=4, recent=64, seed=0,
        fixed_mask=(1, 1, 0, 0)),
    # Llama-2-7B-shaped MHA layer: 32 heads of 128, 25% retrieval.
    "llama2_7b_mha_32k": Workload(
        "llama2_7b_mha_32k", batch=1, num_q_heads=32, num_kv_heads=32, head_dim=128,
        n_retrieval=8, prefill=32768, decode_steps=256, sink=64, recent=256, seed=1),
    # Llama-3-8B-shaped GQA layer, batch 8 x 131072 context, 50% retrieval.
    "llama3_8b_gqa_b8_128k": Workload(
        "llama3_8b_gqa_b8_128k", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
        n_retrieval=4, prefill=131072, decode_steps=128, sink=64, recent=256, seed=2),
    # 32 layers of the GQA layer at 1,048,576 tokens, cache filled by append.
    "llama3_8b_gqa_stack_1m": Workload(
        "llama3_8b_gqa_stack_1m", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        n_retrieval=4, prefill=1048576, decode_steps=64, sink=64, recent=256, seed=3,
        layers=32),
    # 32 sequences of mixed length, chunked prefill of 4096, ratio swept.
    "mixed_gqa_b32": Workload(
        "mixed_gqa_b32", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
        n_retrieval=4, prefill=65536, decode_steps=64, sink=64, recent=256, seed=4,
        length_range=(4096, 65536), chunk=4096, extra={"ratio_sweep": (2, 4, 6)}),
}


def retrieval_mask(num_kv_heads: int, n_retrieval: int, seed: int) -> np.ndarray:
    """uint8 [Hkv] with ``n_retrieval`` ones at seeded positions."""
    mask = np.zeros(num_kv_heads, dtype=np.uint8)
    idx = np.random.default_rng(seed).permutation(num_kv_heads)[:n_retrieval]
    mask[idx] = 1
    return mask


def workload_mask(w: Workload, layer: int = 0) -> np.ndarray:
    if w.fixed_mask is not None:
        return np.array(w.fixed_mask, dtype=np.uint8)
    return retrieval_mask(w.num_kv_heads, w.n_retrieval, w.seed * 1000 + layer)


def sequence_lengths(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """int64 [batch], uniform in [lo, hi] inclusive."""
    return np.random.default_rng(seed + 1).integers(lo, hi, size=batch, endpoint=True)


def randn_bf16(shape, seed: int, device="cpu"):
    """N(0,1) drawn in fp32 from a seeded torch generator, rounded to bf16."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def qkv(batch: int, tokens: int, hq: int, hkv: int, d: int, seed: int, device="cpu"):
    """Seeded bf16 q [B,T,Hq,D], k and v [B,T,Hkv,D]."""
    q = randn_bf16((batch, tokens, hq, d), 3 * seed + 1, device)
    k = randn_bf16((batch, tokens, hkv, d), 3 * seed + 2, device)
    v = randn_bf16((batch, tokens, hkv, d), 3 * seed + 3, device)
    return q, k, v
