"""Seeded synthetic inputs: looped-Transformer-like K/V states, queries and
rotation sign vectors.

This module holds no quantization or attention arithmetic.  It is the only
piece that both the GPU path's tests/benchmark and the CPU oracle consume, so
that both sides see identical BF16 inputs.

Value recipe (shapes follow the looped models the pages evaluate: Ouro-1.4B
with 24 layers and 4 loops, and Huginn-3.5B with 32 loops in 8 groups of 4;
head shapes are assumptions):
  * per (K/V, layer, kv head, channel) scale lam = exp(0.5 * N(0,1));
    on K only, 2 channels per (layer, head) are outliers with lam * 10;
  * per loop group, the anchor (last loop of the group) is N(0,1) * lam,
    drawn independently for every group, batch row, token and channel;
  * loop j < P-1 of the group is anchor + sigma_j * N(0,1) (additive, not
    channel-scaled), sigma = (0.3, 0.2, 0.1) for the Ouro-like and tiny
    workloads, (0.3, 0.175, 0.05) for the Huginn-like one;
  * every state is rounded to BF16; queries are BF16 N(0,1);
  * rotation signs are independent +-1 per (K/V, layer, channel).
All draws come from torch generators seeded from the workload seed and the
token chunk, so a chunk is reproducible on the device it is generated on.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    loops: int
    layers: int
    kv_heads: int
    q_heads: int
    head_dim: int
    n_tokens: int
    loops_per_group: int = 4
    sigmas: tuple = (0.3, 0.2, 0.1)
    seed: int = 0
    mode: int = 0                # 0 residual, 1 direct, 2 chained
    anchor_bits: int = 4
    residual_bits: int = 2
    alpha_mode: int = 0          # 0 least squares, 1 norm ratio, 2 fixed 1
    rotation: int = 1            # 1 randomized Hadamard, 0 none
    outlier_channels: int = 2
    outlier_factor: float = 10.0
    lognormal_sigma: float = 0.5
    page_tokens: int = 0         # > 0: paged cache of blocks this size, scattered over the pool

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 1 layer, 4 loops (loop 3 = anchor), 2 KV heads x 64, 256 tokens, batch 1.
    "tiny": Workload("tiny", batch=1, loops=4, layers=1, kv_heads=2, q_heads=2,
                     head_dim=64, n_tokens=256),
    # Ouro-1.4B-like decode step: 24 layers x 4 loops, 16 heads x 128, 8k, batch 4.
    "ouro8k_b4": Workload("ouro8k_b4", batch=4, loops=4, layers=24, kv_heads=16,
                          q_heads=16, head_dim=128, n_tokens=8192),
    "ouro16k_b2": Workload("ouro16k_b2", batch=2, loops=4, layers=24, kv_heads=16,
                           q_heads=16, head_dim=128, n_tokens=16384),
    "ouro16k_b4": Workload("ouro16k_b4", batch=4, loops=4, layers=24, kv_heads=16,
                           q_heads=16, head_dim=128, n_tokens=16384),
    "ouro16k_b2_direct": Workload("ouro16k_b2_direct", batch=2, loops=4, layers=24,
                                  kv_heads=16, q_heads=16, head_dim=128, n_tokens=16384,
                                  mode=1),
    "ouro16k_b4_direct": Workload("ouro16k_b4_direct", batch=4, loops=4, layers=24,
                                  kv_heads=16, q_heads=16, head_dim=128, n_tokens=16384,
                                  mode=1),
    # the ablation's chained (previous-loop) reference on the 8k/batch 4 shapes
    "ouro8k_b4_chained": Workload("ouro8k_b4_chained", batch=4, loops=4, layers=24, kv_heads=16,
                                  q_heads=16, head_dim=128, n_tokens=8192, mode=2),
    # the 8k/batch 4 shapes in a paged cache: blocks of 16 tokens in random pool order
    "ouro8k_b4_paged16": Workload("ouro8k_b4_paged16", batch=4, loops=4, layers=24, kv_heads=16,
                                  q_heads=16, head_dim=128, n_tokens=8192, page_tokens=16),
    # grouped-query variants of the Ouro-like shapes with the same KV bytes per call
    # (64 (batch, KV head) rows x 8192 tokens): 4 and 8 query heads per KV head
    "ouro8k_b16_gqa4": Workload("ouro8k_b16_gqa4", batch=16, loops=4, layers=24, kv_heads=4,
                                q_heads=16, head_dim=128, n_tokens=8192),
    "ouro8k_b32_gqa8": Workload("ouro8k_b32_gqa8", batch=32, loops=4, layers=24, kv_heads=2,
                                q_heads=16, head_dim=128, n_tokens=8192),
    # Huginn-3.5B-like looped core: 4 layers x 32 loops (8 groups of 4), 55 x 96, 8k, b2.
    "huginn8k_b2": Workload("huginn8k_b2", batch=2, loops=32, layers=4, kv_heads=55,
                            q_heads=55, head_dim=96, n_tokens=8192,
                            sigmas=(0.3, 0.175, 0.05)),
}


def channel_scales(w: Workload) -> torch.Tensor:
    """float32 [2, layers, kv_heads, head_dim] per-channel scales (CPU)."""
    g = torch.Generator().manual_seed(w.seed * 7919 + 11)
    lam = torch.exp(w.lognormal_sigma *
                    torch.randn(2, w.layers, w.kv_heads, w.head_dim, generator=g))
    for layer in range(w.layers):
        for h in range(w.kv_heads):
            ch = torch.randperm(w.head_dim, generator=g)[: w.outlier_channels]
            lam[0, layer, h, ch] *= w.outlier_factor
    return lam


def rotation_signs(w: Workload) -> torch.Tensor:
    """int8 [2, layers, head_dim] of +-1 (CPU)."""
    g = torch.Generator().manual_seed(w.seed * 7919 + 23)
    bits = torch.randint(0, 2, (2, w.layers, w.head_dim), generator=g, dtype=torch.int8)
    return (1 - 2 * bits).to(torch.int8)


def kv_chunk(w: Workload, t0: int, t1: int, device="cpu", lam: torch.Tensor | None = None,
             batch_rows=None) -> torch.Tensor:
    """BF16 [2, B, loops, layers, kv_heads, t1-t0, head_dim] for tokens [t0, t1).

    `batch_rows` (a range) restricts generation to some batch rows; every row
    has its own generator stream, so a row's values do not depend on which
    other rows are generated alongside it.
    """
    if lam is None:
        lam = channel_scales(w)
    lam = lam.to(device)
    rows = range(w.batch) if batch_rows is None else batch_rows
    T = t1 - t0
    P = w.loops_per_group
    out = torch.empty(2, len(rows), w.loops, w.layers, w.kv_heads, T, w.head_dim,
                      dtype=torch.bfloat16, device=device)
    sig = list(w.sigmas)
    assert len(sig) == P - 1
    for kv in range(2):
        for ri, b in enumerate(rows):
            gen = torch.Generator(device=device).manual_seed(
                ((w.seed * 1_000_003 + t0) * 8 + kv) * 4099 + b + 1)
            scale = lam[kv].unsqueeze(-2)  # [layers, H, 1, d]
            for k in range(w.loops // P):
                anchor = torch.randn(w.layers, w.kv_heads, T, w.head_dim, generator=gen,
                                     device=device) * scale
                for j in range(P - 1):
                    noise = torch.randn(w.layers, w.kv_heads, T, w.head_dim, generator=gen,
                                        device=device)
                    out[kv, ri, k * P + j] = (anchor + sig[j] * noise).to(torch.bfloat16)
                out[kv, ri, k * P + P - 1] = anchor.to(torch.bfloat16)
    return out


def queries(w: Workload, device="cpu") -> torch.Tensor:
    """BF16 [loops, layers, B, q_heads, head_dim]: one query per (loop, layer)."""
    gen = torch.Generator(device=device).manual_seed(w.seed * 7919 + 41)
    return torch.randn(w.loops, w.layers, w.batch, w.q_heads, w.head_dim, generator=gen,
                       device=device).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a BF16 tensor's bit patterns (copied to host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
