"""Synthetic looped-Transformer decode workloads over librq.

A decode step is what a looped model does per generated token, restricted to
the KV-cache path: for every loop (outer) and layer (inner), one query token
per (batch row, head) attends to that loop's cache, then the new token's K/V
for all loops and layers is quantize-appended (ai4snews summary, paragraph 4;
agihunt "Confirmed": Ouro-1.4B, 24 layers, 4 loops).  The cache is filled
beforehand by chunked quantize-append of generated BF16 states, so no full
BF16 copy of a large cache ever exists.
"""
from __future__ import annotations

from typing import Dict, Iterable, Tuple

import numpy as np
import torch

from . import rq
from .synth import Workload, channel_scales, kv_chunk, queries, rotation_signs

SliceKey = Tuple[int, int, int]  # (batch row, layer, kv head)


def bf16_bytes_per_token(w: Workload) -> int:
    return 2 * w.batch * w.loops * w.layers * w.kv_heads * w.head_dim * 2


def default_chunk(w: Workload, budget_bytes: float = 2.0e9) -> int:
    c = int(budget_bytes // bf16_bytes_per_token(w))
    c = max(64, min(c, w.n_tokens))
    return c - c % 64 if c >= 128 else c


def desc_for(w: Workload, max_tokens: int) -> rq.CacheDesc:
    return rq.make_desc(w.batch, w.loops, w.layers, w.kv_heads, max_tokens, w.head_dim,
                        loops_per_group=w.loops_per_group, anchor_bits=w.anchor_bits,
                        residual_bits=w.residual_bits, mode=w.mode, alpha_mode=w.alpha_mode,
                        rotation=w.rotation)


class RQDecode:
    """A filled ResidualQuant cache plus everything one decode step needs.

    With w.page_tokens > 0 the cache is a paged pool: every batch row owns
    enough blocks for its tokens, drawn in random order from the pool the
    way a serving allocator hands out freed blocks."""

    def __init__(self, w: Workload, device="cuda", keep: Iterable[SliceKey] = (),
                 chunk_tokens: int | None = None, extra_tokens: int = 1):
        self.w = w
        self.N = w.n_tokens
        self.device = device
        self.paged = w.page_tokens > 0
        self._positions: Dict[int, torch.Tensor] = {}   # device start positions of paged appends
        if self.paged:
            per_seq = -(-(w.n_tokens + extra_tokens) // w.page_tokens)
            perm = np.random.default_rng(w.seed + 17).permutation(w.batch * per_seq)
            self.table = torch.from_numpy(perm.reshape(w.batch, per_seq).astype(np.int32)).to(device)
            self.lengths = torch.full((w.batch,), self.N, dtype=torch.int32, device=device)
            self._positions[self.N] = torch.full((w.batch,), self.N, dtype=torch.int32,
                                                 device=device)
            self.desc = desc_for(w, w.page_tokens)
            self.desc.batch = w.batch * per_seq
        else:
            self.desc = desc_for(w, w.n_tokens + extra_tokens)
        self.cache = rq.alloc_cache(self.desc, device)
        self.signs = rotation_signs(w).to(device)
        self.lam = channel_scales(w)
        self.kept: Dict[SliceKey, torch.Tensor] = {}
        self.fill(keep, chunk_tokens or default_chunk(w))
        self.q = queries(w, device)                       # [loops, layers, B, Hq, d]
        self.new_kv = kv_chunk(w, self.N, self.N + 1, device, self.lam)
        ws = rq.paged_decode_workspace_bytes(self.desc, w.q_heads, w.batch, self.N) if self.paged \
            else rq.decode_workspace_bytes(self.desc, w.q_heads, self.N)
        self.ws = rq.alloc_workspace(ws, device)
        self.out = torch.empty(w.loops, w.layers, w.batch, w.q_heads, w.head_dim,
                               dtype=torch.float32, device=device)

    def fill(self, keep: Iterable[SliceKey], chunk: int) -> None:
        keep = list(keep)
        parts = {k: [] for k in keep}
        for t0 in range(0, self.N, chunk):
            t1 = min(self.N, t0 + chunk)
            x = kv_chunk(self.w, t0, t1, self.device, self.lam)
            self._append(x, t0)
            for (b, layer, head) in keep:
                parts[(b, layer, head)].append(x[:, b, :, layer, head].cpu())
            del x
        # [2, loops, N, d] BF16 on the host per kept slice
        self.kept = {k: torch.cat(v, dim=2) if v else None for k, v in parts.items()}

    def _append(self, x: torch.Tensor, t0: int, stream=None) -> None:
        if self.paged:
            if t0 not in self._positions:
                self._positions[t0] = torch.full((self.w.batch,), t0, dtype=torch.int32,
                                                 device=self.device)
            rq.paged_quantize_append(self.desc, self.cache, x, self.table, self._positions[t0],
                                     self.signs, stream=stream)
        else:
            rq.quantize_append(self.desc, self.cache, x, t0, self.signs, stream=stream)

    def attend(self, loop: int, layer: int, stream=None) -> torch.Tensor:
        if self.paged:
            return rq.paged_decode_attention(self.desc, self.cache, self.signs, loop, layer,
                                             self.q[loop, layer], self.table, self.lengths,
                                             self.N, self.w.softmax_scale, self.ws,
                                             out=self.out[loop, layer], stream=stream)
        return rq.decode_attention(self.desc, self.cache, self.signs, loop, layer,
                                   self.q[loop, layer], self.N, self.w.softmax_scale, self.ws,
                                   out=self.out[loop, layer], stream=stream)

    def append_new(self, stream=None) -> None:
        self._append(self.new_kv, self.N, stream)

    def step(self, stream=None) -> None:
        for loop in range(self.w.loops):
            for layer in range(self.w.layers):
                self.attend(loop, layer, stream)
        self.append_new(stream)

    # algorithmic bytes a decode-attention call must read (codes + FP8 + alpha)
    def call_bytes(self, loop: int) -> int:
        w, g = self.w, self.desc
        d, ng = w.head_dim, w.head_dim // 16
        per_token = 0
        P = w.loops_per_group
        anchor = loop % P == P - 1
        if w.mode == rq.MODE_DIRECT or anchor:
            bits = w.anchor_bits if anchor else w.residual_bits
            per_token = d * bits // 8 + 2 * ng
        else:
            # the anchor plus one residual plane (chained mode: one per loop up
            # to the anchor, i.e. distance + 1 reads)
            planes = (P - 1 - loop % P) if w.mode == rq.MODE_CHAINED else 1
            per_token = (d * w.anchor_bits // 8 + 2 * ng) + \
                planes * (d * w.residual_bits // 8 + 2 * ng + 2)
        return 2 * per_token * w.batch * w.kv_heads * self.N

    def step_bytes(self) -> int:
        return sum(self.call_bytes(l) for l in range(self.w.loops)) * self.w.layers


class BF16Decode:
    """Uncompressed BF16 cache of the same workload (the baseline)."""

    def __init__(self, w: Workload, device="cuda", chunk_tokens: int | None = None,
                 extra_tokens: int = 1):
        self.w = w
        self.N = w.n_tokens
        self.desc = desc_for(w, w.n_tokens + extra_tokens)
        shape = (w.batch, w.loops, w.layers, w.kv_heads, self.desc.max_tokens, w.head_dim)
        self.k = torch.empty(shape, dtype=torch.bfloat16, device=device)
        self.v = torch.empty(shape, dtype=torch.bfloat16, device=device)
        lam = channel_scales(w)
        chunk = chunk_tokens or default_chunk(w)
        for t0 in range(0, self.N, chunk):
            t1 = min(self.N, t0 + chunk)
            x = kv_chunk(w, t0, t1, device, lam)
            self.k[:, :, :, :, t0:t1] = x[0]
            self.v[:, :, :, :, t0:t1] = x[1]
            del x
        x = kv_chunk(w, self.N, self.N + 1, device, lam)
        self.new_k, self.new_v = x[0].contiguous(), x[1].contiguous()
        self.q = queries(w, device)
        self.ws = rq.alloc_workspace(rq.bf16_decode_workspace_bytes(self.desc, w.q_heads, self.N),
                                     device)
        self.out = torch.empty(w.loops, w.layers, w.batch, w.q_heads, w.head_dim,
                               dtype=torch.float32, device=device)

    def attend(self, loop: int, layer: int, stream=None) -> torch.Tensor:
        return rq.bf16_decode_attention(self.desc, self.k, self.v, loop, layer,
                                        self.q[loop, layer], self.N, self.w.softmax_scale,
                                        self.ws, out=self.out[loop, layer], stream=stream)

    def append_new(self) -> None:
        self.k[:, :, :, :, self.N:self.N + 1] = self.new_k
        self.v[:, :, :, :, self.N:self.N + 1] = self.new_v

    def step(self, stream=None) -> None:
        for loop in range(self.w.loops):
            for layer in range(self.w.layers):
                self.attend(loop, layer, stream)
        self.append_new()

    def step_bytes(self) -> int:
        w = self.w
        return 2 * w.batch * w.kv_heads * self.N * w.head_dim * 2 * w.loops * w.layers
