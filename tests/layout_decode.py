"""Test-side decoder of the packed cache layout documented in include/rq.h.

Written from the header's description (slot order, sub-planes on 256-byte
boundaries, codes low bits first, sz bytes = [scale, offset] per group, BF16
alpha rows in one block after each loop group's slots), independently of the
library's own geometry code, so the tests can turn the GPU's planes into the
oracle's logical arrays.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def _align(x, a=256):
    return (x + a - 1) // a * a


@dataclass(frozen=True)
class Geom:
    batch: int
    loops: int
    layers: int
    kv_heads: int
    max_tokens: int
    d: int
    P: int
    anchor_bits: int
    residual_bits: int
    mode: int

    @classmethod
    def of(cls, desc):
        return cls(desc.batch, desc.loops, desc.layers, desc.kv_heads, desc.max_tokens,
                   desc.head_dim, desc.loops_per_group, desc.anchor_bits, desc.residual_bits,
                   desc.mode)

    def is_anchor(self, loop):
        return loop % self.P == self.P - 1

    def bits(self, loop):
        return self.anchor_bits if self.is_anchor(loop) else self.residual_bits

    def has_alpha(self, loop):
        return self.mode != 1 and not self.is_anchor(loop)

    def sub_sizes(self, loop):
        T = self.max_tokens
        codes = _align(T * self.d * self.bits(loop) // 8)
        sz = _align(T * 2 * (self.d // 16))
        return codes, sz

    def slot_bytes(self, loop):
        return sum(self.sub_sizes(loop))

    def alpha_row_bytes(self):
        return 2 * self.max_tokens if self.mode != 1 else 0

    def _group_slots(self):
        # the slots of one loop group: P loops (anchor last) x kv heads
        return sum(self.kv_heads * self.slot_bytes(j) for j in range(self.P))

    def group_bytes(self):
        return self._group_slots() + _align((self.P - 1) * self.kv_heads * self.alpha_row_bytes())

    def _group_base(self, kv, b, layer, loop):
        per_layer = (self.loops // self.P) * self.group_bytes()
        return (((kv * self.batch + b) * self.layers + layer) * per_layer
                + (loop // self.P) * self.group_bytes())

    def slot_offset(self, kv, b, layer, loop, head):
        # order: kv, batch, layer, loop group, loop (anchor last), head
        j = loop % self.P
        off = self._group_base(kv, b, layer, loop)
        off += sum(self.kv_heads * self.slot_bytes(l) for l in range(j))
        return off + head * self.slot_bytes(loop)

    def alpha_offset(self, kv, b, layer, loop, head):
        j = loop % self.P
        return (self._group_base(kv, b, layer, loop) + self._group_slots()
                + (j * self.kv_heads + head) * self.alpha_row_bytes())

    def total(self):
        return 2 * self.batch * self.layers * (self.loops // self.P) * self.group_bytes()


def unpack_codes(raw: np.ndarray, bits: int, d: int) -> np.ndarray:
    """raw uint8 [N, d*bits/8] -> codes uint8 [N, d]; element i at bit i*bits."""
    per = 8 // bits
    out = np.empty((raw.shape[0], d), np.uint8)
    mask = (1 << bits) - 1
    for k in range(per):
        out[:, k::per] = (raw >> (k * bits)) & mask
    return out


@dataclass
class Planes:
    codes: np.ndarray  # uint8 [L, N, d]
    s8: np.ndarray     # uint8 [L, N, ng]
    z8: np.ndarray
    alpha: np.ndarray  # uint16 [L, N]


def _bytes(cache: torch.Tensor, off: int, n: int) -> np.ndarray:
    return cache[off:off + n].cpu().numpy()


def decode_slice(cache: torch.Tensor, geom: Geom, kv: int, b: int, layer: int, head: int,
                 n_tokens: int, t0: int = 0) -> Planes:
    """Logical planes of one (kv, batch row, layer, head) slice, tokens [t0, t0+n)."""
    d, ng, N = geom.d, geom.d // 16, n_tokens
    codes = np.zeros((geom.loops, N, d), np.uint8)
    s8 = np.zeros((geom.loops, N, ng), np.uint8)
    z8 = np.zeros((geom.loops, N, ng), np.uint8)
    alpha = np.zeros((geom.loops, N), np.uint16)
    for loop in range(geom.loops):
        off = geom.slot_offset(kv, b, layer, loop, head)
        bits = geom.bits(loop)
        cb = d * bits // 8
        c_sz, _ = geom.sub_sizes(loop)
        raw = _bytes(cache, off + t0 * cb, N * cb).reshape(N, cb)
        codes[loop] = unpack_codes(raw, bits, d)
        sz = _bytes(cache, off + c_sz + t0 * 2 * ng, N * 2 * ng).reshape(N, ng, 2)
        s8[loop], z8[loop] = sz[:, :, 0], sz[:, :, 1]
        if geom.has_alpha(loop):
            a = _bytes(cache, geom.alpha_offset(kv, b, layer, loop, head) + 2 * t0, 2 * N)
            alpha[loop] = a.view(np.uint16)
    return Planes(codes, s8, z8, alpha)
