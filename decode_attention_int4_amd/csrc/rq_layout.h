// rq_layout.h -- cache geometry shared by the host entry points and the kernels.
//
// A cache is a sequence of (kv, batch, layer) blocks, outermost first; a
// block holds its loop groups in order.  A loop group holds, for each loop
// of the group in order (the anchor, the group's last loop, last), one slot
// per kv head, and after them, when the group's other loops carry an alpha
// plane, its alpha block: one row of max_tokens BF16 per (loop, kv head),
// loop-major.  A slot is codes [max_tokens][d*bits/8] | sz
// [max_tokens][2*d/16], each sub-plane starting on a 256-byte boundary; the
// alpha block is padded to 256 bytes as a whole, so small token capacities
// (paged blocks of 16 tokens) do not pay a 256-byte pad per 32-byte row.
#pragma once
#include <stdint.h>

#include "../../include/rq.h"

#ifdef __HIPCC__
#define RQ_HD __host__ __device__
#else
#define RQ_HD
#endif

namespace rq {

constexpr int kGroup = 16;
constexpr uint64_t kAlign = 256;

RQ_HD inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Everything a kernel needs to address a slot, computed once on the host.
struct Geometry {
  int32_t batch, loops, layers, kv_heads, max_tokens, d, P;
  int32_t anchor_bits, residual_bits, mode, alpha_mode, rotation;
  int32_t ng;                 // d / 16
  uint64_t codes_bytes[2];    // [0] anchor-position slot, [1] other slots
  uint64_t sz_bytes;
  uint64_t slot_bytes[2];
  uint64_t alpha_row;         // 2 * max_tokens: one (loop, kv head) alpha row
  uint64_t alpha_block;       // offset of the alpha block in a group; 0 without alpha
  uint64_t group_bytes;       // one loop group of all kv heads: slots + alpha block
  uint64_t layer_block;       // one (kv, batch, layer) block
  uint64_t total;

  RQ_HD bool is_anchor(int loop) const { return loop % P == P - 1; }
  RQ_HD int bits_of(int loop) const { return is_anchor(loop) ? anchor_bits : residual_bits; }
  RQ_HD bool has_alpha(int loop) const { return mode != RQ_MODE_DIRECT && !is_anchor(loop); }

  RQ_HD uint64_t group_offset(int kv, int b, int layer, int loop) const {
    return ((uint64_t)(kv * batch + b) * layers + layer) * layer_block + (uint64_t)(loop / P) * group_bytes;
  }
  // Byte offset of the codes sub-plane of a slot.
  RQ_HD uint64_t slot_offset(int kv, int b, int layer, int loop, int head) const {
    const int j = loop % P;
    return group_offset(kv, b, layer, loop) + (uint64_t)kv_heads * (uint64_t)j * slot_bytes[1] +
           (uint64_t)head * slot_bytes[j == P - 1 ? 0 : 1];
  }
  RQ_HD uint64_t sz_rel(int loop) const { return codes_bytes[is_anchor(loop) ? 0 : 1]; }
  // Byte offset of the alpha row of a non-anchor loop (has_alpha).
  RQ_HD uint64_t alpha_offset(int kv, int b, int layer, int loop, int head) const {
    return group_offset(kv, b, layer, loop) + alpha_block +
           ((uint64_t)(loop % P) * kv_heads + head) * alpha_row;
  }
};

inline Geometry make_geometry(const rq_cache_desc& c) {
  Geometry g{};
  g.batch = c.batch;
  g.loops = c.loops;
  g.layers = c.layers;
  g.kv_heads = c.kv_heads;
  g.max_tokens = c.max_tokens;
  g.d = c.head_dim;
  g.P = c.loops_per_group;
  g.anchor_bits = c.anchor_bits;
  g.residual_bits = c.residual_bits;
  g.mode = c.mode;
  g.alpha_mode = c.alpha_mode;
  g.rotation = c.rotation;
  g.ng = c.head_dim / kGroup;
  const uint64_t T = (uint64_t)c.max_tokens;
  g.codes_bytes[0] = align_up(T * (uint64_t)c.head_dim * c.anchor_bits / 8, kAlign);
  g.codes_bytes[1] = align_up(T * (uint64_t)c.head_dim * c.residual_bits / 8, kAlign);
  g.sz_bytes = align_up(T * 2u * (uint64_t)g.ng, kAlign);
  g.slot_bytes[0] = g.codes_bytes[0] + g.sz_bytes;
  g.slot_bytes[1] = g.codes_bytes[1] + g.sz_bytes;
  const uint64_t H = (uint64_t)c.kv_heads, others = (uint64_t)(c.loops_per_group - 1);
  const uint64_t slots = H * (g.slot_bytes[0] + others * g.slot_bytes[1]);
  const bool alpha = c.mode != RQ_MODE_DIRECT;
  g.alpha_row = alpha ? T * 2u : 0;
  g.alpha_block = alpha ? slots : 0;
  g.group_bytes = slots + (alpha ? align_up(others * H * g.alpha_row, kAlign) : 0);
  g.layer_block = (uint64_t)(c.loops / c.loops_per_group) * g.group_bytes;
  g.total = 2ull * (uint64_t)c.batch * (uint64_t)c.layers * g.layer_block;
  return g;
}

}  // namespace rq
