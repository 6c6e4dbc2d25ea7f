// rq_layout.h -- cache geometry shared by the host entry points and the kernels.
//
// A cache is a sequence of slots ordered (kv, batch, layer, loop, kv_head),
// outermost first.  Within a (kv, batch, layer) block the loops of one loop
// group are consecutive and the anchor (last loop of the group) comes last.
// Each slot is: codes [max_tokens][d*bits/8] | sz [max_tokens][2*d/16] |
// alpha [max_tokens] (BF16; residual slots of residual mode only), each
// sub-plane starting on a 256-byte boundary.
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
  uint64_t alpha_bytes;       // 0 when other slots carry no alpha plane
  uint64_t slot_bytes[2];
  uint64_t group_bytes;       // one loop group of one head: anchor + (P-1) others
  uint64_t layer_block;       // one (kv, batch, layer) block
  uint64_t total;

  RQ_HD bool is_anchor(int loop) const { return loop % P == P - 1; }
  RQ_HD int bits_of(int loop) const { return is_anchor(loop) ? anchor_bits : residual_bits; }
  RQ_HD bool has_alpha(int loop) const { return mode != RQ_MODE_DIRECT && !is_anchor(loop); }

  // Byte offset of the codes sub-plane of a slot.
  RQ_HD uint64_t slot_offset(int kv, int b, int layer, int loop, int head) const {
    const int k = loop / P, j = loop % P;
    const uint64_t sb = slot_bytes[j == P - 1 ? 0 : 1];
    return ((uint64_t)(kv * batch + b) * layers + layer) * layer_block +
           (uint64_t)kv_heads * ((uint64_t)k * group_bytes + (uint64_t)j * slot_bytes[1]) +
           (uint64_t)head * sb;
  }
  RQ_HD uint64_t sz_rel(int loop) const { return codes_bytes[is_anchor(loop) ? 0 : 1]; }
  RQ_HD uint64_t alpha_rel(int loop) const { return codes_bytes[1] + sz_bytes; }
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
  g.alpha_bytes = (c.mode != RQ_MODE_DIRECT) ? align_up(T * 2u, kAlign) : 0;
  g.slot_bytes[0] = g.codes_bytes[0] + g.sz_bytes;
  g.slot_bytes[1] = g.codes_bytes[1] + g.sz_bytes + g.alpha_bytes;
  g.group_bytes = g.slot_bytes[0] + (uint64_t)(c.loops_per_group - 1) * g.slot_bytes[1];
  g.layer_block = (uint64_t)c.kv_heads * (uint64_t)(c.loops / c.loops_per_group) * g.group_bytes;
  g.total = 2ull * (uint64_t)c.batch * (uint64_t)c.layers * g.layer_block;
  return g;
}

}  // namespace rq
