// rq_api.hip -- host side of the C ABI declared in include/rq.h: argument
// validation, cache geometry, split-K planning and kernel launches.  No
// allocation, no synchronization.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/rq.h"
#include "rq_kernels.h"
#include "rq_layout.h"

namespace rq {
int decode_wave_tokens(int d);
int bf16_tile_tokens();

// Split-K planning.  Small batch*heads products are split along the tokens
// until the grid holds about two 4-wave workgroups per CU (512 on 256 CUs)
// for every decode kernel: with the splits merged inside the kernel, fewer
// and longer splits measured faster than filling all workgroup slots (768
// or 1024); the BF16 baseline also targets 512.  Splits never shrink below
// two tiles.  The result is non-decreasing in n_tokens, so a workspace sized
// for n serves any smaller n.
static constexpr int32_t kDecodeTargetTwo = 512;
static constexpr int32_t kDecodeTargetOne = 512;
static constexpr int32_t kDecodeTargetChain = 512;  // chained loops reading 2-3 residual planes
static constexpr int32_t kDecodeTargetWide = 256;   // eight-wave workgroups: one per CU
static constexpr int32_t kGqaTarget = 256;         // grouped-query kernel (eight waves: one per CU)
static constexpr int32_t kDecodeTarget = 512;      // the largest d = 64, 128 target: workspace bound
// d = 96 calls reading at most one residual plane: six of every eight lanes
// hold a group, so the kernel is heavier per byte, and three workgroups per
// CU (768) measured faster than two (Huginn-like shapes: residual call 54.3
// -> 52.4 us; anchor calls gain a little too)
static constexpr int32_t kDecodeTarget96 = 768;
static constexpr int32_t kBf16Target = 512;
// Targets above one workgroup per CU are balanced (see plan_splits).
static constexpr int32_t kOneRound = 256;

static int32_t max_splits_bound(int32_t bh, int32_t n_tokens, int32_t tile, int32_t target) {
  if (n_tokens <= 0 || bh <= 0) return 1;
  const int32_t n_tiles = (n_tokens + tile - 1) / tile;
  // rounded down: a grid of at most `target` workgroups runs in one round
  // (rounding up put 550 workgroups on 512 slots for 110 rows, a second
  // round for 38 of them)
  const int32_t splits = target / bh > 1 ? target / bh : 1;
  const int32_t max_splits = n_tiles / 2 > 1 ? n_tiles / 2 : 1;
  return splits < max_splits ? splits : max_splits;
}

// Whether a balanced plan gives some rows one split more than `s` (the
// rounded-down count): only when s is not capped by the two-tile minimum and
// the rows leave workgroup slots of the target empty.
static bool balances(int32_t bh, int32_t n_tokens, int32_t tile, int32_t target, int32_t s) {
  if (n_tokens <= 0 || bh <= 0 || bh > target || target % bh == 0 || s != target / bh) return false;
  const int32_t n_tiles = (n_tokens + tile - 1) / tile;
  return s + 1 <= n_tiles / 2;
}

// The largest split count of any row in a plan for these sizes (the
// workspace holds that many partial states per row).
static int32_t max_splits_hi(int32_t bh, int32_t n_tokens, int32_t tile, int32_t target, bool balance) {
  const int32_t s = max_splits_bound(bh, n_tokens, tile, target);
  return balance && balances(bh, n_tokens, tile, target, s) ? s + 1 : s;
}

// With `balance` (targets above one workgroup per CU, where several
// workgroups share a CU), rounding the splits down leaves slots empty and
// puts one workgroup more on some CUs than on others: 110 rows at d = 96 took
// 660 workgroups on 768 slots, and the CUs holding three of them set the
// call's time (a 128-row call, 768 workgroups, took 49.4 us against 47.9 us
// for 110 rows: 16 % more bytes in 3 % more time).  A balanced plan gives
// target - rows * s rows one split more, so the grid fills the slots.
SplitPlan plan_splits(int32_t bh, int32_t n_tokens, int32_t tile, int32_t target, bool balance) {
  SplitPlan p{1, tile, 0, 1, tile};
  if (n_tokens <= 0 || bh <= 0) return p;
  const int32_t n_tiles = (n_tokens + tile - 1) / tile;
  auto even = [&](int32_t s, int32_t& splits, int32_t& tps) {
    const int32_t tiles_per = (n_tiles + s - 1) / s;
    tps = tiles_per * tile;
    splits = (n_tokens + tps - 1) / tps;
  };
  const int32_t s = max_splits_bound(bh, n_tokens, tile, target);
  even(s, p.splits, p.tokens_per_split);
  if (balance && balances(bh, n_tokens, tile, target, s)) {
    int32_t sh = 1, th = tile;
    even(s + 1, sh, th);
    if (sh > p.splits) {
      // rows_hi * sh + rows_lo * splits_lo <= target, as sh <= s + 1 and
      // splits_lo <= s
      p.rows_lo = bh - (target - bh * s);
      p.splits_lo = p.splits;
      p.tokens_per_split_lo = p.tokens_per_split;
      p.splits = sh;
      p.tokens_per_split = th;
    }
  }
  return p;
}

}  // namespace rq

using rq::Geometry;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

rq_status check_desc(const rq_cache_desc* d) {
  if (!d) return RQ_ERR_INVALID_ARG;
  if (d->batch <= 0 || d->loops <= 0 || d->layers <= 0 || d->kv_heads <= 0 || d->max_tokens <= 0 ||
      d->head_dim <= 0 || d->loops_per_group <= 0 || d->group_size <= 0)
    return RQ_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 96 && d->head_dim != 128) return RQ_ERR_UNSUPPORTED;
  if (d->group_size != 16) return RQ_ERR_UNSUPPORTED;
  if (d->loops % d->loops_per_group != 0 || d->loops > 64) return RQ_ERR_UNSUPPORTED;
  if ((d->anchor_bits != 2 && d->anchor_bits != 4) || (d->residual_bits != 2 && d->residual_bits != 4))
    return RQ_ERR_UNSUPPORTED;
  if (d->mode != RQ_MODE_RESIDUAL && d->mode != RQ_MODE_DIRECT && d->mode != RQ_MODE_CHAINED)
    return RQ_ERR_UNSUPPORTED;
  // chained mode: the decode kernels read up to three residual planes
  if (d->mode == RQ_MODE_CHAINED &&
      (d->loops_per_group > 4 || d->anchor_bits != 4 || d->residual_bits != 2))
    return RQ_ERR_UNSUPPORTED;
  if (d->alpha_mode != RQ_ALPHA_LS && d->alpha_mode != RQ_ALPHA_NORM_RATIO && d->alpha_mode != RQ_ALPHA_ONE)
    return RQ_ERR_UNSUPPORTED;
  if (d->rotation != RQ_ROT_NONE && d->rotation != RQ_ROT_HADAMARD) return RQ_ERR_UNSUPPORTED;
  // every 64-bit offset must stay far from overflow
  const double total = 2.0 * d->batch * d->loops * (double)d->layers * d->kv_heads *
                       (double)d->max_tokens * (d->head_dim * 0.5 + 2 * d->head_dim / 16.0 + 2.0);
  if (total > 9.0e18) return RQ_ERR_UNSUPPORTED;
  // the decode kernels address one slot with 32-bit buffer offsets
  const double slot = (double)d->max_tokens * (d->head_dim * 0.5 + 2 * d->head_dim / 16.0 + 2.0);
  if (slot > 2.0e9) return RQ_ERR_UNSUPPORTED;
  return RQ_OK;
}

bool needs_signs(const rq_cache_desc* d) {
  return d->mode != RQ_MODE_DIRECT && d->rotation == RQ_ROT_HADAMARD;
}

// A pool descriptor of a paged cache: blocks of max_tokens tokens, a power of
// two no smaller than one wave tile of the decode kernel (so no tile straddles
// two blocks).  Returns log2 of the block size, or -1.
int paged_block_shift(const rq_cache_desc* pool) {
  const int bt = pool->max_tokens;
  if (bt < rq::decode_wave_tokens(pool->head_dim) || (bt & (bt - 1)) != 0) return -1;
  int sh = 0;
  while ((1 << sh) < bt) ++sh;
  return sh;
}

// Shared checks of the paged entry points; fills `pg`.
rq_status check_paged(const rq_cache_desc* pool, int32_t n_seqs, const int32_t* block_table,
                      int32_t max_blocks, rq::Paging& pg) {
  rq_status st = check_desc(pool);
  if (st != RQ_OK) return st;
  const int sh = paged_block_shift(pool);
  if (sh < 0) return RQ_ERR_UNSUPPORTED;
  // the decode kernels reach every plane of a block (all layers of its K or
  // V half) through one buffer resource with 32-bit offsets
  const Geometry g = rq::make_geometry(*pool);
  if ((uint64_t)g.layers * g.layer_block >= (1ull << 32)) return RQ_ERR_UNSUPPORTED;
  if (n_seqs <= 0 || max_blocks <= 0 || !block_table) return RQ_ERR_INVALID_ARG;
  // at most 2^30 tokens per sequence, so token counts rounded up to whole
  // tiles and splits stay far inside int32
  if (((int64_t)max_blocks << sh) > (int64_t)1 << 30) return RQ_ERR_UNSUPPORTED;
  if (!aligned(block_table, 4)) return RQ_ERR_ALIGNMENT;
  pg.table = block_table;
  pg.max_blocks = max_blocks;
  pg.block_shift = sh;
  return RQ_OK;
}

}  // namespace

extern "C" {

const char* rq_status_string(rq_status s) {
  // a C caller may pass any int: read it as one (a value outside the
  // enumeration is not a valid rq_status in C++)
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case RQ_OK: return "ok";
    case RQ_ERR_INVALID_ARG: return "invalid argument";
    case RQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case RQ_ERR_CAPACITY: return "token range exceeds cache capacity";
    case RQ_ERR_WORKSPACE: return "workspace too small";
    case RQ_ERR_ALIGNMENT: return "misaligned device pointer";
    case RQ_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

rq_status rq_validate_desc(const rq_cache_desc* desc) { return check_desc(desc); }

rq_status rq_cache_bytes(const rq_cache_desc* desc, uint64_t* total_bytes) {
  rq_status st = check_desc(desc);
  if (st != RQ_OK) return st;
  if (!total_bytes) return RQ_ERR_INVALID_ARG;
  *total_bytes = rq::make_geometry(*desc).total;
  return RQ_OK;
}

rq_status rq_cache_layout(const rq_cache_desc* desc, rq_layout* out) {
  rq_status st = check_desc(desc);
  if (st != RQ_OK) return st;
  if (!out) return RQ_ERR_INVALID_ARG;
  const Geometry g = rq::make_geometry(*desc);
  out->total_bytes = g.total;
  out->layer_bytes = g.layer_block;
  out->group_bytes = g.group_bytes;
  for (int k = 0; k < 2; ++k) {
    out->slot_bytes[k] = g.slot_bytes[k];
    out->sz_offset[k] = g.codes_bytes[k];
    out->code_row_bytes[k] = desc->head_dim * (k == 0 ? desc->anchor_bits : desc->residual_bits) / 8;
  }
  out->alpha_offset = g.alpha_row ? g.alpha_block : UINT64_MAX;
  out->alpha_row_bytes = g.alpha_row;
  out->sz_row_bytes = 2 * desc->head_dim / 16;
  out->token_tile = rq::decode_wave_tokens(desc->head_dim);
  return RQ_OK;
}

rq_status rq_cache_slot(const rq_cache_desc* desc, int32_t kv, int32_t batch, int32_t layer,
                        int32_t loop, int32_t kv_head, rq_slot* out) {
  rq_status st = check_desc(desc);
  if (st != RQ_OK) return st;
  if (!out || kv < 0 || kv > 1 || batch < 0 || batch >= desc->batch || layer < 0 ||
      layer >= desc->layers || loop < 0 || loop >= desc->loops || kv_head < 0 ||
      kv_head >= desc->kv_heads)
    return RQ_ERR_INVALID_ARG;
  const Geometry g = rq::make_geometry(*desc);
  const uint64_t off = g.slot_offset(kv, batch, layer, loop, kv_head);
  out->codes_offset = off;
  out->sz_offset = off + g.sz_rel(loop);
  out->alpha_offset = g.has_alpha(loop) ? g.alpha_offset(kv, batch, layer, loop, kv_head) : UINT64_MAX;
  out->slot_bytes = g.slot_bytes[g.is_anchor(loop) ? 0 : 1];
  out->bits = g.bits_of(loop);
  out->code_bytes = desc->head_dim * out->bits / 8;
  return RQ_OK;
}

static rq_status quantize_append_impl(const rq_cache_desc* desc, void* cache, const uint16_t* kv_bf16,
                                      int32_t n_tokens, const int32_t* positions, int32_t t_new,
                                      const int8_t* signs, void* stream, int32_t rows,
                                      rq::Paging pg) {
  if (t_new == 0) return RQ_OK;
  if (!cache || !kv_bf16 || (needs_signs(desc) && !signs)) return RQ_ERR_INVALID_ARG;
  if (!aligned(cache, 256) || !aligned(kv_bf16, 4) || !aligned(positions, 4)) return RQ_ERR_ALIGNMENT;
  rq::QuantArgs a{};
  a.g = rq::make_geometry(*desc);
  a.cache = static_cast<uint8_t*>(cache);
  a.kv = kv_bf16;
  a.signs = signs;
  a.n_tokens = n_tokens;
  a.t_new = t_new;
  a.positions = positions;
  a.rows = rows;
  a.paging = pg;
  a.items = 2ull * rows * desc->layers * desc->kv_heads *
            (uint64_t)(desc->loops / desc->loops_per_group) * (uint64_t)t_new;
  return rq::launch_quant_append(a, static_cast<hipStream_t>(stream)) == hipSuccess ? RQ_OK
                                                                                      : RQ_ERR_LAUNCH;
}

rq_status rq_quantize_append(const rq_cache_desc* desc, void* cache, const uint16_t* kv_bf16,
                             int32_t n_tokens, int32_t t_new, const int8_t* signs, void* stream) {
  rq_status st = check_desc(desc);
  if (st != RQ_OK) return st;
  if (n_tokens < 0 || t_new < 0) return RQ_ERR_INVALID_ARG;
  if ((int64_t)n_tokens + t_new > desc->max_tokens) return RQ_ERR_CAPACITY;
  return quantize_append_impl(desc, cache, kv_bf16, n_tokens, nullptr, t_new, signs, stream,
                              desc->batch, rq::Paging{});
}

rq_status rq_quantize_append_ragged(const rq_cache_desc* desc, void* cache, const uint16_t* kv_bf16,
                                    const int32_t* positions, int32_t t_new, const int8_t* signs,
                                    void* stream) {
  rq_status st = check_desc(desc);
  if (st != RQ_OK) return st;
  if (t_new < 0) return RQ_ERR_INVALID_ARG;
  if (t_new > desc->max_tokens) return RQ_ERR_CAPACITY;
  if (t_new > 0 && !positions) return RQ_ERR_INVALID_ARG;
  return quantize_append_impl(desc, cache, kv_bf16, 0, positions, t_new, signs, stream, desc->batch,
                              rq::Paging{});
}

rq_status rq_paged_quantize_append(const rq_cache_desc* pool, void* cache, const uint16_t* kv_bf16,
                                   int32_t n_seqs, const int32_t* block_table,
                                   int32_t max_blocks_per_seq, const int32_t* positions,
                                   int32_t t_new, const int8_t* signs, void* stream) {
  rq::Paging pg{};
  rq_status st = check_paged(pool, n_seqs, block_table, max_blocks_per_seq, pg);
  if (st != RQ_OK) return st;
  if (t_new < 0) return RQ_ERR_INVALID_ARG;
  if ((int64_t)t_new > ((int64_t)max_blocks_per_seq << pg.block_shift)) return RQ_ERR_CAPACITY;
  if (t_new > 0 && !positions) return RQ_ERR_INVALID_ARG;
  return quantize_append_impl(pool, cache, kv_bf16, 0, positions, t_new, signs, stream, n_seqs, pg);
}

rq_status rq_reconstruct(const rq_cache_desc* desc, const void* cache, const int8_t* signs,
                         int32_t tok_begin, int32_t tok_end, int32_t out_dtype, void* out,
                         void* stream) {
  rq_status st = check_desc(desc);
  if (st != RQ_OK) return st;
  if (tok_begin < 0 || tok_end < tok_begin) return RQ_ERR_INVALID_ARG;
  if (tok_end > desc->max_tokens) return RQ_ERR_CAPACITY;
  if (out_dtype != RQ_OUT_F32 && out_dtype != RQ_OUT_BF16) return RQ_ERR_INVALID_ARG;
  if (tok_end == tok_begin) return RQ_OK;
  if (!cache || !out || (needs_signs(desc) && !signs)) return RQ_ERR_INVALID_ARG;
  if (!aligned(cache, 256) || !aligned(out, 4)) return RQ_ERR_ALIGNMENT;
  rq::ReconArgs a{};
  a.g = rq::make_geometry(*desc);
  a.cache = static_cast<const uint8_t*>(cache);
  a.signs = signs;
  a.tok_begin = tok_begin;
  a.n_out = tok_end - tok_begin;
  a.out_bf16 = out_dtype == RQ_OUT_BF16;
  a.out = out;
  a.vectors = 2ull * desc->batch * desc->loops * desc->layers * desc->kv_heads * (uint64_t)a.n_out;
  return rq::launch_reconstruct(a, static_cast<hipStream_t>(stream)) == hipSuccess ? RQ_OK
                                                                                    : RQ_ERR_LAUNCH;
}

// The workspace starts with a fixed block of split-arrival counters, one per
// (row, query head), so that calls of any shape find them at the same place
// and never overlap another call's partial states; the partial states follow.
static constexpr int32_t kMaxRowHeads = 1 << 16;  // also the grid's y extent
static constexpr uint64_t kCounterBytes = (uint64_t)kMaxRowHeads * 4u;

// Whether a call runs the grouped-query kernel (one workgroup per KV head);
// its split plan then counts (batch row, KV head) rows.
static bool grouped(const rq_cache_desc* desc, int32_t loop, int32_t q_heads) {
  return q_heads % desc->kv_heads == 0 &&
         rq::gqa_supported(rq::make_geometry(*desc), loop, q_heads / desc->kv_heads);
}

static uint64_t workspace_for(const rq_cache_desc* desc, int32_t rows, int32_t q_heads,
                              int32_t max_n_tokens) {
  if (check_desc(desc) != RQ_OK || q_heads <= 0 || rows <= 0) return 0;
  const int32_t bh = rows * q_heads;
  // four-wave tiles at the largest target bound the eight-wave plans too
  int32_t s = rq::max_splits_hi(bh, max_n_tokens, rq::decode_tile_tokens(desc->head_dim, 4),
                                desc->head_dim == 96 ? rq::kDecodeTarget96 : rq::kDecodeTarget, true);
  bool any_grouped = false;
  for (int32_t loop = 0; loop < desc->loops_per_group; ++loop)
    any_grouped = any_grouped || grouped(desc, loop, q_heads);
  if (any_grouped) {
    const int32_t sg = rq::max_splits_bound(rows * desc->kv_heads, max_n_tokens,
                                            rq::gqa_tile_tokens(), rq::kGqaTarget);
    s = sg > s ? sg : s;
  }
  return s > 1 ? kCounterBytes + (uint64_t)bh * s * (2 + 2 * desc->head_dim) * 4ull : 0;
}

uint64_t rq_decode_workspace_bytes(const rq_cache_desc* desc, int32_t q_heads, int32_t max_n_tokens) {
  return check_desc(desc) == RQ_OK ? workspace_for(desc, desc->batch, q_heads, max_n_tokens) : 0;
}

uint64_t rq_paged_decode_workspace_bytes(const rq_cache_desc* pool, int32_t q_heads, int32_t n_seqs,
                                         int32_t max_n_tokens) {
  return workspace_for(pool, n_seqs, q_heads, max_n_tokens);
}

// The split plan of one decode call and the per-head kernel's waves per
// workgroup (the grouped kernel's plan counts (row, KV head) pairs).
static rq::SplitPlan decode_plan(const rq_cache_desc* desc, int32_t rows, int32_t loop,
                                 int32_t q_heads, int32_t n_tokens, bool paged, int* waves) {
  const int j = loop % desc->loops_per_group, a_pos = desc->loops_per_group - 1;
  const bool two = desc->mode != RQ_MODE_DIRECT && j != a_pos;
  const bool chain = desc->mode == RQ_MODE_CHAINED && a_pos - j > 1;  // several residual planes
  *waves = rq::decode_waves(desc->head_dim, chain, paged, two);
  const int32_t target = *waves == 8            ? rq::kDecodeTargetWide
                         : chain                  ? rq::kDecodeTargetChain
                         : desc->head_dim == 96   ? rq::kDecodeTarget96
                         : two                    ? rq::kDecodeTargetTwo
                                                  : rq::kDecodeTargetOne;
  if (grouped(desc, loop, q_heads))
    return rq::plan_splits(rows * desc->kv_heads, n_tokens, rq::gqa_tile_tokens(), rq::kGqaTarget,
                           false);
  return rq::plan_splits(rows * q_heads, n_tokens, rq::decode_tile_tokens(desc->head_dim, *waves),
                         target, target > rq::kOneRound);
}

int32_t rq_decode_splits(const rq_cache_desc* desc, int32_t loop, int32_t q_heads, int32_t n_tokens) {
  if (check_desc(desc) != RQ_OK || loop < 0 || loop >= desc->loops || q_heads <= 0 ||
      q_heads % desc->kv_heads != 0 || n_tokens < 0)
    return 0;
  int waves = 4;
  return decode_plan(desc, desc->batch, loop, q_heads, n_tokens, false, &waves).splits;
}

static rq_status decode_attention_impl(const rq_cache_desc* desc, const void* cache,
                                       const int8_t* signs, int32_t loop, int32_t layer,
                                       const uint16_t* q_bf16, int32_t q_heads, int32_t n_tokens,
                                       const int32_t* lengths, float softmax_scale, void* workspace,
                                       uint64_t workspace_bytes, float* out, void* stream,
                                       int32_t rows, rq::Paging pg) {
  rq_status st = check_desc(desc);
  if (st != RQ_OK) return st;
  if (loop < 0 || loop >= desc->loops || layer < 0 || layer >= desc->layers || q_heads <= 0 ||
      n_tokens < 0)
    return RQ_ERR_INVALID_ARG;
  if (q_heads % desc->kv_heads != 0) return RQ_ERR_UNSUPPORTED;
  if ((int64_t)rows * q_heads > kMaxRowHeads) return RQ_ERR_UNSUPPORTED;
  const int64_t cap = pg.table ? ((int64_t)pg.max_blocks << pg.block_shift) : desc->max_tokens;
  if (n_tokens > cap) return RQ_ERR_CAPACITY;
  const uint64_t need = workspace_for(desc, rows, q_heads, n_tokens);
  if (!cache || !q_bf16 || !out || (needs_signs(desc) && !signs) || (need && !workspace))
    return RQ_ERR_INVALID_ARG;
  if (!aligned(cache, 256) || !aligned(workspace, 256) || !aligned(q_bf16, 4) || !aligned(out, 4) ||
      !aligned(lengths, 4))
    return RQ_ERR_ALIGNMENT;
  if (!(softmax_scale == softmax_scale)) return RQ_ERR_INVALID_ARG;
  if (workspace_bytes < need) return RQ_ERR_WORKSPACE;
  int waves = 4;
  const rq::SplitPlan plan = decode_plan(desc, rows, loop, q_heads, n_tokens, pg.table != nullptr, &waves);
  // workspace_for bounds every plan; a plan past it would write partials
  // beyond the caller's buffer, so refuse rather than launch
  const uint64_t used = plan.splits > 1 ? kCounterBytes + (uint64_t)rows * q_heads * plan.splits *
                                                             (2 + 2 * desc->head_dim) * 4ull
                                        : 0;
  if (used > workspace_bytes) return RQ_ERR_WORKSPACE;
  rq::DecodeArgs a{};
  a.g = rq::make_geometry(*desc);
  a.cache = static_cast<const uint8_t*>(cache);
  a.signs = signs;
  a.q = q_bf16;
  a.out = out;
  a.counters = static_cast<uint32_t*>(workspace);
  a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kCounterBytes);
  a.lengths = lengths;
  a.rows = rows;
  a.paging = pg;
  a.loop = loop;
  a.layer = layer;
  a.q_heads = q_heads;
  a.group_ratio = q_heads / desc->kv_heads;
  a.n_tokens = n_tokens;
  a.splits = plan.splits;
  a.tokens_per_split = plan.tokens_per_split;
  a.rows_lo = plan.rows_lo;
  a.splits_lo = plan.splits_lo;
  a.tokens_per_split_lo = plan.tokens_per_split_lo;
  a.qscale = softmax_scale * 1.4426950408889634f;
  a.waves = waves;
  return rq::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? RQ_OK : RQ_ERR_LAUNCH;
}

rq_status rq_decode_attention(const rq_cache_desc* desc, const void* cache, const int8_t* signs,
                              int32_t loop, int32_t layer, const uint16_t* q_bf16, int32_t q_heads,
                              int32_t n_tokens, float softmax_scale, void* workspace,
                              uint64_t workspace_bytes, float* out, void* stream) {
  return decode_attention_impl(desc, cache, signs, loop, layer, q_bf16, q_heads, n_tokens, nullptr,
                               softmax_scale, workspace, workspace_bytes, out, stream, desc->batch,
                               rq::Paging{});
}

}  // extern "C"

// ---- rq_decode_attention_noalloc: the split-K workspace is this file-scope
// device array (one per GPU, held until the process ends).  Its first
// kCounterBytes are the split counters, which must start at zero; every call
// leaves them at zero.  In host code `scratch` names a host-side stand-in:
// only the address from hipGetSymbolAddress, kept per device, is passed to
// kernels or copies.
static constexpr uint64_t kScratchBytes = 2ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
bool g_scratch_zeroed[kMaxDevices];

// The current device's scratch address; the first call on a device also
// clears the counter block with a kernel on `stream` (ahead of the decode
// kernel on the same stream).  Returns nullptr on a HIP error.
void* scratch_for_current_device(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  if (!g_scratch_zeroed[dev]) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream,
                       static_cast<uint32_t*>(g_scratch_ptr[dev]), (uint32_t)(kCounterBytes / 4));
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch_zeroed[dev] = true;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

rq_status rq_decode_attention_noalloc(const rq_cache_desc* desc, const void* cache,
                                      const int8_t* signs, int32_t loop, int32_t layer,
                                      const uint16_t* q_bf16, int32_t q_heads, int32_t n_tokens,
                                      float softmax_scale, float* out, void* stream) {
  // the same argument checks as rq_decode_attention, and the size limit,
  // before anything touches the device
  rq_status st = check_desc(desc);
  if (st != RQ_OK) return st;
  if (q_heads <= 0 || n_tokens < 0) return RQ_ERR_INVALID_ARG;
  if (q_heads % desc->kv_heads != 0) return RQ_ERR_UNSUPPORTED;
  if ((int64_t)desc->batch * q_heads > kMaxRowHeads) return RQ_ERR_UNSUPPORTED;
  if (loop < 0 || loop >= desc->loops || layer < 0 || layer >= desc->layers) return RQ_ERR_INVALID_ARG;
  if (n_tokens > desc->max_tokens) return RQ_ERR_CAPACITY;
  const uint64_t need = workspace_for(desc, desc->batch, q_heads, n_tokens);
  if (need > kScratchBytes) return RQ_ERR_WORKSPACE;
  if (!cache || !q_bf16 || !out || (needs_signs(desc) && !signs)) return RQ_ERR_INVALID_ARG;
  if (!aligned(cache, 256) || !aligned(q_bf16, 4) || !aligned(out, 4)) return RQ_ERR_ALIGNMENT;
  if (!(softmax_scale == softmax_scale)) return RQ_ERR_INVALID_ARG;
  void* ws = scratch_for_current_device(static_cast<hipStream_t>(stream));
  if (!ws) return RQ_ERR_LAUNCH;
  return decode_attention_impl(desc, cache, signs, loop, layer, q_bf16, q_heads, n_tokens, nullptr,
                               softmax_scale, ws, kScratchBytes, out, stream, desc->batch,
                               rq::Paging{});
}

rq_status rq_decode_attention_ragged(const rq_cache_desc* desc, const void* cache,
                                     const int8_t* signs, int32_t loop, int32_t layer,
                                     const uint16_t* q_bf16, int32_t q_heads, const int32_t* lengths,
                                     int32_t max_n_tokens, float softmax_scale, void* workspace,
                                     uint64_t workspace_bytes, float* out, void* stream) {
  if (!lengths) return RQ_ERR_INVALID_ARG;
  return decode_attention_impl(desc, cache, signs, loop, layer, q_bf16, q_heads, max_n_tokens,
                               lengths, softmax_scale, workspace, workspace_bytes, out, stream,
                               desc->batch, rq::Paging{});
}

rq_status rq_paged_decode_attention(const rq_cache_desc* pool, const void* cache,
                                    const int8_t* signs, int32_t loop, int32_t layer,
                                    const uint16_t* q_bf16, int32_t q_heads, int32_t n_seqs,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    const int32_t* lengths, int32_t max_n_tokens,
                                    float softmax_scale, void* workspace, uint64_t workspace_bytes,
                                    float* out, void* stream) {
  rq::Paging pg{};
  rq_status st = check_paged(pool, n_seqs, block_table, max_blocks_per_seq, pg);
  if (st != RQ_OK) return st;
  if (!lengths) return RQ_ERR_INVALID_ARG;
  return decode_attention_impl(pool, cache, signs, loop, layer, q_bf16, q_heads, max_n_tokens,
                               lengths, softmax_scale, workspace, workspace_bytes, out, stream,
                               n_seqs, pg);
}

uint64_t rq_bf16_decode_workspace_bytes(const rq_cache_desc* desc, int32_t q_heads,
                                        int32_t max_n_tokens) {
  if (check_desc(desc) != RQ_OK || q_heads <= 0) return 0;
  const int32_t bh = desc->batch * q_heads;
  const int32_t s = rq::max_splits_bound(bh, max_n_tokens, rq::bf16_tile_tokens(), rq::kBf16Target);
  return s > 1 ? (uint64_t)bh * s * (2 + desc->head_dim) * 4ull : 0;
}

rq_status rq_bf16_decode_attention(const rq_cache_desc* desc, const uint16_t* k_cache,
                                   const uint16_t* v_cache, int32_t loop, int32_t layer,
                                   const uint16_t* q_bf16, int32_t q_heads, int32_t n_tokens,
                                   float softmax_scale, void* workspace, uint64_t workspace_bytes,
                                   float* out, void* stream) {
  rq_status st = check_desc(desc);
  if (st != RQ_OK) return st;
  if (loop < 0 || loop >= desc->loops || layer < 0 || layer >= desc->layers || q_heads <= 0 ||
      n_tokens < 0)
    return RQ_ERR_INVALID_ARG;
  if (q_heads % desc->kv_heads != 0) return RQ_ERR_UNSUPPORTED;
  if (n_tokens > desc->max_tokens) return RQ_ERR_CAPACITY;
  const uint64_t need = rq_bf16_decode_workspace_bytes(desc, q_heads, n_tokens);
  if (!k_cache || !v_cache || !q_bf16 || !out || (need && !workspace)) return RQ_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(workspace, 256) ||
      !aligned(q_bf16, 4) || !aligned(out, 4))
    return RQ_ERR_ALIGNMENT;
  if (workspace_bytes < need) return RQ_ERR_WORKSPACE;
  const int32_t bh = desc->batch * q_heads;
  const rq::SplitPlan plan = rq::plan_splits(bh, n_tokens, rq::bf16_tile_tokens(), rq::kBf16Target, false);
  if (plan.splits > 1 && (uint64_t)bh * plan.splits * (2 + desc->head_dim) * 4ull > workspace_bytes)
    return RQ_ERR_WORKSPACE;
  rq::Bf16DecodeArgs a{};
  a.batch = desc->batch;
  a.loops = desc->loops;
  a.layers = desc->layers;
  a.kv_heads = desc->kv_heads;
  a.max_tokens = desc->max_tokens;
  a.d = desc->head_dim;
  a.k = k_cache;
  a.v = v_cache;
  a.q = q_bf16;
  a.out = out;
  a.partials = static_cast<float*>(workspace);
  a.loop = loop;
  a.layer = layer;
  a.q_heads = q_heads;
  a.group_ratio = q_heads / desc->kv_heads;
  a.n_tokens = n_tokens;
  a.splits = plan.splits;
  a.tokens_per_split = plan.tokens_per_split;
  a.qscale = softmax_scale * 1.4426950408889634f;
  return rq::launch_bf16_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? RQ_OK
                                                                                   : RQ_ERR_LAUNCH;
}

uint32_t rq_read_probe_sink_words(void) { return rq::kProbeBlocks; }

rq_status rq_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16) return RQ_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return RQ_ERR_ALIGNMENT;
  return rq::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)) == hipSuccess
             ? RQ_OK
             : RQ_ERR_LAUNCH;
}

}  // extern "C"
