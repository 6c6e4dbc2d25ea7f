// rq_kernels.h -- argument blocks and launchers of the library's kernels
// (internal; the public interface is include/rq.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq_layout.h"

namespace rq {

// Paged cache (vLLM-style block tables): the descriptor describes a pool whose
// "batch" rows are physical blocks of max_tokens = 2^block_shift tokens, and
// row r's logical token t lives at token t & (2^block_shift - 1) of block
// table[r * max_blocks + (t >> block_shift)].  table == null: not paged.
struct Paging {
  const int32_t* table;
  int32_t max_blocks, block_shift;
};

struct QuantArgs {
  Geometry g;
  uint8_t* cache;
  const uint16_t* kv;     // [2][B][L][layers][H][t_new][d] BF16
  const int8_t* signs;    // [2][layers][d]
  int32_t n_tokens, t_new;
  const int32_t* positions;  // [rows] first position per row, or null (all at n_tokens)
  uint64_t items;         // 2*rows*layers*H*(L/P)*t_new
  int32_t rows;           // batch rows of kv (the descriptor's batch unless paged)
  Paging paging;
};
hipError_t launch_quant_append(const QuantArgs& a, hipStream_t s);

struct ReconArgs {
  Geometry g;
  const uint8_t* cache;
  const int8_t* signs;
  int32_t tok_begin, n_out;
  int32_t out_bf16;
  void* out;              // [2][B][L][layers][H][n_out][d]
  uint64_t vectors;       // 2*B*L*layers*H*n_out
};
hipError_t launch_reconstruct(const ReconArgs& a, hipStream_t s);

// Split-K decode: with more than one split, partial states live in the
// workspace, and the workgroup that finishes a row last (by a ticket counter
// per row, also in the workspace) merges them.
struct DecodeArgs {
  Geometry g;
  const uint8_t* cache;
  const int8_t* signs;
  const uint16_t* q;      // [B][Hq][d]
  float* out;             // [B][Hq][d]
  float* partials;        // [B*Hq][splits][2 + 2d]
  uint32_t* counters;     // [B*Hq] split arrivals, zero between calls
  const int32_t* lengths;  // [rows] tokens per row (clamped to n_tokens), or null
  int32_t rows;           // query rows (the descriptor's batch unless paged)
  Paging paging;
  int32_t loop, layer, q_heads, group_ratio, n_tokens;
  int32_t splits, tokens_per_split;
  // per-head kernel: the first rows_lo rows take splits_lo splits of
  // tokens_per_split_lo tokens, the others `splits` of tokens_per_split
  // (partials keep the stride `splits`); the grouped kernel leaves rows_lo 0
  int32_t rows_lo, splits_lo, tokens_per_split_lo;
  float qscale;           // softmax scale * log2(e)
  int32_t waves;          // per-head kernel: waves per workgroup (decode_waves)
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// per-head kernel geometry, shared by the split plan and the launch
int decode_waves(int d, bool several_planes, bool paged, bool residual);
int decode_tile_tokens(int d, int waves);
// grouped-query decode on matrix cores: one workgroup per (split, batch row,
// KV head) serves the group_ratio query heads of the KV head
bool gqa_supported(const Geometry& g, int loop, int group_ratio);
hipError_t launch_gqa(const DecodeArgs& a, hipStream_t s);
int gqa_tile_tokens();

struct Bf16DecodeArgs {
  int32_t batch, loops, layers, kv_heads, max_tokens, d;
  const uint16_t* k;      // [B][L][layers][H][max_tokens][d]
  const uint16_t* v;
  const uint16_t* q;
  float* out;
  float* partials;        // [B*Hq][splits][2 + d]
  int32_t loop, layer, q_heads, group_ratio, n_tokens;
  int32_t splits, tokens_per_split;
  float qscale;
};
hipError_t launch_bf16_decode(const Bf16DecodeArgs& a, hipStream_t s);

constexpr uint32_t kProbeBlocks = 1024;
hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s);

// Split-K partition shared by workspace sizing and the launch.  A balanced
// plan gives the first rows_lo rows one split fewer (splits_lo of
// tokens_per_split_lo tokens), so that the grid holds the target number of
// workgroups exactly; otherwise rows_lo is 0.
struct SplitPlan {
  int32_t splits;
  int32_t tokens_per_split;
  int32_t rows_lo, splits_lo, tokens_per_split_lo;
  int64_t workgroups(int32_t bh) const {
    return (int64_t)rows_lo * splits_lo + (int64_t)(bh - rows_lo) * splits;
  }
};
SplitPlan plan_splits(int32_t bh, int32_t n_tokens, int32_t tile_tokens, int32_t target_blocks,
                      bool balance);

}  // namespace rq
