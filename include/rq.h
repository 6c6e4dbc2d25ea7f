/*
 * rq.h -- C ABI of librq, an MI355X (gfx950) implementation of the
 * ResidualQuant KV cache for looped Transformers: per-loop-group
 * quantize-and-append, reconstruction, and fused decode attention that reads
 * the packed cache directly.
 *
 * The method (web pages about "ResidualQuant: KV Cache Quantization for Looped
 * Transformers with 2-Bit Residuals"; arXiv abstract, ai4snews summary
 * paragraphs 1-4, agihunt "Confirmed" list):
 *   - each loop of a looped Transformer keeps its own K/V per layer, so the KV
 *     cache grows with the loop count (abstract);
 *   - within a loop group, the final loop's state is the anchor, stored at
 *     INT4; every other loop stores only its INT2 residual against the
 *     dequantized anchor (ai4snews para. 1; agihunt);
 *   - the residual is rotated by a fixed orthogonal matrix before
 *     quantization (the anchor is not rotated) and carries a BF16
 *     least-squares scale alpha; every group of 16 head_dim values has an FP8
 *     scale and offset (ai4snews paras. 1-2);
 *   - any loop is reconstructed from two reads, the anchor and its own
 *     residual (ai4snews para. 3).
 * The rotation is a randomized Walsh-Hadamard transform
 * H = (1/sqrt(d)) WHT_d diag(signs) (d = 96: block diagonal 64 + 32).
 *
 * Conventions for every call:
 *   - All buffers except `desc` and `out` structs are DEVICE pointers owned by
 *     the caller.  The library never allocates, frees or synchronizes; work is
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns before it completes.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-RQ_OK status means nothing was enqueued, except RQ_ERR_LAUNCH, which
 *     reports a failed kernel launch (later kernels of the same call are not
 *     enqueued).  Statuses are never thrown across the ABI.
 *   - The library is stateless: the caller tracks how many tokens are cached.
 *
 * Cache descriptor and supported values:
 *   head_dim 64, 96 or 128; group_size 16; loops % loops_per_group == 0;
 *   anchor_bits and residual_bits each 2 or 4; mode RESIDUAL, DIRECT or
 *   CHAINED (CHAINED: anchor 4 bits, residuals 2 bits, loops_per_group <= 4);
 *   alpha_mode LS, NORM_RATIO or ONE; rotation HADAMARD or NONE;
 *   1 <= batch, layers, kv_heads; 1 <= loops <= 64; 1 <= max_tokens, and one
 *   slot (below) at most 2e9 bytes.
 *
 * Modes.  RESIDUAL is the method: every non-anchor loop stores its residual
 * against the dequantized anchor, so any loop is rebuilt from two reads.
 * DIRECT stores every loop on its own (the comparison without residuals).
 * CHAINED is the ablation's previous-loop reference (ai4snews para. 3):
 * loop l < anchor stores its residual against the reconstruction of loop
 * l + 1, the anchor ending the chain, so loop j is rebuilt from the anchor and
 * the residuals of loops j .. anchor - 1 (distance + 1 reads); its rotated
 * residual is computed as H (x_l - deq(anchor)) - sum alpha_i yhat_i over
 * i = anchor-1 down to l+1.
 *
 * Byte layout of a cache buffer (little endian).  A "slot" holds one
 * (kv, batch row, layer, loop, kv head) stream of max_tokens tokens, where
 * kv = 0 is K and kv = 1 is V.  Slot order, outermost first:
 *     kv, batch, layer, loop, kv_head
 * Loop j of loop group k (j = loop % P, P = loops_per_group) is the group's
 * anchor when j == P-1.  Its bit width is anchor_bits for the anchor and
 * residual_bits otherwise (direct mode: the anchor-position loop is stored at
 * anchor_bits, the others at residual_bits, all as plain quantized states).
 * A slot is two sub-planes, each starting on a 256-byte boundary:
 *     codes [max_tokens][d*bits/8]  element i of a token is in byte i*bits/8,
 *                                   at bit (i*bits) % 8 (low bits first)
 *     sz    [max_tokens][2*d/16]    byte 2g = FP8 e4m3fn scale of group g,
 *                                   byte 2g+1 = FP8 e4m3fn offset of group g
 * In RESIDUAL and CHAINED modes each non-anchor (loop, kv head) also has an
 * alpha row, [max_tokens] uint16 BF16 coefficients; the rows of one loop
 * group follow the group's slots as one block, padded to 256 bytes as a
 * whole (see rq_layout).
 * A dequantized group value is scale * code + offset.  Slot sizes and
 * offsets are given by rq_cache_slot(); the total by rq_cache_bytes().
 */
#ifndef RQ_H
#define RQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RQ_OK = 0,
  RQ_ERR_INVALID_ARG = 1, /* null pointer, bad index or negative size */
  RQ_ERR_UNSUPPORTED = 2, /* well-formed descriptor outside the supported set */
  RQ_ERR_CAPACITY = 3,    /* token range exceeds max_tokens */
  RQ_ERR_WORKSPACE = 4,   /* workspace smaller than rq_*_workspace_bytes() */
  RQ_ERR_ALIGNMENT = 5,   /* a device pointer is not aligned as required */
  RQ_ERR_LAUNCH = 6       /* the HIP runtime refused a kernel launch */
} rq_status;

enum { RQ_MODE_RESIDUAL = 0, RQ_MODE_DIRECT = 1, RQ_MODE_CHAINED = 2 };
enum { RQ_ALPHA_LS = 0, RQ_ALPHA_NORM_RATIO = 1, RQ_ALPHA_ONE = 2 };
enum { RQ_ROT_NONE = 0, RQ_ROT_HADAMARD = 1 };
enum { RQ_OUT_F32 = 0, RQ_OUT_BF16 = 1 };

typedef struct rq_cache_desc {
  int32_t batch;
  int32_t loops;           /* total loops L */
  int32_t layers;
  int32_t kv_heads;
  int32_t max_tokens;      /* capacity per slot */
  int32_t head_dim;        /* d */
  int32_t loops_per_group; /* P; the anchor is loop P-1 of each group */
  int32_t anchor_bits;
  int32_t residual_bits;
  int32_t group_size;      /* must be 16 */
  int32_t mode;            /* RQ_MODE_* */
  int32_t alpha_mode;      /* RQ_ALPHA_* (RESIDUAL mode) */
  int32_t rotation;        /* RQ_ROT_* (RESIDUAL mode) */
} rq_cache_desc;

typedef struct rq_slot {
  uint64_t codes_offset; /* bytes from the start of the cache buffer */
  uint64_t sz_offset;
  uint64_t alpha_offset; /* the slot's alpha row; UINT64_MAX when it has none */
  uint64_t slot_bytes;   /* bytes from codes_offset to the next slot */
  int32_t bits;          /* code width of this slot */
  int32_t code_bytes;    /* bytes per token in the codes sub-plane */
} rq_slot;

/* The whole byte layout of a cache for one descriptor, so a caller can
 * address any slot without further calls (host only).  With P =
 * loops_per_group, loop = k * P + j (group k, position j; j == P - 1 is the
 * anchor), kind = (j == P - 1 ? 0 : 1) and
 *     base = ((kv * batch + b) * layers + layer) * layer_bytes + k * group_bytes,
 * the slot of (kv, batch row b, layer, loop, kv_head h) starts at
 *     base + j * kv_heads * slot_bytes[1] + h * slot_bytes[kind]
 * and its sub-planes at that offset + 0 (codes) and + sz_offset[kind] (FP8
 * scale/offset pairs).  In RESIDUAL and CHAINED modes the BF16 alpha row of
 * a non-anchor (loop, h) starts at
 *     base + alpha_offset + (j * kv_heads + h) * alpha_row_bytes
 * (the loop group's slots come first, then its alpha block, padded to 256
 * bytes).  Token t's rows are code_row_bytes[kind], sz_row_bytes and 2 bytes
 * long, at t times those sizes from their sub-plane or row.  total_bytes
 * equals rq_cache_bytes().  token_tile is the decode kernels' wave tile in
 * tokens (16 at head_dim 96 and 128, 32 at 64): the smallest block size a
 * paged pool accepts.  (rq_cache_slot gives the same offsets for one slot.) */
typedef struct rq_layout {
  uint64_t total_bytes;
  uint64_t layer_bytes;       /* one (kv, batch row, layer) block */
  uint64_t group_bytes;       /* one loop group: all kv heads' slots, then the alpha block */
  uint64_t slot_bytes[2];     /* [0] anchor-position slots, [1] other slots */
  uint64_t sz_offset[2];      /* sz sub-plane offset inside a slot of each kind */
  uint64_t alpha_offset;      /* alpha block offset inside a loop group, or UINT64_MAX */
  uint64_t alpha_row_bytes;   /* 2 * max_tokens, or 0 without alpha */
  int32_t code_row_bytes[2];  /* d * bits / 8 of each kind */
  int32_t sz_row_bytes;       /* 2 * d / 16 */
  int32_t token_tile;
} rq_layout;

rq_status rq_cache_layout(const rq_cache_desc* desc, rq_layout* out);

/* Human-readable name of a status; never NULL. */
const char* rq_status_string(rq_status s);

/* Checks a descriptor against the supported set (host only). */
rq_status rq_validate_desc(const rq_cache_desc* desc);

/* Total size in bytes of a cache buffer for `desc` (host only).  The buffer
 * must be 256-byte aligned. */
rq_status rq_cache_bytes(const rq_cache_desc* desc, uint64_t* total_bytes);

/* Location of one slot inside the cache buffer (host only). */
rq_status rq_cache_slot(const rq_cache_desc* desc, int32_t kv, int32_t batch, int32_t layer,
                        int32_t loop, int32_t kv_head, rq_slot* out);

/*
 * Quantize-and-append (ai4snews paras. 1-2; agihunt "Confirmed").  For every
 * (kv, batch row, layer, kv head, token, loop group), quantizes the anchor
 * loop (group 16, asymmetric, FP8 e4m3fn scale = fp8((max-min)/Q), offset =
 * fp8(min), codes rounded to nearest-even against the stored FP8 values and
 * clamped to [0, Q]), then for each other loop forms r = x - deq(anchor),
 * y = H r (signs of (kv, layer)), quantizes y at residual_bits and stores
 * alpha = bf16(<y,yhat>/<yhat,yhat>) (0 when yhat = 0).  All arithmetic that
 * decides a stored value is done in IEEE double precision.
 *   cache    device, rq_cache_bytes() bytes, 256-byte aligned; written at
 *            token positions [n_tokens, n_tokens + t_new) of every slot.
 *   kv_bf16  device BF16 [2][batch][loops][layers][kv_heads][t_new][d],
 *            contiguous, 4-byte aligned.
 *   signs    device int8 [2][layers][d] of +-1 (may be NULL when rotation is
 *            NONE or mode is DIRECT).
 * Errors: RQ_ERR_CAPACITY when n_tokens + t_new > max_tokens; t_new == 0 is a
 * no-op returning RQ_OK.
 */
rq_status rq_quantize_append(const rq_cache_desc* desc, void* cache, const uint16_t* kv_bf16,
                             int32_t n_tokens, int32_t t_new, const int8_t* signs,
                             void* stream);

/*
 * Reconstruction from two reads (ai4snews para. 3): xhat = deq(anchor) +
 * alpha * H^T deq(residual) for residual loops, deq(anchor) for the anchor,
 * deq(own codes) in DIRECT mode.  Computed in fp32.
 *   out  device [2][batch][loops][layers][kv_heads][tok_end - tok_begin][d],
 *        fp32 (out_dtype RQ_OUT_F32) or BF16 round-to-nearest-even
 *        (RQ_OUT_BF16).
 */
rq_status rq_reconstruct(const rq_cache_desc* desc, const void* cache, const int8_t* signs,
                         int32_t tok_begin, int32_t tok_end, int32_t out_dtype, void* out,
                         void* stream);

/*
 * Quantize-and-append with a position per batch row, for batches whose
 * sequences have different lengths (the serving case; ai4snews para. 4
 * describes the method inside a batching inference server).  Identical to
 * rq_quantize_append except that batch row b is written at token positions
 * [positions[b], positions[b] + t_new).
 *   positions  device int32 [batch], 4-byte aligned.  They are read on the
 *              device: a row whose range does not fit [0, max_tokens) is
 *              skipped (nothing of it is written) rather than reported.
 * Errors: RQ_ERR_CAPACITY when t_new > max_tokens; RQ_ERR_INVALID_ARG when
 * positions is NULL and t_new > 0.
 */
rq_status rq_quantize_append_ragged(const rq_cache_desc* desc, void* cache,
                                    const uint16_t* kv_bf16, const int32_t* positions,
                                    int32_t t_new, const int8_t* signs, void* stream);

/* Bytes of workspace rq_decode_attention needs for `q_heads` query heads and
 * any n_tokens <= max_n_tokens (0 when no call of that size splits the
 * tokens).  The workspace starts with a fixed block of 65536 split counters
 * followed by the split partial states; see rq_decode_attention. */
uint64_t rq_decode_workspace_bytes(const rq_cache_desc* desc, int32_t q_heads,
                                   int32_t max_n_tokens);

/* Number of token splits rq_decode_attention plans for loop `loop`,
 * `q_heads` query heads and n_tokens tokens of every batch row (host only;
 * 0 for invalid arguments).  Splits are counted per (batch row, query head),
 * or per (batch row, KV head) for grouped query heads served on matrix
 * cores; 1 means the call uses no workspace.  Where the rows do not divide
 * the planned number of workgroups, the first rows take one split fewer
 * than the others, so that the grid fills it; the count returned is the
 * larger one. */
int32_t rq_decode_splits(const rq_cache_desc* desc, int32_t loop, int32_t q_heads,
                         int32_t n_tokens);

/*
 * Fused decode attention over the packed cache (abstract: reduced KV memory
 * traffic; ai4snews para. 4: reconstruction must not offset the saved
 * traffic).  One query token per (batch row, query head) attends to tokens
 * [0, n_tokens) of loop `loop`, layer `layer`:
 *     out = softmax_t(scale * q . xhat^K_t) . xhat^V_t
 * computed without materializing xhat: q . deq(anchor) + alpha (H q) .
 * deq(residual) per token, and H^T applied once to the accumulated residual-V
 * term.  Query head h reads kv head h / (q_heads / kv_heads).
 *   q_bf16     device BF16 [batch][q_heads][d], contiguous, 4-byte aligned
 *   workspace  device, >= rq_decode_workspace_bytes(desc, q_heads, n_tokens),
 *              256-byte aligned (may be NULL when that size is 0).  Holds the
 *              split-K partial states and, in its first 256 KiB, one arrival
 *              counter per (batch row, query head): the workgroup that
 *              finishes a row last merges the row's partial states.  Those
 *              counters must be ZERO before a workspace is first used (fill
 *              it with zeros once); every call returns the counters it used
 *              to zero, so the workspace then serves any sequence of calls of
 *              any shape.  Calls that share a workspace must be ordered (same
 *              stream), not concurrent.
 *   out        device fp32 [batch][q_heads][d]; n_tokens == 0 writes zeros.
 * Errors: RQ_ERR_UNSUPPORTED when q_heads is not a multiple of kv_heads or
 * batch * q_heads exceeds 65536;
 * RQ_ERR_CAPACITY when n_tokens > max_tokens; RQ_ERR_WORKSPACE.
 */
rq_status rq_decode_attention(const rq_cache_desc* desc, const void* cache,
                              const int8_t* signs, int32_t loop, int32_t layer,
                              const uint16_t* q_bf16, int32_t q_heads, int32_t n_tokens,
                              float softmax_scale, void* workspace, uint64_t workspace_bytes,
                              float* out, void* stream);

/*
 * rq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The split-K partial states and counters
 * live in a 2 MiB array inside the library, one per GPU, held until the
 * process ends; the call allocates nothing.  Arguments, results and errors are
 * those of rq_decode_attention, plus RQ_ERR_WORKSPACE when the call would need
 * more than that array (rq_decode_workspace_bytes(desc, q_heads, n_tokens) >
 * 2 MiB: every per-head plan fits; grouped-query calls with many query heads
 * per KV head over many rows may not), and RQ_ERR_LAUNCH if the array's
 * address cannot be obtained.  The first call on a GPU also enqueues a small
 * kernel on `stream` that clears the array's counters (make that first call
 * outside graph capture if the captured graph should hold only the decode
 * kernel).  All calls on one GPU share the array: calls that overlap in time
 * on one GPU (different streams without ordering) race and give wrong
 * results; calls ordered on one stream are fine.
 */
rq_status rq_decode_attention_noalloc(const rq_cache_desc* desc, const void* cache,
                                      const int8_t* signs, int32_t loop, int32_t layer,
                                      const uint16_t* q_bf16, int32_t q_heads, int32_t n_tokens,
                                      float softmax_scale, float* out, void* stream);

/*
 * Decode attention with a length per batch row: row b attends to tokens
 * [0, lengths[b]) of its slots; otherwise identical to rq_decode_attention.
 *   lengths       device int32 [batch], 4-byte aligned, read on the device and
 *                 clamped to [0, max_n_tokens]; a row of length 0 gets zeros.
 *   max_n_tokens  bound on the lengths; plans the split-K grid and sizes the
 *                 workspace (rq_decode_workspace_bytes(desc, q_heads,
 *                 max_n_tokens)).  Work scales with max_n_tokens per row.
 * Errors: as rq_decode_attention with n_tokens = max_n_tokens;
 * RQ_ERR_INVALID_ARG when lengths is NULL.
 */
rq_status rq_decode_attention_ragged(const rq_cache_desc* desc, const void* cache,
                                     const int8_t* signs, int32_t loop, int32_t layer,
                                     const uint16_t* q_bf16, int32_t q_heads,
                                     const int32_t* lengths, int32_t max_n_tokens,
                                     float softmax_scale, void* workspace,
                                     uint64_t workspace_bytes, float* out, void* stream);

/*
 * Paged cache (the block-table memory manager of a batching inference server;
 * ai4snews para. 4 places the method inside vLLM).  The cache buffer is a pool
 * of physical blocks described by an ordinary descriptor `pool` in which
 *   pool->batch       is the number of blocks in the pool, and
 *   pool->max_tokens  is the tokens per block: a power of two, at least 16
 *                     (head_dim 96, 128) or 32 (head_dim 64), with one
 *                     block's K (or V) bytes over all layers under 4 GiB;
 * the byte layout above then holds with "batch row" read as "block".  Sequence
 * s keeps logical token t in block block_table[s * max_blocks_per_seq +
 * t / block_tokens] at token t % block_tokens; the entries a call reads are
 * those of the tokens it touches.  Blocks are owned and recycled by the
 * caller; the results equal those of a contiguous cache holding the same
 * logical tokens.
 *   block_table  device int32 [n_seqs][max_blocks_per_seq], 4-byte aligned,
 *                read on the device.  Capacity per sequence is
 *                max_blocks_per_seq * block_tokens (at most 2^30; larger
 *                tables return RQ_ERR_UNSUPPORTED).
 */

/* Workspace for rq_paged_decode_attention: as rq_decode_workspace_bytes with
 * n_seqs rows (same layout and zero-once rule). */
uint64_t rq_paged_decode_workspace_bytes(const rq_cache_desc* pool, int32_t q_heads,
                                         int32_t n_seqs, int32_t max_n_tokens);

/*
 * Quantize-and-append into a paged cache: as rq_quantize_append_ragged for
 * n_seqs sequences, sequence s written at logical positions [positions[s],
 * positions[s] + t_new) through its block-table row.
 *   kv_bf16    device BF16 [2][n_seqs][loops][layers][kv_heads][t_new][d]
 *   positions  device int32 [n_seqs]; a sequence whose range does not fit its
 *              capacity is skipped, and so is a token whose block id is
 *              outside [0, pool->batch) (nothing of it is written).
 * Errors: RQ_ERR_UNSUPPORTED for a block size outside the supported set;
 * RQ_ERR_INVALID_ARG when n_seqs or max_blocks_per_seq < 1, block_table is
 * NULL, or positions is NULL with t_new > 0; RQ_ERR_CAPACITY when t_new
 * exceeds the capacity per sequence.
 */
rq_status rq_paged_quantize_append(const rq_cache_desc* pool, void* cache, const uint16_t* kv_bf16,
                                   int32_t n_seqs, const int32_t* block_table,
                                   int32_t max_blocks_per_seq, const int32_t* positions,
                                   int32_t t_new, const int8_t* signs, void* stream);

/*
 * Decode attention over a paged cache: as rq_decode_attention_ragged for
 * n_seqs sequences (q_bf16 [n_seqs][q_heads][d], out fp32 [n_seqs][q_heads][d],
 * lengths int32 [n_seqs] clamped to [0, max_n_tokens]).  Block ids outside
 * [0, pool->batch) are clamped into the pool: the output of such a sequence is
 * then unspecified, but nothing outside the cache buffer is read.
 * Errors: as rq_paged_quantize_append for the pool and table; RQ_ERR_CAPACITY
 * when max_n_tokens exceeds the capacity per sequence; otherwise as
 * rq_decode_attention_ragged (workspace from rq_paged_decode_workspace_bytes).
 */
rq_status rq_paged_decode_attention(const rq_cache_desc* pool, const void* cache,
                                    const int8_t* signs, int32_t loop, int32_t layer,
                                    const uint16_t* q_bf16, int32_t q_heads, int32_t n_seqs,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    const int32_t* lengths, int32_t max_n_tokens,
                                    float softmax_scale, void* workspace,
                                    uint64_t workspace_bytes, float* out, void* stream);

/*
 * Baseline: split-K flash decode over an uncompressed BF16 cache of the same
 * logical shape (the comparison the pages make against BF16 attention,
 * ai4snews para. 4).  k_cache and v_cache are device BF16
 * [batch][loops][layers][kv_heads][max_tokens][d]; everything else as in
 * rq_decode_attention (same workspace rules, sized by
 * rq_bf16_decode_workspace_bytes).
 */
uint64_t rq_bf16_decode_workspace_bytes(const rq_cache_desc* desc, int32_t q_heads,
                                        int32_t max_n_tokens);
rq_status rq_bf16_decode_attention(const rq_cache_desc* desc, const uint16_t* k_cache,
                                   const uint16_t* v_cache, int32_t loop, int32_t layer,
                                   const uint16_t* q_bf16, int32_t q_heads, int32_t n_tokens,
                                   float softmax_scale, void* workspace,
                                   uint64_t workspace_bytes, float* out, void* stream);

/*
 * Streaming-read probe: reads `bytes` bytes (a multiple of 16, 16-byte
 * aligned) once with non-temporal 16-byte loads, one contiguous chunk per
 * workgroup, and writes an XOR of each workgroup's words into `sink` (device,
 * rq_read_probe_sink_words() uint32 words).  Measures attainable HBM read
 * bandwidth: it was the fastest of the read patterns tried, so the decode
 * kernels' rates are reported against it.
 */
uint32_t rq_read_probe_sink_words(void);
rq_status rq_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RQ_H */
