// rq_gqa.hip -- fused decode attention for grouped-query heads on matrix cores.
//
// When G = q_heads / kv_heads query heads share one KV head, one workgroup
// serves all G of them for its token range, so the packed cache is read once
// per KV head instead of once per query head.  With G heads per cached token
// the logits and the value sums are dense contractions, and both run on
// MFMA (v_mfma_f32_16x16x32_f16 for Q K^T, v_mfma_f32_16x16x16_f16 for P V);
// the per-token quantization scales are folded into the code operand first:
//
//   * codes enter fp16 through the magic-number unpack (1024 + 2^p c, the
//     code masked where it sits, p < 8), and one v_pk_fma_f16 with
//     (s', -1024 s') turns a pair into (2^p s' c_a, 2^p s' c_b) EXACTLY: s'
//     is the FP8 scale times 2^-8 read straight from its bits (an e4m3 byte
//     shifted left by 7 is an fp16 of value x 2^-8, subnormals included),
//     and 2^p s' c has at most 8 significant bits; the 2^p is taken out on
//     the query side (K) or per output element (V);
//   * queries are exact in fp16 after a power-of-two prescale per head
//     (down to 2^-26 of the head's largest element once a slot carries its
//     2^-p); the rotated query H q is not, so it enters as an fp16 high and
//     low part;
//   * offsets z multiply per-group query sums, one more small MFMA whose
//     K slots are (group, high/low part);
//   * softmax weights enter the P V products as fp16 high + low parts.
// The logit of a residual loop is q . deq(A) + alpha^K (H q) . deq(R) and
// the value side keeps sum p deq(A^V) and sum p alpha^V deq(R^V) apart, so
// H^T is applied once per head at the end (ai4snews summary, paragraphs 3-4).
//
// Layouts (lane l, r = l % 16, c = l / 16; checked against the hardware):
//   16x16xK MFMA:  A[i][k] at lane i + 16 * (k / KP), item k % KP
//                  B[k][n] at lane n + 16 * (k / KP), item k % KP   (KP = K / 4)
//                  D[i][n] at lane n + 16 * (i / 4),  item i % 4
//   Q K^T: M = 16 tokens, N = 16 query heads (G used), K = head_dim elements,
//          so D holds S^T: lane (head r, tokens 4c..4c+3);
//   P V:   M = 16 elements of one quantization group, K = 16 tokens,
//          N = heads, with B = P^T read straight from the S^T layout.
// A wave streams 16-token tiles through a private two-stage LDS ring filled
// by buffer_load ... lds DMA.  Code planes land in blocks of whole tokens,
// [dword][token] inside a block (Blocks below); scale planes are gathered
// dword by dword into [dword][token] order.  A lane then reads the dword it
// needs of one token (K side), or of four consecutive tokens (V side), with
// one LDS read.
#include <hip/hip_runtime.h>

#include "rq_device.h"
#include "rq_kernels.h"
#include "rq_stage.h"

namespace rq {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int TT = 16;  // tokens per wave tile
// Waves per workgroup: eight, one workgroup per CU at a 256-workgroup split
// target (two waves per SIMD); measured faster than four waves at 512.
constexpr int NWG = 8;
// Group sums of prescaled queries reach 16 * 2^14: they enter fp16 scaled by
// 2^-4 and the offset products are scaled back in fp32.
constexpr float kZs = 1.f / 16.f;

// 64-lane dword DMAs moving 16 tokens x w dwords
__host__ __device__ constexpr int gather_dmas(int w) { return (16 * w + 63) / 64; }

// Code planes of W dwords per token are staged in blocks of BT whole tokens,
// one 64-lane dword DMA per block, so that every DMA instruction reads BT
// consecutive token rows: one contiguous range of global memory.  Inside a
// block the dwords are stored [dword][token], so four consecutive tokens'
// dword w are adjacent (one 128-bit read on the value side).  Blocks lie P
// dwords further apart than their 64, which spreads the reads of different
// blocks over the LDS banks.  (A [dword][token] gather over all 16 tokens of
// a tile, the layout before, reads 16 bytes of each token row per DMA
// instruction; it streamed at well under half the rate.)
template <int W, int P>
struct Blocks {
  static constexpr int BT = W > 8 ? 4 : (W > 4 ? 8 : 16);   // tokens per block
  static constexpr int NB = 16 / BT;                         // blocks (DMA instructions) per tile
  static constexpr int STRIDE = 64 + P;                      // dwords from block to block
  static constexpr int SPAN = NB * STRIDE * 4;               // bytes per tile
  static_assert(BT * W <= 64, "a block fits one DMA instruction");
  // dword position of dword w of token t
  __host__ __device__ static constexpr int pos(int t, int w) { return (t / BT) * STRIDE + w * BT + t % BT; }
};

template <int D, int B1, int B2>
struct GStage {
  static constexpr int NG = D / 16;
  static constexpr bool TWO = B2 != 0;
  static constexpr int W1 = D * B1 / 32, W2 = D * (TWO ? B2 : 2) / 32;  // code dwords per token
  static constexpr int WS = NG / 2;                                     // sz dwords per token
  static constexpr int RS = 2 * NG;                                     // sz bytes per token
  // code planes in blocks (padding measured against bank conflicts of the
  // operand reads); sz planes as [dword][token] gathers of 16 * WS dwords
  using CB1 = Blocks<W1, D == 64 ? 16 : 8>;
  using CB2 = Blocks<W2, D == 64 ? 16 : 8>;
  static constexpr int n_gather(int w) { return gather_dmas(w); }
  static constexpr int span(int w) { return gather_dmas(w) * 256; }
  static constexpr int k1c = 0;
  static constexpr int k1s = k1c + CB1::SPAN;    // sz rows padded to 16 bytes: 16 tokens
  static constexpr int v1c = k1s + 256;
  static constexpr int v1s = v1c + CB1::SPAN;
  static constexpr int k2c = v1s + span(WS);
  static constexpr int k2s = k2c + (TWO ? CB2::SPAN : 0);
  static constexpr int v2c = k2s + (TWO ? 256 : 0);
  static constexpr int v2s = v2c + (TWO ? CB2::SPAN : 0);
  static constexpr int ka = v2s + (TWO ? span(WS) : 0);
  static constexpr int va = ka + (TWO ? 256 : 0);
  static constexpr int BYTES = va + (TWO ? 256 : 0);
  static constexpr int N_DMA = 2 * CB1::NB + 1 + n_gather(WS) +
                               (TWO ? 2 * CB2::NB + 1 + n_gather(WS) + 2 : 0);
  static constexpr int KM1 = D / 32, KM2 = D / 32;   // K-side MFMAs (32 elements each) per plane
  // the V scale tables (96 bytes per group) reuse the K planes' space
  static_assert(k1s + 256 - k1c >= NG * 96 && (!TWO || k2s + 256 - k2c >= NG * 96), "V table space");
  static_assert(N_DMA < 64, "pending DMA count must fit vmcnt");
};

// [dword][token] gather of one plane: DMA lane p (over the instructions)
// moves dword w = p / 16 of token p % 16; lanes past the plane, and tokens
// past `valid` in a partial tile, re-read in-range data.
template <int W, int ROWB, bool FULL>
__device__ __forceinline__ void dma_gather(rsrc_t r, uint32_t so, int valid, lds_u8* dst, int lane) {
#pragma unroll
  for (int c = 0; c < gather_dmas(W); ++c) {
    const int p = min(c * 64 + lane, 16 * W - 1);
    const int w = p >> 4, m = FULL ? (p & 15) : min(p & 15, valid - 1);
    dma1<4, true>(r, dst + c * 256, m * ROWB + w * 4, so);
  }
}

// One code plane of a tile in blocks: DMA instruction b moves block b, lane
// p the dword at position p of its [dword][token] order; lanes past the
// block's W * BT dwords, and tokens past `valid` in a partial tile, re-read
// in-range data.
template <class CB, int W, int ROWB, bool FULL>
__device__ __forceinline__ void dma_blocks(rsrc_t r, uint32_t so, int valid, lds_u8* dst, int lane) {
  const int p = min(lane, CB::BT * W - 1);
  const int w = p / CB::BT, tl = p % CB::BT;
#pragma unroll
  for (int b = 0; b < CB::NB; ++b) {
    const int t = b * CB::BT + tl;
    const int m = FULL ? t : min(t, valid - 1);
    dma1<4, true>(r, dst + b * CB::STRIDE * 4, m * ROWB + w * 4, so);
  }
}

// Token-major sz rows padded to four dwords: DMA lane p moves dword p % 4
// (clamped to the row) of token p / 4.
template <int WS, int ROWB, bool FULL>
__device__ __forceinline__ void dma_szrows(rsrc_t r, uint32_t so, int valid, lds_u8* dst, int lane) {
  const int m = FULL ? (lane >> 2) : min(lane >> 2, valid - 1);
  dma1<4, true>(r, dst, m * ROWB + min(lane & 3, WS - 1) * 4, so);
}

__device__ __forceinline__ u32x4 lds_u32x4(const lds_u8* p) {
  typedef __attribute__((address_space(3))) const u32x4 l4;
  return *reinterpret_cast<l4*>(p);
}

__device__ __forceinline__ h2 pk_fma(h2 a, h2 b, h2 c) { return __builtin_elementwise_fma(a, b, c); }

// fp16 pair (x0 * 2^-8, x1 * 2^-8) of two FP8 e4m3 bytes held at bits 0-7 and
// 16-23 of t (other bits zero): the byte's sign moves to bit 15, its
// exponent and mantissa bits shift left by 7.
__device__ __forceinline__ h2 fp8pair_h(uint32_t t) {
  return as_h2(((t & 0x007F007Fu) << 7) | ((t & 0x00800080u) << 8));
}
// The same for non-negative bytes (scales).
__device__ __forceinline__ h2 fp8pair_pos_h(uint32_t t) { return as_h2(t << 7); }

// selector putting byte b of src1 at byte 0 and byte b of src0 at byte 2
// (bytes 1 and 3 zero) for v_perm_b32(src0, src1, sel)
__device__ __forceinline__ uint32_t sel2(uint32_t b) { return b | 0x0C00u | ((4u + b) << 16) | 0x0C000000u; }
// the same byte of one source in both halves
__device__ __forceinline__ uint32_t sel1(uint32_t b) { return b | 0x0C00u | (b << 16) | 0x0C000000u; }

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Element index of K-side slot `slot` (0..7) of lane group c in MFMA mm:
// the slots are the fp16 pairs of one code dword in unpack order.
template <int BITS>
__host__ __device__ constexpr int kslot_elem(int mm, int c, int slot) {
  if (BITS == 4) {
    const int w = 4 * mm + c, k = slot >> 1;
    return 8 * w + k + 4 * (slot & 1);
  } else {
    const int w = 2 * mm + (c >> 1), k = 4 * (c & 1) + (slot >> 1);
    return 16 * w + k + 8 * (slot & 1);
  }
}

// Inverse of kslot_elem: MFMA, lane group and slot of element e.
template <int BITS>
__device__ __forceinline__ void kslot_of(int e, int& mm, int& c, int& slot) {
  if (BITS == 4) {
    const int w = e >> 3, k8 = e & 7;
    mm = w >> 2;
    c = w & 3;
    slot = 2 * (k8 & 3) + (k8 >> 2);
  } else {
    const int w = e >> 4, k16 = e & 15, k = k16 & 7;
    mm = w >> 1;
    c = 2 * (w & 1) + (k >> 2);
    slot = 2 * (k & 3) + (k16 >> 3);
  }
}

// The K-side code pairs are masked where they sit in the dword (after one
// shift by 8 for the upper half of each 16-bit unit of 4-bit codes): pair k
// reads 2^p(k) times its codes, p = 0 or 4 for 4 bits, 2k for 2 bits.  The
// matching query slots carry 2^-p(k) (exact: a power of two), so each
// product is unchanged.
template <int BITS>
__device__ __forceinline__ float kslot_factor(int slot) {
  const int k = slot >> 1;
  return BITS == 4 ? ((k & 1) ? 1.f / 16.f : 1.f) : 1.f / (float)(1 << (2 * k));
}

// K-side A operand of MFMA mm for lane (token r, group c): eight codes of
// one dword times the FP8 scale s' of their group (and 2^p(k)), exact in
// fp16: at most 8 significant bits, below 2^9.
template <int BITS, class CB>
__device__ __forceinline__ h8 k_operand(const lds_u8* codes, u32x4 szrow, int mm, int r, int c,
                                        uint32_t magic) {
  const int w = BITS == 4 ? 4 * mm + c : 2 * mm + (c >> 1);
  const uint32_t x = lds_u32(codes + CB::pos(r, w) * 4);
  // the dword's group (w / 2 for 4 bits, w for 2 bits) has its scale in sz
  // row dword mm, at byte 2 (c >> 1) in both cases
  const uint32_t sdw = szrow[mm];
  const uint32_t sb = 2u * (uint32_t)(c >> 1);
  const h2 sp = fp8pair_pos_h(__builtin_amdgcn_perm(sdw, sdw, sel1(sb)));
  const h2 op = sp * (h2){(_Float16)-1024.f, (_Float16)-1024.f};
  h8 a;
  if constexpr (BITS == 4) {
    const uint32_t xh = x >> 8;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const h2 v = pk_fma(as_h2(and_or(k < 2 ? x : xh, 0x000F000Fu << (4 * (k & 1)), magic)), sp, op);
      a[2 * k] = v.x;
      a[2 * k + 1] = v.y;
    }
  } else {
    const uint32_t xs = x >> (8 * (c & 1));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const h2 v = pk_fma(as_h2(and_or(xs, 0x00030003u << (2 * k), magic)), sp, op);
      a[2 * k] = v.x;
      a[2 * k + 1] = v.y;
    }
  }
  return a;
}

// K-side offset operand: slot j of lane group c is group 4 (c & 1) + j (high
// query sums for c < 2, low for c >= 2); z' = z 2^-8 of the lane's token.
template <int NG>
__device__ __forceinline__ h4 kz_operand(u32x4 szrow, int c) {
  const bool hi = c & 1;
  uint32_t d0 = hi ? szrow[2] : szrow[0], d1 = hi ? szrow[3] : szrow[1];
  if (NG <= 4 && hi) d0 = 0;          // groups 4-7 do not exist
  if (NG <= 6 && hi) d1 = 0;          // groups 6-7 do not exist
  const h2 z01 = fp8pair_h(__builtin_amdgcn_perm(d0, d0, 0x0C030C01u));
  const h2 z23 = fp8pair_h(__builtin_amdgcn_perm(d1, d1, 0x0C030C01u));
  return (h4){z01.x, z01.y, z23.x, z23.y};
}

// Scale tables of one V plane for one tile, built by the wave before its
// value products so that the 16 lanes sharing a token quad do not each
// rebuild the same fp16 pairs.  Entry [g][c] of the first table holds, for
// tokens 4c..4c+3 of group g, the pairs (s'_0, s'_1), (s'_2, s'_3) and the
// same times -1024; entry [g][c] of the second holds (z'_0, z'_1),
// (z'_2, z'_3).  Lane l fills token pair l % 8 of group l / 8.  The tables
// (96 bytes per group) take the place of the tile's K-side planes, which are
// no longer needed once the logits are known.
template <int NG>
__device__ __forceinline__ void v_tables(const lds_u8* szg, lds_u8* tab, int lane) {
  typedef __attribute__((address_space(3))) uint32_t lu32;
  typedef __attribute__((address_space(3))) const u32x2 lu32x2;
  const int g = lane >> 3, tp = lane & 7;
  const u32x2 y = *reinterpret_cast<lu32x2*>(szg + (min(g >> 1, NG / 2 - 1) * 16 + 2 * tp) * 4);
  const uint32_t sb = 2u * (uint32_t)(g & 1);
  const h2 sp = fp8pair_pos_h(__builtin_amdgcn_perm(y.y, y.x, sel2(sb)));
  const h2 op = sp * (h2){(_Float16)-1024.f, (_Float16)-1024.f};
  const h2 zp = fp8pair_h(__builtin_amdgcn_perm(y.y, y.x, sel2(sb + 1u)));
  if (NG == 8 || g < NG) {
    lu32* S = reinterpret_cast<lu32*>(tab) + (g * 4 + (tp >> 1)) * 4;
    S[tp & 1] = __builtin_bit_cast(uint32_t, sp);
    S[2 + (tp & 1)] = __builtin_bit_cast(uint32_t, op);
    lu32* Z = reinterpret_cast<lu32*>(tab + NG * 64) + (g * 4 + (tp >> 1)) * 2;
    Z[tp & 1] = __builtin_bit_cast(uint32_t, zp);
  }
}

// V-side code pairs: the byte holding element e's code of two tokens goes
// to the low byte of each half, and the code is masked where it sits, at bit
// sh(e) of that byte: the pair reads 1024 + 2^sh c, and the scale fold gives
// 2^sh s' c, still exact (at most 8 significant bits, below 2^9).  The
// factor 2^sh(e) is taken out of the element's value sum at the end
// (v_unshift); sh(e) depends on e mod 4 only, which is the MFMA output item.
template <int BITS>
__device__ __forceinline__ uint32_t v_mask(int e) {
  const uint32_t m = BITS == 4 ? 0xFu << (4 * (e & 1)) : 0x3u << (2 * (e & 3));
  return m | (m << 16);
}
template <int BITS>
__device__ __forceinline__ f4 v_unshift() {
  return BITS == 4 ? (f4){1.f, 1.f / 16.f, 1.f, 1.f / 16.f} : (f4){1.f, 1.f / 4.f, 1.f / 16.f, 1.f / 64.f};
}
// (plain C, selected as one v_and_or_b32 with the mask in a VGPR; see and_or)
__device__ __forceinline__ uint32_t and_or_v(uint32_t x, uint32_t mask, uint32_t magic) {
  return (x & mask) | magic;
}

// V-side A operand for group g: element e (lane row) of tokens 4c..4c+3,
// times their scales (from the plane's table) and 2^sh(e), exact in fp16.
template <int BITS, class CB>
__device__ __forceinline__ h4 v_operand(const lds_u8* codes, const lds_u8* tab, int g, int e, int c,
                                        uint32_t mask, uint32_t magic) {
  const int w = BITS == 4 ? 2 * g + (e >> 3) : g;
  const u32x4 x = lds_u32x4(codes + CB::pos(4 * c, w) * 4);   // tokens 4c..4c+3
  const u32x4 sc = lds_u32x4(tab + (g * 4 + c) * 16);
  const uint32_t b = BITS == 4 ? (uint32_t)((e >> 1) & 3) : (uint32_t)(e >> 2);
  const uint32_t p01 = __builtin_amdgcn_perm(x.y, x.x, sel2(b));
  const uint32_t p23 = __builtin_amdgcn_perm(x.w, x.z, sel2(b));
  const h2 v01 = pk_fma(as_h2(and_or_v(p01, mask, magic)), as_h2(sc.x), as_h2(sc.z));
  const h2 v23 = pk_fma(as_h2(and_or_v(p23, mask, magic)), as_h2(sc.y), as_h2(sc.w));
  return (h4){v01.x, v01.y, v23.x, v23.y};
}

// V-side offset operand: row i = group (lane row), tokens 4c..4c+3.
template <int NG>
__device__ __forceinline__ h4 vz_operand(const lds_u8* tab, int i, int c) {
  typedef __attribute__((address_space(3))) const u32x2 lu32x2;
  const int ii = min(i, NG - 1);
  const u32x2 z = *reinterpret_cast<lu32x2*>(tab + NG * 64 + (ii * 4 + c) * 8);
  h2 z01 = as_h2(z.x), z23 = as_h2(z.y);
  if (i >= NG) z01 = z23 = (h2){(_Float16)0.f, (_Float16)0.f};
  return (h4){z01.x, z01.y, z23.x, z23.y};
}

// v as an fp16 high part and the fp16 rounding of the rest
__device__ __forceinline__ h2 split_hl(float v) {
  const _Float16 h = (_Float16)v;
  return (h2){h, (_Float16)(v - (float)h)};
}

template <int D, int B1, int B2, bool PAGED>
__global__ void __launch_bounds__(NWG * 64, 2) gqa_kernel(DecodeArgs a) {
  using GS = GStage<D, B1, B2>;
  constexpr int NG = GS::NG;
  constexpr bool TWO = GS::TWO;
  constexpr int B2E = TWO ? B2 : 2;
  constexpr int KM1 = GS::KM1, KM2 = GS::KM2;
  constexpr int R1 = D * B1 / 8, R2 = D * B2E / 8, RS = GS::RS;
  constexpr int kRing = NWG * 2 * GS::BYTES;
  // merge rows of one head: value sums (first plane | residual) and the
  // offset sums per group, padded to whole float4s plus one
  constexpr int kZOff = (TWO ? 2 : 1) * D;
  constexpr int kRowF = (kZOff + (TWO ? 2 : 1) * NG + 3) / 4 * 4 + 4;
  constexpr int kMerge = NWG * 8 * kRowF * 4;   // NWG regions x 8 heads, or NWG / 2 x 16
  const Geometry& g = a.g;

  __shared__ __attribute__((aligned(16))) uint8_t smem[kRing > kMerge ? kRing : kMerge];
  // B operands of the Q K^T products in lane order, [mm][lane][8 halves]:
  // the prescaled queries (exact) and the rotated queries' high and low parts.
  // Before they are built, the same bytes stage the query rows (256 bytes
  // per head) and the key signs by DMA.
  typedef _Float16 QOp[64][8];
  constexpr int kOpBytes = (KM1 + 2 * (TWO ? KM2 : 1)) * (int)sizeof(QOp);
  constexpr int kStageBytes = 16 * 256 + 256;
  __shared__ __attribute__((aligned(16))) uint8_t qop[kOpBytes > kStageBytes ? kOpBytes : kStageBytes];
  QOp* fq = reinterpret_cast<QOp*>(qop);
  QOp* fuh = fq + KM1;
  QOp* ful = fuh + (TWO ? KM2 : 1);
  __shared__ float sqs[16][8], sus[16][8];       // per-group sums of the two
  __shared__ float spq[16], spu[16];             // per-head prescales
  __shared__ float sm_m[NWG][16], sm_l[NWG][16];
  __shared__ uint32_t s_ticket;
  __shared__ uint32_t s_claim;   // next unclaimed wave tile of this split

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int split = blockIdx.x, bk = blockIdx.y;     // bk = batch row * kv_heads + kv head
  const int b = bk / g.kv_heads, kvh = bk % g.kv_heads;
  const int G = a.group_ratio;
  const bool rotated = TWO && g.rotation == RQ_ROT_HADAMARD;
  uint32_t magic;
  asm("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kMagic));

  const int n_row = a.lengths ? min(max(a.lengths[b], 0), a.n_tokens) : a.n_tokens;
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(n_row, t_begin + a.tokens_per_split);

  // ---- buffer resources.  Contiguous cache: one per plane (a slot, or the
  // residual plane's alpha row).  Paged pool: one over the tile's pool block
  // in the K half and one in the V half, rebuilt per tile, with every plane
  // at its offset inside the block (the same for K and V).
  const int loop1 = (g.mode == RQ_MODE_DIRECT || !TWO) ? a.loop : (a.loop - a.loop % g.P + g.P - 1);
  const uint32_t sb1 = (uint32_t)g.slot_bytes[g.is_anchor(loop1) ? 0 : 1];
  const uint32_t sb2 = (uint32_t)g.slot_bytes[g.is_anchor(a.loop) ? 0 : 1];
  const uint32_t arow = (uint32_t)g.alpha_row;
  const int brow = PAGED ? 0 : b;
  const uint64_t o1 = g.slot_offset(0, brow, a.layer, loop1, kvh);
  const uint64_t o2 = g.slot_offset(0, brow, a.layer, a.loop, kvh);
  const uint64_t oa = TWO ? g.alpha_offset(0, brow, a.layer, a.loop, kvh) : 0;
  const uint64_t vhalf = (uint64_t)g.batch * g.layers * g.layer_block;  // K -> V
  const uint64_t bstride = (uint64_t)g.layers * g.layer_block;          // one pool block
  rsrc_t rk1, rv1, rk2, rv2, rka, rva;
  uint32_t po1 = 0, po2 = 0, poa = 0;  // paged: plane offsets inside the block
  if constexpr (!PAGED) {
    rk1 = make_rsrc(a.cache + o1, sb1);
    rv1 = make_rsrc(a.cache + vhalf + o1, sb1);
    rk2 = make_rsrc(a.cache + o2, sb2);
    rv2 = make_rsrc(a.cache + vhalf + o2, sb2);
    if constexpr (TWO) {
      rka = make_rsrc(a.cache + oa, arow);
      rva = make_rsrc(a.cache + vhalf + oa, arow);
    }
  } else {
    po1 = (uint32_t)o1;
    po2 = (uint32_t)o2;
    poa = (uint32_t)oa;
  }
  auto point_at = [&](uint64_t delta) __attribute__((always_inline)) {
    rk1 = rk2 = rka = make_rsrc(a.cache + delta, (uint32_t)bstride);
    rv1 = rv2 = rva = make_rsrc(a.cache + vhalf + delta, (uint32_t)bstride);
  };
  typedef const __attribute__((address_space(4))) int32_t c_i32;
  const c_i32* btab = (const c_i32*)(a.paging.table + (uint64_t)b * a.paging.max_blocks);
  const uint32_t s1rel = po1 + (uint32_t)g.sz_rel(loop1), s2rel = po2 + (uint32_t)g.sz_rel(a.loop);

  // ---- this wave's tiles through its two-stage ring
  lds_u8* ring = (lds_u8*)smem + w * 2 * GS::BYTES;
  // Tile k of the split holds tokens [t_begin + k TT, + TT).  Waves start
  // with tiles w and NWG + w; after that each wave claims the next unclaimed
  // tile from an LDS counter, one tile ahead, so no wave idles while another
  // still holds an equal share of the split (the second wave of a SIMD loses
  // issue arbitration to the first).  Tiles are summed in a different order
  // from call to call: results agree to fp32 summation order.
  const int n_tot = t_end > t_begin ? (t_end - t_begin + TT - 1) / TT : 0;
  int kcur = w, knext = NWG + w;   // tile being computed, tile after it
  uint32_t claimed = 0;             // lane 0: the tile claimed for the one after
  auto issue_t = [&](auto full, uint32_t tb, lds_u8* st, int vt) __attribute__((always_inline)) {
    constexpr bool F = decltype(full)::value;
    dma_blocks<typename GS::CB1, GS::W1, R1, F>(rk1, po1 + tb * R1, vt, st + GS::k1c, lane);
    dma_szrows<GS::WS, RS, F>(rk1, s1rel + tb * RS, vt, st + GS::k1s, lane);
    dma_blocks<typename GS::CB1, GS::W1, R1, F>(rv1, po1 + tb * R1, vt, st + GS::v1c, lane);
    dma_gather<GS::WS, RS, F>(rv1, s1rel + tb * RS, vt, st + GS::v1s, lane);
    if constexpr (TWO) {
      dma_blocks<typename GS::CB2, GS::W2, R2, F>(rk2, po2 + tb * R2, vt, st + GS::k2c, lane);
      dma_szrows<GS::WS, RS, F>(rk2, s2rel + tb * RS, vt, st + GS::k2s, lane);
      dma_blocks<typename GS::CB2, GS::W2, R2, F>(rv2, po2 + tb * R2, vt, st + GS::v2c, lane);
      dma_gather<GS::WS, RS, F>(rv2, s2rel + tb * RS, vt, st + GS::v2s, lane);
      dma_alpha(rka, poa + tb * 2, F ? TT : vt, st + GS::ka, lane);
      dma_alpha(rva, poa + tb * 2, F ? TT : vt, st + GS::va, lane);
    }
  };
  auto issue = [&](int k, int slot) __attribute__((always_inline)) {
    uint32_t tb = (uint32_t)(t_begin + k * TT);
    lds_u8* st = ring + slot * GS::BYTES;
    const int vt = t_end - (int)tb;
    if constexpr (PAGED) {
      const int blk = min(max(btab[tb >> a.paging.block_shift], 0), g.batch - 1);
      point_at((uint64_t)blk * bstride);
      tb &= (1u << a.paging.block_shift) - 1u;
    }
    if (vt >= TT)
      issue_t(std::integral_constant<bool, true>{}, tb, st, TT);
    else
      issue_t(std::integral_constant<bool, false>{}, tb, st, vt);
  };
  // ---- the query rows of this wave's heads (w, w + NWG, ... below G) and the
  // key signs come in by DMA ahead of the first tile: a plain load issued
  // after the tile's DMAs would wait for all of them.  (Issuing the second
  // tile here as well measured slower.)
  lds_u8* stage = (lds_u8*)qop;
  for (int n = w; n < G; n += NWG) {
    const uint16_t* qrow = a.q + ((uint64_t)b * a.q_heads + kvh * G + n) * D;
    dma1<4>(make_rsrc((const uint8_t*)qrow, 2 * D), stage + n * 256, min(4 * lane, 2 * D - 4), 0u);
  }
  if (rotated && w == 0)
    dma1<4>(make_rsrc((const uint8_t*)(a.signs + (uint64_t)a.layer * D), D), stage + 16 * 256,
            min(4 * lane, D - 4), 0u);
  if (kcur < n_tot) issue(kcur, 0);
  if (tid == 0) s_claim = 2 * NWG;
  if (kcur < n_tot) wait_vm<GS::N_DMA>();
  else wait_vm<0>();
  __syncthreads();   // every wave's rows and the signs are in LDS
  constexpr int kHw = 16 / NWG;   // operand columns per wave
  const bool v1ok = (D > 64) && (lane + 64 < D);
  float qv0[kHw], qv1[kHw];
#pragma unroll
  for (int j = 0; j < kHw; ++j) {
    const int n = w + NWG * j;
    const lds_u8* row = stage + min(n, 15) * 256;
    qv0[j] = n < G ? bf16_to_f32(lds_u16(row + 2 * lane)) : 0.f;
    qv1[j] = (n < G && v1ok) ? bf16_to_f32(lds_u16(row + 2 * (lane + 64))) : 0.f;
  }
  float sg0 = 1.f, sg1 = 1.f;
  if (rotated) {
    const int8_t* sg = (const int8_t*)(qop + 16 * 256);  // K signs of this layer
    sg0 = (float)sg[lane];
    sg1 = v1ok ? (float)sg[lane + 64] : 0.f;
  }
  __syncthreads();   // the operand tables below overwrite the staged rows

  // ---- query side: prescaled queries and rotated queries of the G heads;
  // the columns n >= G are zero
#pragma unroll
  for (int j = 0; j < kHw; ++j) {
    const int n = w + NWG * j;
    if (n >= G) {
      int mm, cc, sl;
      kslot_of<B1>(lane, mm, cc, sl);
      fq[mm][n + 16 * cc][sl] = (_Float16)0.f;
      if (v1ok) {
        kslot_of<B1>(lane + 64, mm, cc, sl);
        fq[mm][n + 16 * cc][sl] = (_Float16)0.f;
      }
      if (r == 0) {
        sqs[n][c] = 0.f;
        if (c + 4 < NG) sqs[n][c + 4] = 0.f;
      }
      if (lane == 0) spq[n] = 1.f;
      if constexpr (TWO) {
        kslot_of<B2E>(lane, mm, cc, sl);
        fuh[mm][n + 16 * cc][sl] = (_Float16)0.f;
        ful[mm][n + 16 * cc][sl] = (_Float16)0.f;
        if (v1ok) {
          kslot_of<B2E>(lane + 64, mm, cc, sl);
          fuh[mm][n + 16 * cc][sl] = (_Float16)0.f;
          ful[mm][n + 16 * cc][sl] = (_Float16)0.f;
        }
        if (r == 0) {
          sus[n][c] = 0.f;
          if (c + 4 < NG) sus[n][c + 4] = 0.f;
        }
        if (lane == 0) spu[n] = 1.f;
      }
      continue;
    }
    const float q0 = qv0[j], q1 = qv1[j];
    const float pq = fp16_prescale(wave_max(fmaxf(fabsf(q0), fabsf(q1))));
    const float x0 = q0 * pq, x1 = q1 * pq;
    {
      int mm, cc, sl;
      kslot_of<B1>(lane, mm, cc, sl);
      fq[mm][n + 16 * cc][sl] = (_Float16)(x0 * kslot_factor<B1>(sl));
      if (v1ok) {
        kslot_of<B1>(lane + 64, mm, cc, sl);
        fq[mm][n + 16 * cc][sl] = (_Float16)(x1 * kslot_factor<B1>(sl));
      }
    }
    const float s0 = row_sum16(x0), s1 = row_sum16(x1);
    if (r == 0) {
      sqs[n][c] = s0;
      if (c + 4 < NG) sqs[n][c + 4] = s1;
    }
    if (lane == 0) spq[n] = pq;
    if constexpr (TWO) {
      float u0 = q0, u1 = q1;
      if (rotated) {
        u0 *= sg0;
        u1 = v1ok ? u1 * sg1 : 0.f;
        wave_wht<D>(u0, u1, lane);
        u0 *= (D == 128) ? 0.08838834764831845f : 0.125f;
        u1 = v1ok ? u1 * ((D == 128) ? 0.08838834764831845f : 0.17677669529663687f) : 0.f;
      }
      const float pu = fp16_prescale(wave_max(fmaxf(fabsf(u0), fabsf(u1))));
      const float y0 = u0 * pu, y1 = u1 * pu;
      {
        int mm, cc, sl;
        kslot_of<B2E>(lane, mm, cc, sl);
        h2 hl = split_hl(y0 * kslot_factor<B2E>(sl));
        fuh[mm][n + 16 * cc][sl] = hl.x;
        ful[mm][n + 16 * cc][sl] = hl.y;
        if (v1ok) {
          kslot_of<B2E>(lane + 64, mm, cc, sl);
          hl = split_hl(y1 * kslot_factor<B2E>(sl));
          fuh[mm][n + 16 * cc][sl] = hl.x;
          ful[mm][n + 16 * cc][sl] = hl.y;
        }
      }
      const float t0 = row_sum16(y0), t1 = row_sum16(y1);
      if (r == 0) {
        sus[n][c] = t0;
        if (c + 4 < NG) sus[n][c + 4] = t1;
      }
      if (lane == 0) spu[n] = pu;
    }
  }
  __syncthreads();

  // ---- this lane's B operands (query head r)
  typedef __attribute__((address_space(3))) const h8 lh8;
  h4 BzQ, BzU;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int gz = 4 * (c & 1) + j;
    const h2 hl = gz < NG ? split_hl(sqs[r][gz] * kZs) : (h2){(_Float16)0.f, (_Float16)0.f};
    BzQ[j] = c < 2 ? hl.x : hl.y;
  }
  if constexpr (TWO) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gz = 4 * (c & 1) + j;
      const h2 hl = gz < NG ? split_hl(sus[r][gz] * kZs) : (h2){(_Float16)0.f, (_Float16)0.f};
      BzU[j] = c < 2 ? hl.x : hl.y;
    }
  }
  // logit = qscale * 2^8 * (S_A / pq + alpha S_R / pu)   (s', z' carry 2^-8)
  const float cA = a.qscale * 256.f / spq[r];
  const float cR = TWO ? a.qscale * 256.f / spu[r] : 0.f;

  f4 OA[NG], OR_[TWO ? NG : 1], OZA = {0.f, 0.f, 0.f, 0.f}, OZR = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NG; ++i) OA[i] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < (TWO ? NG : 1); ++i) OR_[i] = (f4){0.f, 0.f, 0.f, 0.f};
  float m = kEmpty, l = 0.f;
  const uint32_t vm1 = v_mask<B1>(r), vm2 = v_mask<B2E>(r);   // this lane's element row

  auto claim = [&]() __attribute__((always_inline)) {
    if (lane == 0)
      claimed = __hip_atomic_fetch_add(&s_claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  claim();
  // Tiles are claimed in increasing order, so once knext is past the split
  // every later claim is too.
  for (int it = 0; kcur < n_tot; ++it) {
    // slot (it & 1) holds kcur; knext goes into the slot the tile before left
    if (knext < n_tot) issue(knext, (it + 1) & 1);
    if (it > 0) claim();
    if (knext < n_tot) wait_vm<GS::N_DMA>();
    else wait_vm<0>();
    const lds_u8* st = ring + (it & 1) * GS::BYTES;
    const int vt = t_end - (t_begin + kcur * TT);  // in-range tokens of this tile

    // ---- logits S^T (lane: head r, tokens 4c + j)
    f4 SA = {0.f, 0.f, 0.f, 0.f};
    {
      const u32x4 szr = lds_u32x4(st + GS::k1s + r * 16);
#pragma unroll
      for (int mm = 0; mm < KM1; ++mm)
        SA = mfma32(k_operand<B1, typename GS::CB1>(st + GS::k1c, szr, mm, r, c, magic),
                    *(lh8*)&fq[mm][lane][0], SA);
      // the offset term starts its own accumulator: chaining a 16x16x16 MFMA
      // onto the 16x16x32 results (C operand) gave wrong sums on gfx950
      SA += mfma16(kz_operand<NG>(szr, c), BzQ, (f4){0.f, 0.f, 0.f, 0.f}) * (1.f / kZs);
    }
    f4 SR = {0.f, 0.f, 0.f, 0.f};
    u32x4 alk = {0u, 0u, 0u, 0u}, alv = {0u, 0u, 0u, 0u};
    if constexpr (TWO) {
      const u32x4 szr = lds_u32x4(st + GS::k2s + r * 16);
#pragma unroll
      for (int mm = 0; mm < KM2; ++mm) {
        const h8 x = k_operand<B2E, typename GS::CB2>(st + GS::k2c, szr, mm, r, c, magic);
        SR = mfma32(x, *(lh8*)&fuh[mm][lane][0], SR);
        SR = mfma32(x, *(lh8*)&ful[mm][lane][0], SR);
      }
      SR += mfma16(kz_operand<NG>(szr, c), BzU, (f4){0.f, 0.f, 0.f, 0.f}) * (1.f / kZs);
      alk = lds_u32x4(st + GS::ka + 16 * c);   // alpha of token i at byte 4 i
      alv = lds_u32x4(st + GS::va + 16 * c);
    }
    float lg[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = SA[j] * cA;
      if constexpr (TWO) v = fmaf(bf16_to_f32(alk[j] & 0xFFFFu) * cR, SR[j], v);
      lg[j] = (4 * c + j < vt) ? v : kEmpty;
    }

    // ---- online softmax per head (the four lanes of a head agree)
    float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mx = pair_max<32>(pair_max<16>(mx));
    if (mx > m + kLazy) {
      const float corr = __builtin_amdgcn_exp2f(m - mx);
      l *= corr;
#pragma unroll
      for (int i = 0; i < NG; ++i) OA[i] *= corr;
      OZA *= corr;
      if constexpr (TWO) {
#pragma unroll
        for (int i = 0; i < NG; ++i) OR_[i] *= corr;
        OZR *= corr;
      }
      m = mx;
    }
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = (4 * c + j < vt) ? __builtin_amdgcn_exp2f(lg[j] - m) : 0.f;
    l += (p[0] + p[1]) + (p[2] + p[3]);
    h4 Ph, Pl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const h2 hl = split_hl(p[j]);
      Ph[j] = hl.x;
      Pl[j] = hl.y;
    }

    // ---- values: O^T[e][head] per group, and the offset sums per group
    {
      lds_u8* tab = const_cast<lds_u8*>(st) + GS::k1c;   // K1 planes are done with
      v_tables<NG>(st + GS::v1s, tab, lane);
#pragma unroll
      for (int gq = 0; gq < NG; ++gq) {
        const h4 x = v_operand<B1, typename GS::CB1>(st + GS::v1c, tab, gq, r, c, vm1, magic);
        OA[gq] = mfma16(x, Ph, OA[gq]);
        OA[gq] = mfma16(x, Pl, OA[gq]);
        // bounds how many groups' loads are hoisted: two groups at a time
        if (gq & 1) __builtin_amdgcn_sched_barrier(0);
      }
      const h4 z = vz_operand<NG>(tab, r, c);
      OZA = mfma16(z, Ph, OZA);
      OZA = mfma16(z, Pl, OZA);
    }
    if constexpr (TWO) {
      h4 Qh, Ql;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const h2 hl = split_hl(p[j] * bf16_to_f32(alv[j] & 0xFFFFu));
        Qh[j] = hl.x;
        Ql[j] = hl.y;
      }
      lds_u8* tab = const_cast<lds_u8*>(st) + GS::k2c;   // K2 planes are done with
      v_tables<NG>(st + GS::v2s, tab, lane);
#pragma unroll
      for (int gq = 0; gq < NG; ++gq) {
        const h4 x = v_operand<B2E, typename GS::CB2>(st + GS::v2c, tab, gq, r, c, vm2, magic);
        OR_[gq] = mfma16(x, Qh, OR_[gq]);
        OR_[gq] = mfma16(x, Ql, OR_[gq]);
        if (gq & 1) __builtin_amdgcn_sched_barrier(0);
      }
      const h4 z = vz_operand<NG>(tab, r, c);
      OZR = mfma16(z, Qh, OZR);
      OZR = mfma16(z, Ql, OZR);
    }
    kcur = knext;
    knext = (int)__builtin_amdgcn_readfirstlane(claimed);
  }

  // ---- merge the waves: running max per head, then the G heads' sums of
  // every wave side by side (one round), or, for G > 8, two waves into each
  // of NWG / 2 regions (two rounds); either way at most 64 head rows
  l = pair_add<32>(pair_add<16>(l));
  if (c == 0) {
    sm_m[w][r] = m;
    sm_l[w][r] = l;
  }
  __syncthreads();  // every wave is done with its ring: the merge regions reuse it
  float M = sm_m[0][r];
#pragma unroll
  for (int ww = 1; ww < NWG; ++ww) M = fmaxf(M, sm_m[ww][r]);
  const float f = exp2f(m - M) * 256.f;  // also takes out the 2^-8 of s' and z'
  const int nreg = G <= 8 ? NWG : NWG / 2;   // regions: at most 64 head rows
  float* regs = reinterpret_cast<float*>(smem);   // [region][head][kRowF]
  auto put = [&](float* row, bool add) __attribute__((always_inline)) {
#pragma unroll
    for (int gq = 0; gq < NG; ++gq) {
      f4* pa = reinterpret_cast<f4*>(row + 16 * gq + 4 * c);
      *pa = (add ? *pa : (f4){0.f, 0.f, 0.f, 0.f}) + (f * v_unshift<B1>()) * OA[gq];
      if constexpr (TWO) {
        f4* pr = reinterpret_cast<f4*>(row + D + 16 * gq + 4 * c);
        *pr = (add ? *pr : (f4){0.f, 0.f, 0.f, 0.f}) + (f * v_unshift<B2E>()) * OR_[gq];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * c + j;
      if (i < NG) {
        float* za = row + kZOff + i;
        *za = (add ? *za : 0.f) + f * OZA[j];
        if constexpr (TWO) {
          float* zr = row + kZOff + NG + i;
          *zr = (add ? *zr : 0.f) + f * OZR[j];
        }
      }
    }
  };
  if (r < G && w < nreg) put(regs + (w * G + r) * kRowF, false);
  if (nreg < NWG) {
    __syncthreads();
    if (r < G && w >= nreg) put(regs + ((w - nreg) * G + r) * kRowF, true);
  }
  __syncthreads();
  auto head_l = [&](int n) {
    float s = 0.f, Mn = sm_m[0][n];
#pragma unroll
    for (int ww = 1; ww < NWG; ++ww) Mn = fmaxf(Mn, sm_m[ww][n]);
#pragma unroll
    for (int ww = 0; ww < NWG; ++ww) s = fmaf(exp2f(sm_m[ww][n] - Mn), sm_l[ww][n], s);
    return s;
  };
  auto head_m = [&](int n) {
    float Mn = sm_m[0][n];
#pragma unroll
    for (int ww = 1; ww < NWG; ++ww) Mn = fmaxf(Mn, sm_m[ww][n]);
    return Mn;
  };
  // element e of head n's value sum (plane 0: first plane, 1: residual)
  auto acc = [&](int n, int plane, int e) {
    float s = 0.f;
    for (int k = 0; k < nreg; ++k) {
      const float* row = regs + (k * G + n) * kRowF;
      s += row[plane * D + e] + row[kZOff + plane * NG + (e >> 4)];
    }
    return s;
  };
  auto accA = [&](int n, int e) { return acc(n, 0, e); };
  auto accR = [&](int n, int e) { return TWO ? acc(n, 1, e) : 0.f; };

  if (a.splits > 1) {
    // partial state (m, l, accA[D], accR[D]) of every head, as the per-head
    // kernel writes it
    constexpr int Wd = 2 + 2 * D;
    for (int i = tid; i < G * Wd; i += NWG * 64) {
      const int n = i / Wd, k = i % Wd;
      const int bh = b * a.q_heads + kvh * G + n;
      float* mine = a.partials + ((uint64_t)bh * a.splits + split) * Wd;
      float v;
      if (k == 0) v = head_m(n);
      else if (k == 1) v = head_l(n);
      else if (k < 2 + D) v = accA(n, k - 2);
      else v = accR(n, k - 2 - D);
      store_dev(mine + k, v);
    }
    // the workgroup that finishes the KV head last merges its G rows (one
    // counter per KV head: that of its first query head)
    const int bh0 = b * a.q_heads + kvh * G;
    if (!arrive_last(a, bh0, a.splits, tid, &s_ticket)) return;
    for (int n = w; n < G; n += NWG) merge_splits<D, TWO>(a, bh0 + n, a.splits, lane);
    return;
  }
  // ---- a single split: finish here, one wave per head
  for (int n = w; n < G; n += NWG) {
    const float Ln = head_l(n);
    const float A0 = accA(n, lane), A1 = v1ok ? accA(n, lane + 64) : 0.f;
    float R0 = accR(n, lane), R1 = v1ok ? accR(n, lane + 64) : 0.f;
    if (rotated) {
      wave_wht<D>(R0, R1, lane);
      const int8_t* sg = a.signs + ((uint64_t)g.layers + a.layer) * D;  // V signs
      R0 *= ((D == 128) ? 0.08838834764831845f : 0.125f) * (float)sg[lane];
      if (v1ok) R1 *= ((D == 128) ? 0.08838834764831845f : 0.17677669529663687f) * (float)sg[lane + 64];
    }
    const float inv = Ln > 0.f ? 1.f / Ln : 0.f;
    const uint64_t bh = (uint64_t)b * a.q_heads + kvh * G + n;
    a.out[bh * D + lane] = (A0 + R0) * inv;
    if (v1ok) a.out[bh * D + lane + 64] = (A1 + R1) * inv;
  }
}

template <int D, int B1, int B2>
hipError_t launch_gqa_t(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.splits, a.rows * a.g.kv_heads);
  if (a.paging.table)
    hipLaunchKernelGGL((gqa_kernel<D, B1, B2, true>), grid, dim3(NWG * 64), 0, s, a);
  else
    hipLaunchKernelGGL((gqa_kernel<D, B1, B2, false>), grid, dim3(NWG * 64), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_gqa_d(const DecodeArgs& a, hipStream_t s) {
  const Geometry& g = a.g;
  if (g.mode == RQ_MODE_DIRECT || g.is_anchor(a.loop))
    return g.bits_of(a.loop) == 4 ? launch_gqa_t<D, 4, 0>(a, s) : launch_gqa_t<D, 2, 0>(a, s);
  return g.anchor_bits == 4 ? launch_gqa_t<D, 4, 2>(a, s) : launch_gqa_t<D, 2, 2>(a, s);
}

}  // namespace

int gqa_tile_tokens() { return NWG * TT; }

bool gqa_supported(const Geometry& g, int loop, int group_ratio) {
  if (group_ratio < 2 || group_ratio > 16) return false;
  if (g.mode == RQ_MODE_DIRECT || g.is_anchor(loop)) return true;   // one plane of 2 or 4 bits
  if (g.mode == RQ_MODE_CHAINED && g.P - 1 - loop % g.P > 1) return false;
  return g.residual_bits == 2;
}

hipError_t launch_gqa(const DecodeArgs& a, hipStream_t s) {
  switch (a.g.d) {
    case 64: return launch_gqa_d<64>(a, s);
    case 96: return launch_gqa_d<96>(a, s);
    default: return launch_gqa_d<128>(a, s);
  }
}

}  // namespace rq
