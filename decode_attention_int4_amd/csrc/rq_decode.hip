// rq_decode.hip -- fused split-K decode attention over the packed cache.
//
// One query token per (batch row, query head) attends to tokens [0, n) of one
// (loop, layer).  Nothing is dequantized to memory: for each cached token the
// logit is
//     q . deq(A_t) + alpha^K_t (H q) . deq(R_t)
// with every group of 16 written as s * sum(q_i c_i) + z * sum(q_i), and the
// value side accumulates sum_t p_t deq(A^V_t) and sum_t p_t alpha^V_t deq(R^V_t)
// separately so H^T is applied once to the second sum at the end (ai4snews
// summary, paragraphs 3-4: two reads per loop, reconstruction must not offset
// the saved memory traffic).
//
// gfx950 mapping.
//   one workgroup per (batch * q_heads row, split), NWK = 4 or 8 waves per workgroup (8 for
//   d = 128 calls reading at most one residual plane, paged anchor calls
//   aside: decode_waves).  A wave takes its
//   tokens in PAIRS (t, t + TPW/2 of its tile); LPP lanes share a pair and each owns one
//   quantization group (16 head_dim elements) of both tokens, so a lane's
//   accumulators cover just 16 elements.
//   Codes are never converted element by element: one v_and_or_b32 drops two
//   codes into the mantissas of an fp16 pair whose exponent encodes 1024 (the
//   "magic number" conversion), giving 1024 + m*c.
//   * Keys at d = 128 and 96 (at most one residual plane): one
//     v_mfma_f32_16x16x32_f16 chain per 16-token tile, the codes in
//     magic-number form against a block-diagonal query operand (one row per
//     group and plane), so the code-times-query sums leave the VALU.
//     Elsewhere (d = 64, chained loops) the pair holds two elements of ONE
//     token and meets (q_a, q_b)/m in v_dot2_f32_f16.  Either way the
//     constant 1024*sum(q)/m is subtracted once per group.  The query is
//     exact in fp16 after a power-of-two prescale (BF16 fits fp16's
//     mantissa); H q is not, so it is split into fp16 high and low parts and
//     each meets the codes.
//   * Values: v_perm_b32 first interleaves the same 16-bit unit of the two
//     tokens, so the pair holds ONE element of BOTH tokens and meets the fp16
//     weight pair (p_t s_t, p_t' s_t') in v_dot2_f32_f16 -- one instruction
//     per two multiply-adds.  The first plane's weights go in as an fp16 high
//     and low part (two dot2s); the residual plane, a smaller term, uses one
//     fp16 weight against codes centred on the middle code.  The magic
//     constant is folded out of a lane's sums every eight tiles (and at the
//     end) from the running sum of the fp16 weights, so the fp32 rounding of
//     the code term does not grow with the context.
//   FP8 scale/offset bytes are decoded by v_cvt_pk_f32_fp8 (OCP e4m3fn on
//   gfx950).  Each wave streams its tiles through a private ring in LDS filled
//   by buffer_load ... lds DMA with scalar offsets, so issuing a tile costs no
//   vector instructions.
//   Each lane keeps its own online-softmax state; the running maximum is only
//   raised when a logit exceeds it by 8 (log2 units), so the rescale of the
//   accumulators is rare.  A wave's token pairs are summed in registers (DPP
//   and the gfx950 permlane swaps), its waves through LDS.
//   With one split the workgroup's first wave applies H^T and writes the fp32
//   output; otherwise each workgroup stores its partial state with
//   write-through (device-scope) stores, waits for them to complete and takes
//   a ticket from the row's counter, and the workgroup holding the last
//   ticket reads all partial states with device-scope loads and merges them.
//   No cache write-back or invalidation is needed (a release fence per
//   workgroup, an L2 write-back, cost far more than a separate merge kernel).
#include <hip/hip_runtime.h>

#include "rq_device.h"
#include "rq_kernels.h"
#include "rq_stage.h"

#include <type_traits>

namespace rq {
namespace {

// Value weights enter fp16 scaled by these powers of two, so that
// p (<= 2^8) times an FP8 scale (<= 448), times alpha for residuals, fits.
constexpr float kWA = 1.f / 16.f, kWR = 1.f / 256.f;

template <int D>
struct Lay {
  static constexpr int NG = D / 16;
  static constexpr int LPP = D == 64 ? 4 : 8;  // lanes per token pair (d = 96: 6 of 8 busy)
  static constexpr int PAIRS = 64 / LPP;        // token pairs per wave step
  static constexpr int TPW = 2 * PAIRS;         // tokens per wave step
};

// ------------------------------------------------------------ code pairs
// A dword of BITS-bit codes holds 32/BITS codes (element j at bit j*BITS),
// i.e. two 16-bit units.  Pair k takes code k of each unit into the two fp16
// halves: after an optional right shift, masking leaves code k of the low
// unit at bit position p of the low half and code k of the high unit at the
// same position of the high half; OR-ing 1024's exponent makes the halves
// 1024 + 2^p * code.
template <int BITS>
struct Pairs {
  static constexpr int PER_UNIT = 16 / BITS;  // 4 (int4) or 8 (int2)
  __host__ __device__ static constexpr int shift(int k) {
    return BITS == 4 ? (k < 2 ? 0 : 8) : (k < 5 ? 0 : 10);
  }
  __host__ __device__ static constexpr int pos(int k) {  // bit position inside a half
    return BITS == 4 ? 4 * (k & 1) : 2 * (k < 5 ? k : k - 5);
  }
  __host__ __device__ static constexpr uint32_t mask(int k) {
    return (((1u << BITS) - 1u) * 0x00010001u) << pos(k);
  }
  __host__ __device__ static constexpr float mult(int k) { return (float)(1u << pos(k)); }
};

template <int BITS, int K>
__device__ __forceinline__ h2 pair_of(uint32_t w, uint32_t magic) {
  using PR = Pairs<BITS>;
  return as_h2(and_or(PR::shift(K) ? (w >> PR::shift(K)) : w, PR::mask(K), magic));
}

// ------------------------------------------------------------ DPP helpers
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;   // lane i <-> 7-i inside each half row

// Sum over the LPP lanes of one token pair.
template <int LPP>
__device__ __forceinline__ float pair_sum(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  if constexpr (LPP == 8) v += dpp<kHalfMirror>(v);
  return v;
}

// (scale, offset) decoded by the hardware from the low or high FP8 byte pair.
__device__ __forceinline__ f2 sz_pair(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, false); }

// ------------------------------------------------------------ LDS staging
// Each wave streams its tiles (TPW consecutive tokens) through a private ring
// of COUNT buffers in LDS, filled by DMA: the bytes in flight occupy LDS
// instead of VGPRs, so COUNT-1 tiles stay in flight while one is consumed.  A
// tile buffer mirrors the contiguous global bytes of each plane piece.
__host__ __device__ constexpr int al16(int x) { return (x + 15) / 16 * 16; }

// DMA granule of a piece: 16 bytes per lane when whole 1 KB instructions
// cover it and tokens stay 16-byte aligned, else 4 bytes per lane.  Every DMA
// instruction runs on all 64 lanes (a lane-masked DMA invites the compiler
// to merge calls across divergent branches, and the LDS base of the merged
// call would no longer be uniform), so each piece's LDS span is rounded up to
// whole instructions and surplus lanes re-read the piece's last granule.
__host__ __device__ constexpr int gran_of(int bytes, int row) {
  return (bytes % 1024 == 0 && row % 16 == 0) ? 16 : 4;
}
__host__ __device__ constexpr int span_of(int bytes, int row) {
  return (bytes + 64 * gran_of(bytes, row) - 1) / (64 * gran_of(bytes, row)) * 64 * gran_of(bytes, row);
}

template <int D, int B1, int B2, int NR = 1>
struct Stage {
  using LY = Lay<D>;
  static constexpr int TPW = LY::TPW;
  static constexpr int R1 = D * B1 / 8;                 // code bytes per token, first plane
  static constexpr int R2 = D * (B2 ? B2 : 2) / 8;      // residual planes
  static constexpr int RS = 2 * LY::NG;                 // sz bytes per token
  static constexpr int C1 = TPW * R1, C2 = TPW * R2, SZ = TPW * RS;
  // alpha: a 2-byte DMA still advances 4 bytes per lane in LDS (token i at 4 i)
  static constexpr int AL = 64 * 4;
  static constexpr int k1c = 0;
  static constexpr int k1s = k1c + span_of(C1, R1);
  static constexpr int v1c = k1s + span_of(SZ, RS);
  static constexpr int v1s = v1c + span_of(C1, R1);
  // residual plane r (r < NR) occupies [res(r), res(r) + RSET): K codes, K sz,
  // V codes, V sz, K alpha, V alpha
  static constexpr int RES0 = v1s + span_of(SZ, RS);
  static constexpr int k2c = 0;
  static constexpr int k2s = k2c + span_of(C2, R2);
  static constexpr int v2c = k2s + span_of(SZ, RS);
  static constexpr int v2s = v2c + span_of(C2, R2);
  static constexpr int ka = v2s + span_of(SZ, RS);
  static constexpr int va = ka + AL;
  static constexpr int RSET = va + AL;
  static constexpr int res(int r) { return RES0 + r * RSET; }
  static constexpr int BYTES = RES0 + (B2 ? NR * RSET : 0);
  static constexpr int n_of(int bytes, int row) { return span_of(bytes, row) / (64 * gran_of(bytes, row)); }
  static constexpr int N_DMA = 2 * (n_of(C1, R1) + n_of(SZ, RS)) +
                               (B2 ? NR * 2 * (n_of(C2, R2) + n_of(SZ, RS) + 1) : 0);
  // ring depth (two measured faster than three for both kernel kinds)
  static constexpr int COUNT = 2;
  static_assert((COUNT - 1) * N_DMA < 64, "pending DMA count must fit vmcnt");
  static_assert(R1 % 4 == 0 && R2 % 4 == 0 && RS % 4 == 0, "token rows are whole dwords");
};

// DMA of one plane piece (BYTES of tokens ROW bytes each) from buffer offset
// `so` into LDS `dst`: lane l of instruction c moves granule c*64 + l.  Lanes
// past the piece, and in a partial tile lanes past `valid` (the bytes of the
// in-range tokens), re-read the last granule in range, so nothing outside the
// range is read and every staged value stays finite.
// Key code planes read by the matrix-core logits at head_dim 128 land
// swizzled inside each token row, so that those reads hit distinct LDS banks:
// lane (token n, block kb) reads 16 bytes (4-bit codes) or 8 bytes (2-bit) of
// row n, and the sixteen rows of a read are 64 or 32 bytes apart, which put
// rows n and n + 4 (n + 8) on the same banks.  Row t's chunk c (16 or 8
// bytes) is stored at chunk (c + rot(t)) mod 4, rot(t) = t / 4 (4-bit rows of
// 64 bytes) or 2 (t / 8) (2-bit rows of 32 bytes).  Only the DMA's per-lane
// global offsets change: slot s of the staged tile takes the byte the
// permutation sends there.
template <int ROW>
struct KSwz {
  static constexpr int CH = ROW / 4;  // chunk bytes
  __host__ __device__ static constexpr int rot(int t) { return ROW == 64 ? t / 4 : 2 * (t / 8); }
  // byte offset, in the tile, of the global byte staged at tile byte `slot`
  __host__ __device__ static constexpr int src(int slot) {
    return (slot / ROW) * ROW + (((slot % ROW) / CH - rot(slot / ROW)) & 3) * CH + slot % CH;
  }
  // tile byte where chunk c of row t is staged
  __host__ __device__ static constexpr int dst(int t, int c) { return t * ROW + ((c + rot(t)) & 3) * CH; }
};

template <int BYTES, int ROW, bool FULL, bool SWZ = false>
__device__ __forceinline__ void dma_piece(rsrc_t r, uint32_t so, int valid, lds_u8* dst, int lane) {
  constexpr int G = gran_of(BYTES, ROW), STEP = 64 * G, N = span_of(BYTES, ROW) / STEP;
  static_assert(!SWZ || ((ROW == 64 && G == 16) || (ROW == 32 && G == 4)) && BYTES % STEP == 0,
                "swizzled planes: whole rows per instruction, granules inside one chunk");
#pragma unroll
  for (int c = 0; c < N; ++c) {
    const int s = c * STEP + lane * G;                // staged byte of this lane
    const int o = SWZ ? KSwz<ROW>::src(s) : s;        // tile byte it takes
    if constexpr (FULL) {
      // the c * STEP part rides in the scalar offset
      const int vo = (SWZ || c * STEP + STEP <= BYTES) ? o - c * STEP : min(o, BYTES - G) - c * STEP;
      dma1<G, true>(r, dst + c * STEP, vo, so + c * STEP);
    } else {
      dma1<G, true>(r, dst + c * STEP, min(o, valid - G), so);
    }
  }
}

template <int BYTES>
__device__ __forceinline__ void lds_codes(const lds_u8* p, uint32_t* w) {
  typedef __attribute__((address_space(3))) const u32x2 l2;
  typedef __attribute__((address_space(3))) const uint32_t l1;
  if constexpr (BYTES == 8) {
    const u32x2 v = *reinterpret_cast<l2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else {
    static_assert(BYTES == 4, "a lane holds 16 codes of 2 or 4 bits");
    w[0] = *reinterpret_cast<l1*>(p);
  }
}

// One plane of one token pair as a lane sees it: 16 codes of each token and
// the (scale, offset) bytes of its group.
template <int BITS>
struct PairPlane {
  static constexpr int CW = 16 * BITS / 32;  // code dwords per token
  uint32_t c0[CW], c1[CW];
  uint32_t sz0, sz1;
};

template <int BITS>
__device__ __forceinline__ void lds_pair(PairPlane<BITS>& pp, const lds_u8* codes, const lds_u8* sz,
                                         int row, int rs) {
  constexpr int CB = 16 * BITS / 8;
  lds_codes<CB>(codes, pp.c0);
  lds_codes<CB>(codes + row, pp.c1);
  pp.sz0 = lds_u16(sz);
  pp.sz1 = lds_u16(sz + rs);
}

// ------------------------------------------------------------ K side on MFMA
// At head_dim 128 the logits of a wave tile (16 tokens) come from
// v_mfma_f32_16x16x32_f16 with the roles A = query, B = codes, D[row][token]:
// rows 0-7 are the anchor (first plane) groups, rows 8-15 the residual
// groups.  Lane (token n = lane % 16, block kb = lane / 16) holds B for its
// token: slab j (32 elements) takes 8 codes of group 2 kb + j / 2 as four
// magic-number pairs -- for 4-bit codes all of dword j of the lane's 16
// bytes, for 2-bit codes pairs 4 (j % 2) .. + 3 of dword j / 2 of its 8 bytes.
// The query operand is block diagonal: lane (row i, block kb) holds, for slab
// j, the fp16 pairs of group 2 kb + j / 2 when row i is that group's row (the
// same pairs the per-pair dot products use, in the same order), else zeros.
// The residual plane runs twice against the high and the low fp16 parts of
// H q, both into its rows, so D holds each group's code dot product plus the
// magic constant.  Lane (n, block rb) then owns rows 4 rb .. 4 rb + 3 of token
// n and applies their scales, offsets and alpha.
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

template <int BITS, int J>
__device__ __forceinline__ h8 kslab(const uint32_t* c, uint32_t magic) {
  if constexpr (BITS == 4) {
    const uint32_t d = c[J];
    const u32x4 v = {and_or(d, Pairs<4>::mask(0), magic), and_or(d, Pairs<4>::mask(1), magic),
                     and_or(d >> 8, Pairs<4>::mask(2), magic), and_or(d >> 8, Pairs<4>::mask(3), magic)};
    return __builtin_bit_cast(h8, v);
  } else {
    const uint32_t d = c[J / 2];
    constexpr int K0 = 4 * (J % 2);
    const u32x4 v = {__builtin_bit_cast(uint32_t, pair_of<2, K0>(d, magic)),
                     __builtin_bit_cast(uint32_t, pair_of<2, K0 + 1>(d, magic)),
                     __builtin_bit_cast(uint32_t, pair_of<2, K0 + 2>(d, magic)),
                     __builtin_bit_cast(uint32_t, pair_of<2, K0 + 3>(d, magic))};
    return __builtin_bit_cast(h8, v);
  }
}

// The lane's code dwords of one plane of token n: 16 bytes (4-bit codes) or
// 8 bytes (2-bit codes), block kb of the token's row, staged at p.
template <int BITS>
__device__ __forceinline__ void kcodes(const lds_u8* p, uint32_t* c) {
  constexpr int W = BITS;  // dwords per lane: 4 or 2
  if constexpr (W == 4) {
    typedef __attribute__((address_space(3))) const u32x4 l4;
    const u32x4 v = *reinterpret_cast<l4*>(p);
    c[0] = v.x; c[1] = v.y; c[2] = v.z; c[3] = v.w;
  } else {
    lds_codes<8>(p, c);
  }
}

// ------------------------------------------------------------ query side
// fp16 pairs matching the code pairs of one token's 16 codes (plane BITS),
// plus the constant 1024 * sum(pair) that the magic exponent adds.
template <int BITS>
struct QPairs {
  static constexpr int N = 8;  // 16 elements
  h2 p[N];
  float off;
};

// Element indices (in the lane's group) of code pair k of dword dw.
template <int BITS>
__host__ __device__ constexpr int elem_lo(int dw, int k) { return dw * (32 / BITS) + k; }
template <int BITS>
__host__ __device__ constexpr int elem_hi(int dw, int k) { return dw * (32 / BITS) + k + 16 / BITS; }

// Pair k of a group (runtime k): its two element indices and the bit
// position of its codes, matching pair_of<BITS, k mod units> on dword k / units.
template <int BITS>
__device__ __forceinline__ void pair_layout(int k, int& ea, int& eb, int& pos) {
  constexpr int PU = Pairs<BITS>::PER_UNIT;
  const int dw = k / PU, kk = k % PU;
  ea = dw * (32 / BITS) + kk;
  eb = ea + 16 / BITS;
  pos = BITS == 4 ? 4 * (kk & 1) : 2 * (kk < 5 ? kk : kk - 5);
}

// sum_i w_i c_i over one token's 16 codes, times the prescale (plus the magic
// offset, removed by starting from -off).
template <int BITS>
__device__ __forceinline__ float key_dot(const uint32_t* c, const QPairs<BITS>& qp, uint32_t magic) {
  using PR = Pairs<BITS>;
  float acc = -qp.off;
#pragma unroll
  for (int dw = 0; dw < 16 * BITS / 32; ++dw)
    static_for<PR::PER_UNIT>([&](auto K) {
      acc = __builtin_amdgcn_fdot2(pair_of<BITS, K>(c[dw], magic), qp.p[dw * PR::PER_UNIT + K], acc,
                                   false);
    });
  return acc;
}

template <int BITS>
__device__ __forceinline__ float key_dot2(const uint32_t* c, const QPairs<BITS>& hi, const QPairs<BITS>& lo,
                                          uint32_t magic) {
  using PR = Pairs<BITS>;
  float acc = -hi.off;
#pragma unroll
  for (int dw = 0; dw < 16 * BITS / 32; ++dw)
    static_for<PR::PER_UNIT>([&](auto K) {
      const h2 x = pair_of<BITS, K>(c[dw], magic);
      acc = __builtin_amdgcn_fdot2(x, hi.p[dw * PR::PER_UNIT + K], acc, false);
      acc = __builtin_amdgcn_fdot2(x, lo.p[dw * PR::PER_UNIT + K], acc, false);
    });
  return acc;
}

// acc_i += w_t (1024 + m_i c_{t,i}) + w_t' (1024 + m_i c_{t',i}) for the 16
// elements: v_perm_b32 interleaves unit u of the two tokens, then each code
// pair feeds one dot2 against the weight pair (two with HILO: the weights as
// an fp16 high part plus an fp16 low part).
template <int BITS, bool HILO>
__device__ __forceinline__ void value_acc(const PairPlane<BITS>& pp, h2 wh, h2 wl, float* acc,
                                          uint32_t magic) {
  using PR = Pairs<BITS>;
#pragma unroll
  for (int dw = 0; dw < PairPlane<BITS>::CW; ++dw) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // bytes 2h, 2h+1 of token t (low half) and of token t' (high half)
      const uint32_t x = __builtin_amdgcn_perm(pp.c1[dw], pp.c0[dw], h ? 0x07060302u : 0x05040100u);
      const int base = (2 * dw + h) * PR::PER_UNIT;
      static_for<PR::PER_UNIT>([&](auto K) {
        const h2 c = pair_of<BITS, K>(x, magic);
        acc[base + K] = __builtin_amdgcn_fdot2(c, wh, acc[base + K], false);
        if constexpr (HILO) acc[base + K] = __builtin_amdgcn_fdot2(c, wl, acc[base + K], false);
      });
    }
  }
}

// NR > 1 (chained mode): loop a.loop reads the residual planes of loops
// a.loop .. a.loop + NR - 1, all accumulated into the one residual sum.
// PAGED: row b's tokens live in the pool blocks its block-table row names; a
// wave tile (TPW tokens, block sizes are powers of two >= TPW) never straddles
// two blocks, so the tile's buffer resources are rebuilt from its block's
// slots, with the block id read through the scalar cache.
template <int D, int B1, int B2, int NR, bool PAGED, int NWK>
__global__ void __launch_bounds__(NWK * 64, NWK == 8 ? 2 : 3) decode_kernel(DecodeArgs a) {
  using LY = Lay<D>;
  constexpr int NG = LY::NG, LPP = LY::LPP, TPW = LY::TPW;
  constexpr bool TWO = B2 != 0;
  constexpr int B2E = TWO ? B2 : 2;
  constexpr int CB1 = 16 * B1 / 8, CB2 = 16 * B2E / 8;  // code bytes per lane and token
  // logits on matrix cores (see kslab): head_dim 128 and 96 with at most one
  // residual plane; chained loops reading several planes keep the dot2 path.
  // At 96 the rows of groups 6 and 7 (and 14, 15) are empty: their query
  // rows are zero and their scale / offset terms are dropped, and the code
  // slab of lane block 3 reads the next bytes of the staged tile (finite
  // codes that meet only zero query entries)
  constexpr bool KM = (D == 128 || D == 96) && NR == 1;
  constexpr bool SWK = KM && D == 128;   // key code planes staged swizzled (KSwz)
  const Geometry& g = a.g;

  using ST = Stage<D, B1, B2, NR>;
  constexpr int kStaging = NWK * ST::COUNT * ST::BYTES;
  constexpr int kRow = (TWO ? 2 * D : D) + 1;              // accA | accR | l
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStaging];
  // each wave's sums, written as soon as its last tile is done (their own
  // space, so no wave waits for the others before reducing its state)
  constexpr int kRowP = (kRow + 3) / 4 * 4;  // rows 16-byte aligned
  __shared__ __attribute__((aligned(16))) float sm_acc[NWK][kRowP];
  __shared__ float sq[D], su[D];
  __shared__ float s_scale[2];
  // per-group query pairs; rows padded to 36 dwords so that the 16-byte
  // reads of the eight groups' rows fall in eight different bank quads
  __shared__ __attribute__((aligned(16))) uint32_t spre[8][36];
  __shared__ float sm_m[NWK];
  __shared__ uint32_t s_ticket;
  __shared__ uint32_t s_claim;   // next unclaimed wave tile of this split
  // the query row (BF16) and this layer's key signs, staged by DMA
  __shared__ __attribute__((aligned(16))) uint8_t s_in[512];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (row, split): the first rows_lo rows take splits_lo splits
  // each, the others a.splits (a balanced plan; rows_lo is 0 otherwise)
  int split, bh;
  {
    const int wg = blockIdx.x, nlo = a.rows_lo * a.splits_lo;
    if (wg < nlo) {
      bh = wg / a.splits_lo;
      split = wg - bh * a.splits_lo;
    } else {
      const int r = (wg - nlo) / a.splits;
      bh = a.rows_lo + r;
      split = wg - nlo - r * a.splits;
    }
  }
  const bool lo_row = bh < a.rows_lo;
  const int ns = lo_row ? a.splits_lo : a.splits;                       // this row's splits
  const int tps = lo_row ? a.tokens_per_split_lo : a.tokens_per_split;
  const int b = bh / a.q_heads, hq = bh % a.q_heads, kvh = hq / a.group_ratio;
  const int pj = lane / LPP, e = lane % LPP;   // token pair, group
  const bool active = e < NG;
  const int eg = active ? e : NG - 1;           // idle lanes (d = 96) shadow the last group
  const bool rotated = TWO && g.rotation == RQ_ROT_HADAMARD;
  uint32_t magic;
  asm("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kMagic));

  // tokens of this batch row (per-row lengths come from device memory and are
  // clamped to the planned maximum)
  const int n_row = a.lengths ? min(max(a.lengths[b], 0), a.n_tokens) : a.n_tokens;
  const int t_begin = split * tps;
  const int t_end = min(n_row, t_begin + tps);

  // ---- buffer resources.  Contiguous cache: one per plane (a slot, or a
  // residual plane's alpha row), its pieces at offset 0.  Paged pool: one
  // over the tile's pool block in the K half of the pool and one in the V
  // half, rebuilt per tile, with every plane at its offset inside the block
  // (the same for K and V), so the per-tile state stays small.
  const int loop1 = (g.mode == RQ_MODE_DIRECT || !TWO) ? a.loop : (a.loop - a.loop % g.P + g.P - 1);
  const uint32_t sb1 = (uint32_t)g.slot_bytes[g.is_anchor(loop1) ? 0 : 1];
  const uint32_t sb2 = (uint32_t)g.slot_bytes[g.is_anchor(a.loop) ? 0 : 1];
  const uint32_t arow = (uint32_t)g.alpha_row;
  const int brow = PAGED ? 0 : b;
  // plane offsets in the K half (paged: inside pool block 0, under 4 GiB)
  const uint64_t o1 = g.slot_offset(0, brow, a.layer, loop1, kvh);
  uint64_t o2[NR], oa[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    o2[r] = g.slot_offset(0, brow, a.layer, a.loop + r, kvh);
    oa[r] = TWO ? g.alpha_offset(0, brow, a.layer, a.loop + r, kvh) : 0;
  }
  const uint64_t vhalf = (uint64_t)g.batch * g.layers * g.layer_block;  // K -> V
  const uint64_t bstride = (uint64_t)g.layers * g.layer_block;          // one pool block
  rsrc_t rk1, rv1, rk2[NR], rv2[NR], rka[NR], rva[NR];
  uint32_t po1 = 0, po2[NR], poa[NR];  // paged: plane offsets inside the block
#pragma unroll
  for (int r = 0; r < NR; ++r) po2[r] = poa[r] = 0;
  if constexpr (!PAGED) {
    rk1 = make_rsrc(a.cache + o1, sb1);
    rv1 = make_rsrc(a.cache + vhalf + o1, sb1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      rk2[r] = make_rsrc(a.cache + o2[r], sb2);
      rv2[r] = make_rsrc(a.cache + vhalf + o2[r], sb2);
      if constexpr (TWO) {
        rka[r] = make_rsrc(a.cache + oa[r], arow);
        rva[r] = make_rsrc(a.cache + vhalf + oa[r], arow);
      }
    }
  } else {
    po1 = (uint32_t)o1;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      po2[r] = (uint32_t)o2[r];
      poa[r] = (uint32_t)oa[r];
    }
  }
  auto point_at = [&](uint64_t delta) __attribute__((always_inline)) {
    const rsrc_t rk = make_rsrc(a.cache + delta, (uint32_t)bstride);
    const rsrc_t rv = make_rsrc(a.cache + vhalf + delta, (uint32_t)bstride);
    rk1 = rk;
    rv1 = rv;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      rk2[r] = rka[r] = rk;
      rv2[r] = rva[r] = rv;
    }
  };
  // block-table row of this sequence, read through the scalar cache
  typedef const __attribute__((address_space(4))) int32_t c_i32;
  const c_i32* btab = (const c_i32*)(a.paging.table + (uint64_t)b * a.paging.max_blocks);
  const uint32_t s1rel = po1 + (uint32_t)g.sz_rel(loop1);

  // ---- stream the split's wave tiles (tile k: TPW tokens from t_begin +
  // k TPW) through each wave's LDS ring.  Waves start with tiles w and
  // NWK + w; after that each wave claims the next unclaimed tile of the split
  // from an LDS counter, one tile ahead.  With a fixed tile-to-wave mapping
  // the second wave on each SIMD, which loses issue arbitration to the
  // first, finished its equal share about 5 us later (residual call at 8k
  // tokens, batch 4); claiming keeps every wave busy until the split is done.
  // The order in which tiles are summed therefore varies from call to call:
  // results agree to fp32 summation order, not bit for bit.
  static_assert(ST::COUNT == 2, "the claim schedule runs a two-slot ring");
  lds_u8* ring = (lds_u8*)smem + w * ST::COUNT * ST::BYTES;
  const int n_tot = t_end > t_begin ? (t_end - t_begin + TPW - 1) / TPW : 0;
  int kcur = w, knext = NWK + w;   // tile being computed, tile after it
  uint32_t claimed = 0;             // lane 0: the tile claimed for the one after
  auto issue_t = [&](auto full, uint32_t tb, lds_u8* st, int vt) __attribute__((always_inline)) {
    constexpr bool F = decltype(full)::value;
    dma_piece<ST::C1, ST::R1, F, SWK>(rk1, po1 + tb * ST::R1, vt * ST::R1, st + ST::k1c, lane);
    dma_piece<ST::SZ, ST::RS, F>(rk1, s1rel + tb * ST::RS, vt * ST::RS, st + ST::k1s, lane);
    dma_piece<ST::C1, ST::R1, F>(rv1, po1 + tb * ST::R1, vt * ST::R1, st + ST::v1c, lane);
    dma_piece<ST::SZ, ST::RS, F>(rv1, s1rel + tb * ST::RS, vt * ST::RS, st + ST::v1s, lane);
    if constexpr (TWO) {
      const uint32_t s2rel = (uint32_t)g.sz_rel(a.loop);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        lds_u8* rs = st + ST::res(r);
        dma_piece<ST::C2, ST::R2, F, SWK>(rk2[r], po2[r] + tb * ST::R2, vt * ST::R2, rs + ST::k2c,
                                          lane);
        dma_piece<ST::SZ, ST::RS, F>(rk2[r], po2[r] + s2rel + tb * ST::RS, vt * ST::RS, rs + ST::k2s,
                                     lane);
        dma_piece<ST::C2, ST::R2, F>(rv2[r], po2[r] + tb * ST::R2, vt * ST::R2, rs + ST::v2c, lane);
        dma_piece<ST::SZ, ST::RS, F>(rv2[r], po2[r] + s2rel + tb * ST::RS, vt * ST::RS, rs + ST::v2s,
                                     lane);
        dma_alpha(rka[r], poa[r] + tb * 2, F ? TPW : vt, rs + ST::ka, lane);
        dma_alpha(rva[r], poa[r] + tb * 2, F ? TPW : vt, rs + ST::va, lane);
      }
    }
  };
  auto issue = [&](int k, int slot) __attribute__((always_inline)) {
    uint32_t tb = (uint32_t)(t_begin + k * TPW);
    lds_u8* st = ring + slot * ST::BYTES;
    const int vt = t_end - (int)tb;  // in-range tokens of this tile (>= 1)
    if constexpr (PAGED) {
      // ids outside the pool are clamped into it: garbage in, but no read
      // outside the cache
      const int blk = min(max(btab[tb >> a.paging.block_shift], 0), g.batch - 1);
      point_at((uint64_t)blk * bstride);
      tb &= (1u << a.paging.block_shift) - 1u;
    }
    if (vt >= TPW)
      issue_t(std::integral_constant<bool, true>{}, tb, st, TPW);
    else
      issue_t(std::integral_constant<bool, false>{}, tb, st, vt);
  };
  // Wave 0 stages the query row and the key signs by DMA ahead of its tiles:
  // a plain load issued after the tiles' DMAs would wait for all of them
  if (w == 0) {
    dma1<4>(make_rsrc((const uint8_t*)(a.q + (uint64_t)bh * D), 2 * D), (lds_u8*)s_in,
            min(4 * lane, 2 * D - 4), 0u);
    if (rotated)
      dma1<4>(make_rsrc((const uint8_t*)(a.signs + (uint64_t)a.layer * D), D), (lds_u8*)s_in + 256,
              min(4 * lane, D - 4), 0u);
  }
  // One tile per wave goes in flight before the query side is built; the
  // second slot is filled at the top of the first iteration.  Filling the
  // whole ring here put twice the bytes (17 MB over the grid at 8k tokens,
  // batch 4) ahead of every workgroup's first tile: the call measured about
  // 1 us longer at 8k and at 16k tokens.
  if (kcur < n_tot) issue(kcur, 0);
  if (tid == 0) s_claim = 2 * NWK;

  // ---- query side, once per workgroup (wave 0): q, u = H q, their fp16
  // prescales, and for every group the fp16 pairs matching the code pairs,
  // the magic constants 1024 * sum(pair) and the plain sums
  if (w == 0) {
    // the staged row has landed once at most the first tile's DMAs are pending
    if (kcur < n_tot) wait_vm<ST::N_DMA>();
    else wait_vm<0>();
    const bool v1ok = (D > 64) && (lane + 64 < D);
    const lds_u8* qin = (const lds_u8*)s_in;
    const float q0 = bf16_to_f32(lds_u16(qin + 2 * lane));
    const float q1 = v1ok ? bf16_to_f32(lds_u16(qin + 2 * (lane + 64))) : 0.f;
    sq[lane] = q0;
    if (v1ok) sq[lane + 64] = q1;
    float u0 = q0, u1 = q1;
    if (rotated) {
      const int8_t* sg = (const int8_t*)(s_in + 256);  // K signs of this layer
      u0 *= (float)sg[lane];
      u1 = v1ok ? u1 * (float)sg[lane + 64] : 0.f;
      wave_wht<D>(u0, u1, lane);
      u0 *= (D == 128) ? 0.08838834764831845f : 0.125f;
      u1 = v1ok ? u1 * ((D == 128) ? 0.08838834764831845f : 0.17677669529663687f) : 0.f;
    }
    if (TWO) {
      su[lane] = u0;
      if (v1ok) su[lane + 64] = u1;
    }
    const float pq0 = fp16_prescale(wave_max(fmaxf(fabsf(q0), fabsf(q1))));
    const float pu0 = TWO ? fp16_prescale(wave_max(fmaxf(fabsf(u0), fabsf(u1)))) : 1.f;
    if (lane == 0) {
      s_scale[0] = pq0;
      s_scale[1] = pu0;
    }
    // lane = (group g, pair k); sq / su were written by this same wave
    const int g8 = lane >> 3, k = lane & 7;
    const int gg = g8 < NG ? g8 : NG - 1;
    int ea, eb, pos;
    pair_layout<B1>(k, ea, eb, pos);
    float qa = sq[gg * 16 + ea], qb = sq[gg * 16 + eb];
    const float im = 1.f / (float)(1 << pos);
    const _Float16 ha = (_Float16)(qa * pq0 * im), hb = (_Float16)(qb * pq0 * im);
    float offq = 1024.f * ((float)ha + (float)hb), qsum = qa + qb;
    uint32_t uhw = 0, ulw = 0;
    float offu = 0.f, usum = 0.f;
    if constexpr (TWO) {
      pair_layout<B2E>(k, ea, eb, pos);
      const float ua = su[gg * 16 + ea], ub = su[gg * 16 + eb];
      const float iu = 1.f / (float)(1 << pos);
      const float xa = ua * pu0 * iu, xb = ub * pu0 * iu;
      const _Float16 ya = (_Float16)xa, yb = (_Float16)xb;
      const _Float16 za = (_Float16)(xa - (float)ya), zb = (_Float16)(xb - (float)yb);
      uhw = __builtin_bit_cast(uint32_t, (h2){ya, yb});
      ulw = __builtin_bit_cast(uint32_t, (h2){za, zb});
      offu = 1024.f * (((float)ya + (float)yb) + ((float)za + (float)zb));
      usum = ua + ub;
    }
    offq = pair_sum<8>(offq);
    qsum = pair_sum<8>(qsum);
    offu = pair_sum<8>(offu);
    usum = pair_sum<8>(usum);
    // rows of groups past NG (d = 96) are zero: the matrix-core logits read
    // them as empty query rows
    const bool gv = g8 < NG;
    spre[g8][k] = gv ? __builtin_bit_cast(uint32_t, (h2){ha, hb}) : 0u;
    spre[g8][8 + k] = gv ? uhw : 0u;
    spre[g8][16 + k] = gv ? ulw : 0u;
    if (k == 0) {
      spre[g8][24] = gv ? __builtin_bit_cast(uint32_t, offq) : 0u;
      spre[g8][25] = gv ? __builtin_bit_cast(uint32_t, offu) : 0u;
      spre[g8][26] = gv ? __builtin_bit_cast(uint32_t, qsum) : 0u;
      spre[g8][27] = gv ? __builtin_bit_cast(uint32_t, usum) : 0u;
    }
  }
  __syncthreads();

  // ---- this lane's group of the query: the sums stay in registers; the fp16
  // pairs are re-read from LDS every tile (broadcast reads), which keeps 24
  // VGPRs free for occupancy
  const float pq = s_scale[0], pu = s_scale[1];
  const float qoff = __builtin_bit_cast(float, spre[eg][24]);
  const float uoff = __builtin_bit_cast(float, spre[eg][25]);
  const float qsum = __builtin_bit_cast(float, spre[eg][26]);
  const float usum = TWO ? __builtin_bit_cast(float, spre[eg][27]) : 0.f;
  typedef __attribute__((address_space(3))) const u32x4 lq4;
  const lq4* prow = (const lq4*)((lds_u8*)&spre[0][0] + eg * (int)sizeof(spre[0]));
  const float ipq = 1.f / pq, ipu = 1.f / pu;
  const float qs = a.qscale;
  const h2 ones = (h2){(_Float16)1.f, (_Float16)1.f};

  // K side on matrix cores: the block-diagonal query operands (slab j:
  // anchor, residual high part, residual low part) and, for the lane's rows,
  // the groups' magic constants and plain query sums
  const int kn = lane & 15, kb = lane >> 4;
  // where the lane's code chunks sit in a staged tile (swizzled at d = 128)
  const int kofs1 = SWK ? KSwz<ST::R1>::dst(kn, kb) : kn * ST::R1 + kb * 4 * B1;
  const int kofs2 = SWK ? KSwz<ST::R2>::dst(kn, kb) : kn * ST::R2 + kb * 4 * B2E;
  h8 Aq[4], Auh[4], Aul[4];
  float koff[4], ksum[4];
  const bool kres = TWO && kb >= 2;   // lane's rows are residual rows
  if constexpr (KM) {
    typedef __attribute__((address_space(3))) const u32x4 lq4k;
    static_for<4>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const int gj = 2 * kb + j / 2;   // rows of groups past NG are zero in spre
      const lds_u8* row = (const lds_u8*)&spre[gj][0] + 16 * (j % 2);
      // lane kn holds row kn: its query entries where it is group gj's row
      const uint32_t mq = kn == gj ? ~0u : 0u, mu = kn == 8 + gj ? ~0u : 0u;
      Aq[j] = __builtin_bit_cast(h8, *reinterpret_cast<lq4k*>(row) & mq);
      if constexpr (TWO) {
        Auh[j] = __builtin_bit_cast(h8, *reinterpret_cast<lq4k*>(row + 32) & mu);
        Aul[j] = __builtin_bit_cast(h8, *reinterpret_cast<lq4k*>(row + 64) & mu);
      }
    });
    // the row sums are in prescaled units (the dot products carry the
    // query's power-of-two prescale, taken out once per row below), so the
    // query sums that meet the offsets are prescaled too (exactly)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gr = 4 * (kb & 1) + r;
      const bool live = (TWO || kb < 2) && gr < NG;
      koff[r] = live ? __builtin_bit_cast(float, spre[gr][kres ? 25 : 24]) : 0.f;
      ksum[r] = live ? __builtin_bit_cast(float, spre[gr][kres ? 27 : 26]) * (kres ? pu : pq) : 0.f;
    }
  }

  float accA[16], accR[TWO ? 16 : 1];
#pragma unroll
  for (int i = 0; i < 16; ++i) accA[i] = 0.f;
#pragma unroll
  for (int i = 0; i < (TWO ? 16 : 1); ++i) accR[i] = 0.f;
  float WA = 0.f, WR = 0.f, zA = 0.f, zR = 0.f;  // fp16 weight sums, offset sums
  float m = kEmpty, l = 0.f;

  // lane-constant LDS offsets inside a tile buffer: the lane's tokens are
  // pj and pj + TS of the tile.  (Tokens 2 pj and 2 pj + 1 put the rows read
  // by one half-wave 2 rows apart, so rows 4 apart met in the same LDS banks;
  // with pj the rows read together are consecutive.)
  constexpr int TS = LY::PAIRS;
  const int t0 = pj;
  const int o1c = t0 * ST::R1 + eg * CB1, o2c = t0 * ST::R2 + eg * CB2;
  const int osz = t0 * ST::RS + eg * 2, oal = t0 * 4;

  // the claim for the third tile; its result is read after the first tile
  auto claim = [&]() __attribute__((always_inline)) {
    if (lane == 0)
      claimed = __hip_atomic_fetch_add(&s_claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  claim();
  // one loop body for every stage: stage-specialized copies would make the
  // compiler shuffle all live accumulators between them on every iteration.
  // Tiles are claimed in increasing order, so once knext is past the split
  // every later claim is too.
  for (int it = 0; kcur < n_tot; ++it) {
    // slot (it & 1) holds kcur; knext goes to the other slot
    if (knext < n_tot) issue(knext, (it + 1) & 1);
    if (it > 0) claim();
    // wait for kcur: the tile issued after it may stay in flight
    if (knext < n_tot) wait_vm<ST::N_DMA>();
    else wait_vm<0>();
    const lds_u8* st = ring + (it & 1) * ST::BYTES;
    if constexpr (NWK == 4) {
      // Four-wave workgroups share a CU with two or three others, and the
      // oldest waves win issue arbitration: with equal priorities the first
      // workgroup on a CU finished its split early and the last ran on alone
      // at a third of the CU's waves (Huginn-like shapes: loop times 17-40 us
      // for equal splits).  A wave's issue priority follows the share of
      // its split still unclaimed, so workgroups that lag catch up.
      const int left4 = 4 * (n_tot - kcur);
      if (left4 > 3 * n_tot) __builtin_amdgcn_s_setprio(3);
      else if (left4 > 2 * n_tot) __builtin_amdgcn_s_setprio(2);
      else if (left4 > n_tot) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    const int tt = t_begin + kcur * TPW + t0;
    const bool ok0 = tt < t_end, ok1 = tt + TS < t_end;

    float lg0, lg1;
    if constexpr (KM) {
      // ---- logits on matrix cores: D[group row][token] for the 16 tokens
      f4 dk = {0.f, 0.f, 0.f, 0.f};
      uint32_t c1[B1];
      kcodes<B1>(st + ST::k1c + kofs1, c1);
      h8 kb1[4], kb2[4];
      static_for<4>([&](auto J) { kb1[decltype(J)::value] = kslab<B1, decltype(J)::value>(c1, magic); });
      const lds_u8* rs = st + ST::res(0);
      if constexpr (TWO) {
        uint32_t c2[B2E];
        kcodes<B2E>(rs + ST::k2c + kofs2, c2);
        static_for<4>([&](auto J) { kb2[decltype(J)::value] = kslab<B2E, decltype(J)::value>(c2, magic); });
      }
      static_for<4>([&](auto J) {
        constexpr int j = decltype(J)::value;
        dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aq[j], kb1[j], dk, 0, 0, 0);
      });
      if constexpr (TWO) {
        static_for<4>([&](auto J) {
          constexpr int j = decltype(J)::value;
          dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(Auh[j], kb2[j], dk, 0, 0, 0);
          dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aul[j], kb2[j], dk, 0, 0, 0);
        });
      }
      // the lane's four rows: scale times (dot - magic) plus offset times the
      // query sum, then alpha for residual rows, summed over the four blocks
      typedef __attribute__((address_space(3))) const u32x2 lq2;
      const lds_u8* szp = (kres ? rs + ST::k2s : st + ST::k1s) + kn * ST::RS + 8 * (kb & 1);
      u32x2 szw;
      if constexpr (D == 128) {
        szw = *reinterpret_cast<lq2*>(szp);
      } else {
        // 12-byte rows: dword reads; groups 6 and 7 do not exist
        szw.x = lds_u32(szp);
        szw.y = (kb & 1) ? 0u : lds_u32(szp + 4);
      }
      const f2 sz0 = sz_pair(szw.x), sz1 = __builtin_amdgcn_cvt_pk_f32_fp8(szw.x, true);
      const f2 sz2 = sz_pair(szw.y), sz3 = __builtin_amdgcn_cvt_pk_f32_fp8(szw.y, true);
      float kp = fmaf(sz0.x, dk[0] - koff[0], sz0.y * ksum[0]);
      kp = fmaf(sz1.x, dk[1] - koff[1], fmaf(sz1.y, ksum[1], kp));
      kp = fmaf(sz2.x, dk[2] - koff[2], fmaf(sz2.y, ksum[2], kp));
      kp = fmaf(sz3.x, dk[3] - koff[3], fmaf(sz3.y, ksum[3], kp));
      float kmul = ipq;
      if constexpr (TWO) kmul = kres ? ipu * bf16_to_f32(lds_u16(rs + ST::ka + 4 * kn)) : ipq;
      kp = (TWO || kb < 2) ? kp * kmul : 0.f;
      kp = pair_add<32>(pair_add<16>(kp)) * qs;   // logit of token kn
      // to the value side's layout: lane (pair pj, group e) takes tokens pj, pj + TS
      const int kbits = __builtin_bit_cast(int, kp);
      const float lk0 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * t0, kbits));
      const float lk1 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (t0 + TS), kbits));
      lg0 = ok0 ? lk0 : kEmpty;
      lg1 = ok1 ? lk1 : kEmpty;
    } else {
      // keys now; the value planes are read after the softmax update, so their
      // registers are not live across the logit computation
      PairPlane<B1> k1;
      lds_pair<B1>(k1, st + ST::k1c + o1c, st + ST::k1s + osz, TS * ST::R1, TS * ST::RS);

      // ---- logits of the pair
      asm volatile("" ::: "memory");  // keep the pair reads inside the loop
      QPairs<B1> qp;
      QPairs<B2E> uh, ul;
  #pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 x = prow[j];
        qp.p[4 * j] = as_h2(x.x);
        qp.p[4 * j + 1] = as_h2(x.y);
        qp.p[4 * j + 2] = as_h2(x.z);
        qp.p[4 * j + 3] = as_h2(x.w);
      }
      qp.off = qoff;
      if constexpr (TWO) {
  #pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 x = prow[2 + j], y = prow[4 + j];
          uh.p[4 * j] = as_h2(x.x);
          uh.p[4 * j + 1] = as_h2(x.y);
          uh.p[4 * j + 2] = as_h2(x.z);
          uh.p[4 * j + 3] = as_h2(x.w);
          ul.p[4 * j] = as_h2(y.x);
          ul.p[4 * j + 1] = as_h2(y.y);
          ul.p[4 * j + 2] = as_h2(y.z);
          ul.p[4 * j + 3] = as_h2(y.w);
        }
        uh.off = uoff;
        ul.off = 0.f;
      }
      float part0, part1;
      {
        f2 s0 = sz_pair(k1.sz0), s1 = sz_pair(k1.sz1);
        if (!active) s0 = s1 = (f2){0.f, 0.f};
        part0 = fmaf(s0.x * key_dot<B1>(k1.c0, qp, magic), ipq, s0.y * qsum);
        part1 = fmaf(s1.x * key_dot<B1>(k1.c1, qp, magic), ipq, s1.y * qsum);
      }
      if constexpr (TWO) {
  #pragma unroll
        for (int r = 0; r < NR; ++r) {
          const lds_u8* rs = st + ST::res(r);
          PairPlane<B2E> k2;
          lds_pair<B2E>(k2, rs + ST::k2c + o2c, rs + ST::k2s + osz, TS * ST::R2, TS * ST::RS);
          const uint32_t ka0 = lds_u16(rs + ST::ka + oal), ka1 = lds_u16(rs + ST::ka + oal + 4 * TS);
          f2 s0 = sz_pair(k2.sz0), s1 = sz_pair(k2.sz1);
          if (!active) s0 = s1 = (f2){0.f, 0.f};
          const float r0 = fmaf(s0.x * key_dot2<B2E>(k2.c0, uh, ul, magic), ipu, s0.y * usum);
          const float r1 = fmaf(s1.x * key_dot2<B2E>(k2.c1, uh, ul, magic), ipu, s1.y * usum);
          part0 = fmaf(bf16_to_f32(ka0), r0, part0);
          part1 = fmaf(bf16_to_f32(ka1), r1, part1);
        }
      }
      lg0 = ok0 ? pair_sum<LPP>(part0) * qs : kEmpty;
      lg1 = ok1 ? pair_sum<LPP>(part1) * qs : kEmpty;
    }

    // ---- online softmax
    const float mx = fmaxf(lg0, lg1);
    if (mx > m + kLazy) {
      const float corr = __builtin_amdgcn_exp2f(m - mx);
      l *= corr;
      WA *= corr;
      zA *= corr;
#pragma unroll
      for (int i = 0; i < 16; ++i) accA[i] *= corr;
      if constexpr (TWO) {
        WR *= corr;
        zR *= corr;
#pragma unroll
        for (int i = 0; i < 16; ++i) accR[i] *= corr;
      }
      m = mx;
    }
    const float p0 = ok0 ? __builtin_amdgcn_exp2f(lg0 - m) : 0.f;
    const float p1 = ok1 ? __builtin_amdgcn_exp2f(lg1 - m) : 0.f;
    l += p0 + p1;

    // ---- values
    PairPlane<B1> v1;
    lds_pair<B1>(v1, st + ST::v1c + o1c, st + ST::v1s + osz, TS * ST::R1, TS * ST::RS);
    {
      // first plane: fp16 high + low weights, so the weights are exact to ~2^-22
      f2 s0 = sz_pair(v1.sz0), s1 = sz_pair(v1.sz1);
      if (!active) s0 = s1 = (f2){0.f, 0.f};
      const float w0 = p0 * s0.x * kWA, w1 = p1 * s1.x * kWA;
      const h2 wh = (h2){(_Float16)w0, (_Float16)w1};
      const h2 wl = (h2){(_Float16)(w0 - (float)wh.x), (_Float16)(w1 - (float)wh.y)};
      WA = __builtin_amdgcn_fdot2(wh, ones, WA, false);
      WA = __builtin_amdgcn_fdot2(wl, ones, WA, false);
      zA = fmaf(p0, s0.y, fmaf(p1, s1.y, zA));
      value_acc<B1, true>(v1, wh, wl, accA, magic);
    }
    if constexpr (TWO) {
      // residual planes: single fp16 weights against codes centred on c0 (the
      // centre is added back exactly through the offset sum), which halves the
      // weight-rounding error of this smaller term
      constexpr float c0 = (float)((1 << B2E) - 1) * 0.5f;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const lds_u8* rs = st + ST::res(r);
        PairPlane<B2E> v2;
        lds_pair<B2E>(v2, rs + ST::v2c + o2c, rs + ST::v2s + osz, TS * ST::R2, TS * ST::RS);
        const uint32_t va0 = lds_u16(rs + ST::va + oal), va1 = lds_u16(rs + ST::va + oal + 4 * TS);
        f2 s0 = sz_pair(v2.sz0), s1 = sz_pair(v2.sz1);
        if (!active) s0 = s1 = (f2){0.f, 0.f};
        const float pa0 = p0 * bf16_to_f32(va0), pa1 = p1 * bf16_to_f32(va1);
        const h2 wr = (h2){(_Float16)(pa0 * s0.x * kWR), (_Float16)(pa1 * s1.x * kWR)};
        WR = __builtin_amdgcn_fdot2(wr, ones, WR, false);
        zR = fmaf(pa0, fmaf(s0.x, c0, s0.y), fmaf(pa1, fmaf(s1.x, c0, s1.y), zR));
        value_acc<B2E, false>(v2, wr, wr, accR, magic);
      }
    }
    // Every 8 tiles, fold the magic constant out of the value sums: each sum
    // holds sum w (1024 + m c), and left in place the 1024 sum w term grows
    // with every tile a lane adds, so the fp32 rounding of the small code term
    // would grow with the context.  The residual sums' centring term
    // (c0 sum w, see the final formula below) moves into their offset sum.
    if ((it & 7) == 7) {
#pragma unroll
      for (int i = 0; i < 16; ++i) accA[i] = fmaf(-1024.f, WA, accA[i]);
      WA = 0.f;
      if constexpr (TWO) {
        constexpr float c0 = (float)((1 << B2E) - 1) * 0.5f;
#pragma unroll
        for (int i = 0; i < 16; ++i) accR[i] = fmaf(-1024.f, WR, accR[i]);
        zR = fmaf(-c0 / kWR, WR, zR);
        WR = 0.f;
      }
    }
    kcur = knext;
    knext = (int)__builtin_amdgcn_readfirstlane(claimed);
  }

  // ---- take out the magic constant of the tiles since the last fold
  // (element i holds sum w (1024 + m_i c_i); the residual sum also takes out
  // its centre c0 * sum w) and align every lane to the wave maximum in the
  // same step
  const float Mw = wave_max(m);
  const float f = __builtin_amdgcn_exp2f(m - Mw);
  l *= f;
  static_for<16>([&](auto I) {
    constexpr int k1 = decltype(I)::value % Pairs<B1>::PER_UNIT;
    constexpr float mA = Pairs<B1>::mult(k1);
    accA[I] = fmaf(accA[I], f * (1.f / (mA * kWA)), f * (zA - WA * (1024.f / (mA * kWA))));
    if constexpr (TWO) {
      constexpr int k2 = decltype(I)::value % Pairs<B2E>::PER_UNIT;
      constexpr float mR = Pairs<B2E>::mult(k2);
      constexpr float c0 = (float)((1 << B2E) - 1) * 0.5f;
      accR[I] = fmaf(accR[I], f * (1.f / (mR * kWR)),
                     f * (zR - WR * (1024.f / (mR * kWR) + c0 / kWR)));
    }
  });
  // ---- sum over the wave's token pairs (the lane bits above the group
  // index) in registers, then the first pair's lanes write the wave's sums:
  // [wave][accA | accR | l]
  auto pairs_sum = [&](float v) __attribute__((always_inline)) {
    if constexpr (LPP == 4) v += xor_lane<4>(v, lane);
    v += dpp_f<kDppRowRor8>(v);
    return pair_add<32>(pair_add<16>(v));
  };
#pragma unroll
  for (int i = 0; i < 16; ++i) accA[i] = pairs_sum(accA[i]);
  if constexpr (TWO) {
#pragma unroll
    for (int i = 0; i < 16; ++i) accR[i] = pairs_sum(accR[i]);
  }
  l = pairs_sum(l);
  if (active && pj == 0) {
    float4* ra = reinterpret_cast<float4*>(&sm_acc[w][e * 16]);
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = make_float4(accA[4 * i], accA[4 * i + 1], accA[4 * i + 2], accA[4 * i + 3]);
    if constexpr (TWO) {
      float4* rr = reinterpret_cast<float4*>(&sm_acc[w][D + e * 16]);
#pragma unroll
      for (int i = 0; i < 4; ++i) rr[i] = make_float4(accR[4 * i], accR[4 * i + 1], accR[4 * i + 2], accR[4 * i + 3]);
    }
    if (e == 0) sm_acc[w][kRow - 1] = l;
  }
  if (lane == 0) sm_m[w] = Mw;
  __syncthreads();

  // ---- merge the waves and token pairs: this workgroup's state for its range
  float M = sm_m[0];
#pragma unroll
  for (int ww = 1; ww < NWK; ++ww) M = fmaxf(M, sm_m[ww]);
  float fw[NWK];
#pragma unroll
  for (int ww = 0; ww < NWK; ++ww) fw[ww] = __builtin_amdgcn_exp2f(sm_m[ww] - M);
  auto merged = [&](int i) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWK; ++ww) s = fmaf(sm_acc[ww][i], fw[ww], s);
    return s;
  };
  if (ns > 1) {
    // partial state (m, l, accA[D], accR[D]) of this split; the workgroup
    // that finishes the row last merges all of them
    float* mine = a.partials + ((uint64_t)bh * a.splits + split) * (2 + 2 * D);
    for (int i = tid; i <= 2 * D; i += NWK * 64) {
      if (i == 2 * D) {
        store_dev(mine, M);
        store_dev(mine + 1, merged(kRow - 1));
      } else {
        store_dev(mine + 2 + i, (TWO || i < D) ? merged(i) : 0.f);
      }
    }
    if (!arrive_last(a, bh, ns, tid, &s_ticket) || w != 0) return;
    merge_splits<D, TWO>(a, bh, ns, lane);
    return;
  }
  // ---- a single split: finish here (first wave, two elements per lane)
  if (w != 0) return;
  const bool v1ok = (D > 64) && (lane + 64 < D);
  const float L = merged(kRow - 1);
  const float A0 = merged(lane), A1 = v1ok ? merged(lane + 64) : 0.f;
  float R0 = 0.f, R1 = 0.f;
  if constexpr (TWO) {
    R0 = merged(D + lane);
    R1 = v1ok ? merged(D + lane + 64) : 0.f;
  }
  if (rotated) {
    wave_wht<D>(R0, R1, lane);
    const int8_t* sg = a.signs + ((uint64_t)g.layers + a.layer) * D;  // V signs
    R0 *= ((D == 128) ? 0.08838834764831845f : 0.125f) * (float)sg[lane];
    if (v1ok) R1 *= ((D == 128) ? 0.08838834764831845f : 0.17677669529663687f) * (float)sg[lane + 64];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  a.out[(uint64_t)bh * D + lane] = (A0 + R0) * inv;
  if (v1ok) a.out[(uint64_t)bh * D + lane + 64] = (A1 + R1) * inv;
}

template <int D, int B1, int B2, int NR = 1>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  const int bh = a.rows * a.q_heads;
  const dim3 grid(a.rows_lo * a.splits_lo + (bh - a.rows_lo) * a.splits);
  if constexpr (D == 128 && NR == 1) {
    if (a.waves == 8) {
      if (a.paging.table)
        hipLaunchKernelGGL((decode_kernel<D, B1, B2, NR, true, 8>), grid, dim3(8 * 64), 0, s, a);
      else
        hipLaunchKernelGGL((decode_kernel<D, B1, B2, NR, false, 8>), grid, dim3(8 * 64), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.paging.table)
    hipLaunchKernelGGL((decode_kernel<D, B1, B2, NR, true, 4>), grid, dim3(4 * 64), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, B1, B2, NR, false, 4>), grid, dim3(4 * 64), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const Geometry& g = a.g;
  const bool anchor = g.is_anchor(a.loop);
  if (g.mode == RQ_MODE_DIRECT || anchor) {
    const int bits = g.bits_of(a.loop);
    return bits == 4 ? launch_t<D, 4, 0>(a, s) : launch_t<D, 2, 0>(a, s);
  }
  const int ab = g.anchor_bits, rb = g.residual_bits;
  if (g.mode == RQ_MODE_CHAINED) {
    // loop j reads the residual planes of loops j .. anchor - 1 (4/2 bits only)
    const int nr = g.P - 1 - a.loop % g.P;
    if (nr == 3) return launch_t<D, 4, 2, 3>(a, s);
    if (nr == 2) return launch_t<D, 4, 2, 2>(a, s);
  }
  if (ab == 4 && rb == 2) return launch_t<D, 4, 2>(a, s);
  if (ab == 4 && rb == 4) return launch_t<D, 4, 4>(a, s);
  if (ab == 2 && rb == 2) return launch_t<D, 2, 2>(a, s);
  return launch_t<D, 2, 4>(a, s);
}

}  // namespace

int decode_wave_tokens(int d) {
  switch (d) {
    case 64: return Lay<64>::TPW;
    case 96: return Lay<96>::TPW;
    default: return Lay<128>::TPW;
  }
}

// Waves per workgroup: eight (one workgroup per CU, half the splits to
// merge) for d = 128 calls reading at most one residual plane, except anchor
// calls on a paged cache, where that measured faster; four otherwise (eight
// were slower at d = 96, for chained loops and for paged anchors).
int decode_waves(int d, bool several_planes, bool paged, bool residual) {
  return (d == 128 && !several_planes && (!paged || residual)) ? 8 : 4;
}

int decode_tile_tokens(int d, int waves) {
  switch (d) {
    case 64: return waves * Lay<64>::TPW;
    case 96: return waves * Lay<96>::TPW;
    default: return waves * Lay<128>::TPW;
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (gqa_supported(a.g, a.loop, a.group_ratio)) return launch_gqa(a, s);
  switch (a.g.d) {
    case 64: return launch_d<64>(a, s);
    case 96: return launch_d<96>(a, s);
    default: return launch_d<128>(a, s);
  }
}

}  // namespace rq
