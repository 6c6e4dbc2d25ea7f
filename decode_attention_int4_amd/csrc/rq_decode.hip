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
//   grid (splits, batch * q_heads), 4 waves per workgroup.  LPT lanes share one
//   token; each owns GPL consecutive groups of 16, i.e. a contiguous byte range
//   of every plane, so a wave reads 64 lanes x 16 bytes of anchor codes per
//   instruction, contiguous across lanes.
//   Code unpacking never goes through per-element shifts: one v_and_or_b32
//   drops two codes into the mantissas of an fp16 pair whose exponent encodes
//   1024 (the "magic number" conversion), giving 1024 + m*c.  The query side
//   consumes the pair with v_dot2_f32_f16 against (q_a, q_b)/m, the constant
//   1024*sum(q)/m being subtracted once per group; the query is held in fp16
//   after an exact power-of-two prescale (BF16 fits fp16's mantissa).  H q is
//   not exact in fp16, so against the residual codes, and on the value side,
//   the pair is first turned into the exact codes with one v_pk_fma_f16 and
//   accumulated in fp32 with v_fma_mix_f32.  FP8 scale/offset bytes are
//   decoded by v_cvt_pk_f32_fp8 (OCP e4m3fn on gfx950).
//   Each lane slot keeps its own online-softmax state; the running maximum is
//   only raised when a logit exceeds it by 8 (log2 units), so the rescale of
//   the accumulators is rare.  Slots are merged with DPP row rotations and
//   LDS.  With one split the workgroup's first wave applies H^T and writes the
//   fp32 output; otherwise each workgroup stores its partial state and a small
//   combine kernel merges the splits (the kernel boundary orders the two, so
//   no device-scope fences, which would write back L2, are needed).
#include <hip/hip_runtime.h>

#include "rq_device.h"
#include "rq_kernels.h"

#include <type_traits>

namespace rq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr int NW = 4;              // waves per workgroup
constexpr float kEmpty = -1e30f;   // running max of an empty stream (finite on purpose)
constexpr float kLazy = 8.f;       // log2-domain headroom before the running max moves
constexpr uint32_t kMagic = 0x64006400u;  // fp16 pair (1024, 1024)

template <int D>
struct Shape {
  static constexpr int NG = D / 16;
  static constexpr int LPT = (D == 96) ? 2 : NG / 2;  // lanes per token
  static constexpr int GPL = NG / LPT;                 // groups per lane
  static constexpr int E = GPL * 16;                   // elements per lane
  static constexpr int TPW = 64 / LPT;                 // tokens per wave step
};

// ------------------------------------------------------------ code pairs
// A dword of BITS-bit codes holds 32/BITS codes (element j at bit j*BITS).
// Pair k takes two of them into the two fp16 halves: after an optional right
// shift, masking leaves code_lo at bit position p of the low half and code_hi
// at the same position of the high half; OR-ing 1024's exponent makes the
// halves 1024 + 2^p * code.
template <int BITS>
struct Pairs {
  static constexpr int PER_DWORD = 16 / BITS;  // 4 pairs (int4) or 8 pairs (int2)
  __host__ __device__ static constexpr int lo(int k) { return k; }
  __host__ __device__ static constexpr int hi(int k) { return k + 32 / BITS / 2; }
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

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
  return r;
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 h) { return __builtin_bit_cast(uint32_t, h); }

template <int BITS, int K>
__device__ __forceinline__ uint32_t pair_bits(uint32_t w, uint32_t magic) {
  using PR = Pairs<BITS>;
  return and_or(PR::shift(K) ? (w >> PR::shift(K)) : w, PR::mask(K), magic);
}

// ------------------------------------------------------------ DPP helpers
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// Sum over the LPT lanes of one token (consecutive lanes inside a quad).
template <int LPT>
__device__ __forceinline__ float token_sum(float v) {
  v += dpp<kQuadSwap1>(v);
  if constexpr (LPT == 4) v += dpp<kQuadSwap2>(v);
  return v;
}

// ------------------------------------------------------------ loads
template <int BYTES, int ALIGN>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t* w) {
  if constexpr (BYTES % 16 == 0 && ALIGN % 16 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (BYTES % 8 == 0 && ALIGN % 8 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 8; ++i) {
      const uint2 v = reinterpret_cast<const uint2*>(p)[i];
      w[2 * i] = v.x; w[2 * i + 1] = v.y;
    }
  } else if constexpr (BYTES % 4 == 0 && ALIGN % 4 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 4; ++i) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  } else {
    static_assert(BYTES % 2 == 0 && ALIGN % 2 == 0, "unsupported load shape");
#pragma unroll
    for (int i = 0; i < (BYTES + 3) / 4; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < BYTES / 2; ++i)
      w[i / 2] |= (uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << (16 * (i % 2));
  }
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

template <int D, int BITS>
struct PlaneView {
  using S = Shape<D>;
  static constexpr int CB = S::E * BITS / 8;          // code bytes per lane
  static constexpr int CW = CB / 4;                   // code dwords per lane
  static constexpr int DPG = 16 * BITS / 32;          // code dwords per group
  static constexpr int SB = 2 * S::GPL;               // sz bytes per lane
  static constexpr int SW = (SB + 3) / 4;
  static constexpr int ROW = D * BITS / 8;            // code bytes per token
  static constexpr int CALIGN = gcd_c(gcd_c(ROW, CB), 256);
  static constexpr int SALIGN = gcd_c(gcd_c(2 * S::NG, SB), 256);
};

template <int D, int BITS>
struct PlaneData {
  uint32_t c[PlaneView<D, BITS>::CW];
  uint32_t s[PlaneView<D, BITS>::SW];
};

template <int D, int BITS>
__device__ __forceinline__ void load_plane(PlaneData<D, BITS>& pd, const uint8_t* codes,
                                           const uint8_t* sz, int t, int part) {
  using V = PlaneView<D, BITS>;
  load_bytes<V::CB, V::CALIGN>(codes + (uint64_t)t * V::ROW + part * V::CB, pd.c);
  load_bytes<V::SB, V::SALIGN>(sz + (uint64_t)t * (2 * Shape<D>::NG) + part * V::SB, pd.s);
}

// (scale, offset) of the lane's group g, decoded by the hardware.
template <int D, int BITS>
__device__ __forceinline__ f2 group_sz(const PlaneData<D, BITS>& pd, int g) {
  return (g & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(pd.s[g / 2], true)
                 : __builtin_amdgcn_cvt_pk_f32_fp8(pd.s[g / 2], false);
}

// ------------------------------------------------------------ per-lane query
// fp16 pairs matching the code pairs of one plane, plus the per-group constant
// 1024 * sum(pair) that the magic exponent adds.
template <int D, int BITS>
struct QueryPairs {
  static constexpr int NP = PlaneView<D, BITS>::CW * Pairs<BITS>::PER_DWORD;
  h2 p[NP];
  float off[Shape<D>::GPL];
};

template <int D, int BITS>
__device__ __forceinline__ void build_pairs(QueryPairs<D, BITS>& qp, const float* v, float prescale) {
  using PR = Pairs<BITS>;
  using V = PlaneView<D, BITS>;
#pragma unroll
  for (int g = 0; g < Shape<D>::GPL; ++g) qp.off[g] = 0.f;
#pragma unroll
  for (int dw = 0; dw < V::CW; ++dw) {
#pragma unroll
    for (int k = 0; k < PR::PER_DWORD; ++k) {
      const int base = dw * (32 / BITS);
      const float m = PR::mult(k);
      const _Float16 a = (_Float16)(v[base + PR::lo(k)] * prescale / m);
      const _Float16 b = (_Float16)(v[base + PR::hi(k)] * prescale / m);
      qp.p[dw * PR::PER_DWORD + k] = (h2){a, b};
      qp.off[dw / V::DPG] += 1024.f * ((float)a + (float)b);
    }
  }
}

// sum over the lane's groups of  s_g * (sum_i w_i c_i) * inv_prescale + z_g * wsum_g
template <int D, int BITS>
__device__ __forceinline__ float plane_logit(const PlaneData<D, BITS>& pd, const QueryPairs<D, BITS>& qp,
                                             const float* wsum, float inv_prescale, uint32_t magic) {
  using PR = Pairs<BITS>;
  using V = PlaneView<D, BITS>;
  float sdot = 0.f, zsum = 0.f;
#pragma unroll
  for (int g = 0; g < Shape<D>::GPL; ++g) {
    float acc = -qp.off[g];
#pragma unroll
    for (int dd = 0; dd < V::DPG; ++dd) {
      const int dw = g * V::DPG + dd;
      const uint32_t w = pd.c[dw];
#pragma unroll
      for (int k = 0; k < PR::PER_DWORD; ++k) {
        uint32_t bits;
        switch (k) {  // keeps K a compile-time constant
          case 0: bits = pair_bits<BITS, 0>(w, magic); break;
          case 1: bits = pair_bits<BITS, 1>(w, magic); break;
          case 2: bits = pair_bits<BITS, 2>(w, magic); break;
          case 3: bits = pair_bits<BITS, 3>(w, magic); break;
          case 4: bits = pair_bits<BITS, 4>(w, magic); break;
          case 5: bits = pair_bits<BITS, 5>(w, magic); break;
          case 6: bits = pair_bits<BITS, 6>(w, magic); break;
          default: bits = pair_bits<BITS, 7>(w, magic); break;
        }
        acc = __builtin_amdgcn_fdot2(as_h2(bits), qp.p[dw * PR::PER_DWORD + k], acc, false);
      }
    }
    const f2 sz = group_sz<D, BITS>(pd, g);
    sdot = fmaf(sz.x, acc, sdot);
    zsum = fmaf(sz.y, wsum[g], zsum);
  }
  return fmaf(sdot, inv_prescale, zsum);
}

// Same quantity with fp32 weights: the codes become exact fp16 values (one
// v_pk_fma_f16 per pair) and meet the weights in v_fma_mix_f32, so the weights
// need no fp16 rounding (used for H q, which is not exact in fp16).
template <int D, int BITS>
__device__ __forceinline__ float plane_logit_mix(const PlaneData<D, BITS>& pd, const float* wv,
                                                 const float* wsum, uint32_t magic) {
  using PR = Pairs<BITS>;
  using V = PlaneView<D, BITS>;
  float sdot = 0.f, zsum = 0.f;
#pragma unroll
  for (int g = 0; g < Shape<D>::GPL; ++g) {
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int dd = 0; dd < V::DPG; ++dd) {
      const int dw = g * V::DPG + dd;
      const uint32_t w = pd.c[dw];
#pragma unroll
      for (int k = 0; k < PR::PER_DWORD; ++k) {
        uint32_t bits;
        switch (k) {
          case 0: bits = pair_bits<BITS, 0>(w, magic); break;
          case 1: bits = pair_bits<BITS, 1>(w, magic); break;
          case 2: bits = pair_bits<BITS, 2>(w, magic); break;
          case 3: bits = pair_bits<BITS, 3>(w, magic); break;
          case 4: bits = pair_bits<BITS, 4>(w, magic); break;
          case 5: bits = pair_bits<BITS, 5>(w, magic); break;
          case 6: bits = pair_bits<BITS, 6>(w, magic); break;
          default: bits = pair_bits<BITS, 7>(w, magic); break;
        }
        const float m = PR::mult(k);
        const _Float16 im = (_Float16)(1.f / m), ib = (_Float16)(-1024.f / m);
        const h2 c = __builtin_elementwise_fma(as_h2(bits), (h2){im, im}, (h2){ib, ib});  // exact codes
        const int e = dw * (32 / BITS);
        acc0 = fmaf((float)c.x, wv[e + PR::lo(k)], acc0);
        acc1 = fmaf((float)c.y, wv[e + PR::hi(k)], acc1);
      }
    }
    const f2 sz = group_sz<D, BITS>(pd, g);
    sdot = fmaf(sz.x, acc0 + acc1, sdot);
    zsum = fmaf(sz.y, wsum[g], zsum);
  }
  return sdot + zsum;
}

// acc_i += w * s_g * c_i for the lane's elements; zacc_g += w * z_g
template <int D, int BITS>
__device__ __forceinline__ void plane_accumulate(const PlaneData<D, BITS>& pd, float w, float* acc,
                                                 float* zacc, uint32_t magic) {
  using PR = Pairs<BITS>;
  using V = PlaneView<D, BITS>;
#pragma unroll
  for (int g = 0; g < Shape<D>::GPL; ++g) {
    const f2 sz = group_sz<D, BITS>(pd, g);
    const float ws = w * sz.x;
    zacc[g] = fmaf(w, sz.y, zacc[g]);
#pragma unroll
    for (int dd = 0; dd < V::DPG; ++dd) {
      const int dw = g * V::DPG + dd;
      const uint32_t wd = pd.c[dw];
#pragma unroll
      for (int k = 0; k < PR::PER_DWORD; ++k) {
        uint32_t bits;
        switch (k) {
          case 0: bits = pair_bits<BITS, 0>(wd, magic); break;
          case 1: bits = pair_bits<BITS, 1>(wd, magic); break;
          case 2: bits = pair_bits<BITS, 2>(wd, magic); break;
          case 3: bits = pair_bits<BITS, 3>(wd, magic); break;
          case 4: bits = pair_bits<BITS, 4>(wd, magic); break;
          case 5: bits = pair_bits<BITS, 5>(wd, magic); break;
          case 6: bits = pair_bits<BITS, 6>(wd, magic); break;
          default: bits = pair_bits<BITS, 7>(wd, magic); break;
        }
        const float m = PR::mult(k);
        const _Float16 im = (_Float16)(1.f / m), ib = (_Float16)(-1024.f / m);
        const h2 c = __builtin_elementwise_fma(as_h2(bits), (h2){im, im}, (h2){ib, ib});  // exact codes
        const int e = dw * (32 / BITS);
        acc[e + PR::lo(k)] = fmaf((float)c.x, ws, acc[e + PR::lo(k)]);
        acc[e + PR::hi(k)] = fmaf((float)c.y, ws, acc[e + PR::hi(k)]);
      }
    }
  }
}

// ------------------------------------------------------------ LDS staging
// Each wave streams its tiles (TPW consecutive tokens) through a private ring
// of STAGES buffers in LDS, filled by global_load_lds DMA: the bytes in
// flight occupy LDS instead of VGPRs, so STAGES-1 tiles stay in flight while
// one is consumed.  A tile buffer mirrors the contiguous global bytes of each
// plane piece, so lane l later reads back exactly the bytes a direct load of
// its own (token, part) would have returned: piece_base + l * bytes_per_lane.
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__host__ __device__ constexpr int al16(int x) { return (x + 15) / 16 * 16; }

template <int D, int B1, int B2>
struct Stage {
  using S = Shape<D>;
  static constexpr int TPW = S::TPW;
  static constexpr int R1 = D * B1 / 8;                 // code bytes per token, first plane
  static constexpr int R2 = D * (B2 ? B2 : 2) / 8;      // second plane
  static constexpr int RS = 2 * S::NG;                  // sz bytes per token
  // alpha pieces: a 2-byte DMA still advances 4 bytes per lane in LDS
  static constexpr int C1 = TPW * R1, C2 = TPW * R2, SZ = TPW * RS, AL = TPW * 4;
  static constexpr int k1c = 0;
  static constexpr int k1s = al16(k1c + C1);
  static constexpr int v1c = al16(k1s + SZ);
  static constexpr int v1s = al16(v1c + C1);
  static constexpr int k2c = al16(v1s + SZ);
  static constexpr int k2s = al16(k2c + (B2 ? C2 : 0));
  static constexpr int v2c = al16(k2s + (B2 ? SZ : 0));
  static constexpr int v2s = al16(v2c + (B2 ? C2 : 0));
  static constexpr int ka = al16(v2s + (B2 ? SZ : 0));
  static constexpr int va = al16(ka + (B2 ? AL : 0));
  static constexpr int BYTES = al16(va + (B2 ? AL : 0));
  // DMA instructions for a piece: 1 KB granules (16 bytes per lane) while the
  // row size keeps them 16-byte aligned, then 256-byte dword granules.
  static constexpr int dma_of(int bytes, int row) {
    return (row % 16 == 0 ? bytes / 1024 + (bytes % 1024 + 255) / 256 : (bytes + 255) / 256);
  }
  static constexpr int N_DMA = 2 * (dma_of(C1, R1) + dma_of(SZ, RS)) +
                               (B2 ? 2 * (dma_of(C2, R2) + dma_of(SZ, RS) + 1) : 0);
  static constexpr int COUNT = 3;  // ring depth
  static_assert((COUNT - 1) * N_DMA < 64, "pending DMA count must fit vmcnt");
};

// Copies `BYTES` (a multiple of 4) starting at `src` into LDS at `dst` by DMA:
// 1 KB per instruction (16 bytes per lane) while ROW (the bytes per token)
// keeps lanes 16-byte aligned, then 256 bytes per instruction.  Lane reads at
// or beyond `valid` (the bytes of the tile's in-range tokens) are redirected
// to the last valid granule, so nothing past the range is read and every value
// stays finite.
template <int BYTES, int ROW, bool CLAMP>
__device__ __forceinline__ void dma_piece(const uint8_t* src, int valid, lds_u8* dst, int lane) {
  constexpr int KB = (ROW % 16 == 0) ? BYTES / 1024 : 0;
  constexpr int REST = BYTES - KB * 1024;
  constexpr int FULL = REST / 256, REM = REST % 256;
#pragma unroll
  for (int c = 0; c < KB; ++c) {
    const int o = c * 1024 + lane * 16;
    __builtin_amdgcn_global_load_lds(src + (CLAMP ? min(o, valid - 16) : o), dst + c * 1024, 16, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < FULL; ++c) {
    const int o = KB * 1024 + c * 256;
    const int ol = o + lane * 4;
    __builtin_amdgcn_global_load_lds(src + (CLAMP ? min(ol, valid - 4) : ol), dst + o, 4, 0, 0);
  }
  if constexpr (REM != 0) {
    const int o = KB * 1024 + FULL * 256;
    const int ol = o + lane * 4;
    if (lane < REM / 4)
      __builtin_amdgcn_global_load_lds(src + (CLAMP ? min(ol, valid - 4) : ol), dst + o, 4, 0, 0);
  }
}

// Same for a BF16 alpha piece (2 bytes per token), one ushort DMA; as for
// every sub-dword DMA, lane l lands at dst + 4*l.
template <int TOKENS, bool CLAMP>
__device__ __forceinline__ void dma_alpha(const uint8_t* src, int valid, lds_u8* dst, int lane) {
  if (lane < TOKENS)
    __builtin_amdgcn_global_load_lds(src + (CLAMP ? min(lane * 2, valid - 2) : lane * 2), dst, 2, 0, 0);
}

// s_waitcnt that waits until at most n vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int BYTES, int ALIGN>
__device__ __forceinline__ void lds_bytes(const lds_u8* p, uint32_t* w) {
  typedef __attribute__((address_space(3))) const u32x4 l4;
  typedef __attribute__((address_space(3))) const u32x2 l2;
  typedef __attribute__((address_space(3))) const uint32_t l1;
  typedef __attribute__((address_space(3))) const uint16_t lh;
  if constexpr (BYTES % 16 == 0 && ALIGN % 16 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i) {
      const u32x4 v = reinterpret_cast<l4*>(p)[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (BYTES % 8 == 0 && ALIGN % 8 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 8; ++i) {
      const u32x2 v = reinterpret_cast<l2*>(p)[i];
      w[2 * i] = v.x; w[2 * i + 1] = v.y;
    }
  } else if constexpr (BYTES % 4 == 0 && ALIGN % 4 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 4; ++i) w[i] = reinterpret_cast<l1*>(p)[i];
  } else {
#pragma unroll
    for (int i = 0; i < (BYTES + 3) / 4; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < BYTES / 2; ++i) w[i / 2] |= (uint32_t)reinterpret_cast<lh*>(p)[i] << (16 * (i % 2));
  }
}

template <int D, int BITS>
__device__ __forceinline__ void lds_plane(PlaneData<D, BITS>& pd, const lds_u8* codes, const lds_u8* sz,
                                          int lane) {
  using V = PlaneView<D, BITS>;
  lds_bytes<V::CB, gcd_c(V::CB, 16)>(codes + lane * V::CB, pd.c);
  lds_bytes<V::SB, gcd_c(V::SB, 16)>(sz + lane * V::SB, pd.s);
}

template <int D, int B1, int B2>
struct TokenData {
  PlaneData<D, B1> k1, v1;
  PlaneData<D, (B2 ? B2 : 2)> k2, v2;
  uint32_t ka, va;  // BF16 alphas
};

// Walsh-Hadamard transform of a vector held two elements per lane (l, l+64)
// by one wave; block diagonal 64+32 when D == 96.  Unscaled.
template <int D>
__device__ __forceinline__ void wave_wht(float& y0, float& y1, int lane) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const float p0 = __shfl_xor(y0, h);
    y0 = (lane & h) ? (p0 - y0) : (y0 + p0);
    if constexpr (D == 128) {
      const float p1 = __shfl_xor(y1, h);
      y1 = (lane & h) ? (p1 - y1) : (y1 + p1);
    } else if constexpr (D == 96) {
      if (h < 32) {
        const float p1 = __shfl_xor(y1, h);
        y1 = (lane & h) ? (p1 - y1) : (y1 + p1);
      }
    }
  }
  if constexpr (D == 128) {
    const float a = y0, b = y1;
    y0 = a + b;
    y1 = a - b;
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// 2^k with max|v| * 2^k in [2^13, 2^14): fp16 then holds BF16 inputs exactly.
__device__ __forceinline__ float fp16_prescale(float maxabs) {
  if (!(maxabs > 0.f)) return 1.f;
  int e;
  frexpf(maxabs, &e);
  return ldexpf(1.f, 14 - e);
}

template <int D, int B1, int B2>
__global__ void __launch_bounds__(NW * 64, 2) decode_kernel(DecodeArgs a) {
  using S = Shape<D>;
  constexpr int E = S::E, LPT = S::LPT, TPW = S::TPW, GPL = S::GPL;
  constexpr bool TWO = B2 != 0;
  constexpr int B2E = TWO ? B2 : 2;
  const Geometry& g = a.g;

  using ST = Stage<D, B1, B2>;
  constexpr int kStaging = NW * ST::COUNT * ST::BYTES;
  constexpr int kEpilogue = NW * 4 * (2 * D + 1) * 4;
  // the epilogue buffers reuse the staging area once every wave has finished
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStaging > kEpilogue ? kStaging : kEpilogue];
  __shared__ float sq[D], su[D];
  __shared__ float s_scale[4];
  __shared__ float sm_m[NW];
  typedef float AccRow[4][2 * D + 1];
  AccRow* sm_acc = reinterpret_cast<AccRow*>(smem);               // [wave][row][acc | l]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.q_heads, hq = bh % a.q_heads, kvh = hq / a.group_ratio;
  const int slot = lane / LPT, part = lane % LPT;
  const bool rotated = TWO && g.rotation == RQ_ROT_HADAMARD;
  uint32_t magic;
  asm("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kMagic));

  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(a.n_tokens, t_begin + a.tokens_per_split);
  // ---- plane bases
  const int loop1 = (g.mode == RQ_MODE_DIRECT || !TWO) ? a.loop : (a.loop - a.loop % g.P + g.P - 1);
  const uint8_t* k1 = a.cache + g.slot_offset(0, b, a.layer, loop1, kvh);
  const uint8_t* v1 = a.cache + g.slot_offset(1, b, a.layer, loop1, kvh);
  const uint8_t* k1s = k1 + g.sz_rel(loop1);
  const uint8_t* v1s = v1 + g.sz_rel(loop1);
  const uint8_t* k2 = a.cache + g.slot_offset(0, b, a.layer, a.loop, kvh);
  const uint8_t* v2 = a.cache + g.slot_offset(1, b, a.layer, a.loop, kvh);
  const uint8_t* k2s = k2 + g.sz_rel(a.loop);
  const uint8_t* v2s = v2 + g.sz_rel(a.loop);
  const uint16_t* k2a = reinterpret_cast<const uint16_t*>(k2 + g.alpha_rel(a.loop));
  const uint16_t* v2a = reinterpret_cast<const uint16_t*>(v2 + g.alpha_rel(a.loop));


  // ---- stream this wave's tiles through its LDS ring
  lds_u8* ring = (lds_u8*)smem + w * ST::COUNT * ST::BYTES;
  const int first = t_begin + w * TPW;
  const int n_tiles = first < t_end ? (t_end - first + NW * TPW - 1) / (NW * TPW) : 0;
  auto issue_t = [&](auto clamp, int tb, lds_u8* st, int vt) {
    constexpr bool C = decltype(clamp)::value;
    dma_piece<ST::C1, ST::R1, C>(k1 + (uint64_t)tb * ST::R1, vt * ST::R1, st + ST::k1c, lane);
    dma_piece<ST::SZ, ST::RS, C>(k1s + (uint64_t)tb * ST::RS, vt * ST::RS, st + ST::k1s, lane);
    dma_piece<ST::C1, ST::R1, C>(v1 + (uint64_t)tb * ST::R1, vt * ST::R1, st + ST::v1c, lane);
    dma_piece<ST::SZ, ST::RS, C>(v1s + (uint64_t)tb * ST::RS, vt * ST::RS, st + ST::v1s, lane);
    if constexpr (TWO) {
      dma_piece<ST::C2, ST::R2, C>(k2 + (uint64_t)tb * ST::R2, vt * ST::R2, st + ST::k2c, lane);
      dma_piece<ST::SZ, ST::RS, C>(k2s + (uint64_t)tb * ST::RS, vt * ST::RS, st + ST::k2s, lane);
      dma_piece<ST::C2, ST::R2, C>(v2 + (uint64_t)tb * ST::R2, vt * ST::R2, st + ST::v2c, lane);
      dma_piece<ST::SZ, ST::RS, C>(v2s + (uint64_t)tb * ST::RS, vt * ST::RS, st + ST::v2s, lane);
      dma_alpha<TPW, C>(reinterpret_cast<const uint8_t*>(k2a + tb), vt * 2, st + ST::ka, lane);
      dma_alpha<TPW, C>(reinterpret_cast<const uint8_t*>(v2a + tb), vt * 2, st + ST::va, lane);
    }
  };
  auto issue = [&](int tile) {
    const int tb = first + tile * NW * TPW;
    lds_u8* st = ring + (tile % ST::COUNT) * ST::BYTES;
    const int vt = t_end - tb;  // in-range tokens of this tile (>= 1)
    if (vt >= TPW)
      issue_t(std::integral_constant<bool, false>{}, tb, st, vt);
    else
      issue_t(std::integral_constant<bool, true>{}, tb, st, vt);
  };
#pragma unroll
  for (int i = 0; i < ST::COUNT - 1; ++i)
    if (i < n_tiles) issue(i);


  // ---- query, u = H q and their fp16 prescales (wave 0)
  if (w == 0) {
    const bool v1ok = (D > 64) && (lane + 64 < D);
    const float q0 = bf16_to_f32(a.q[(uint64_t)bh * D + lane]);
    const float q1 = v1ok ? bf16_to_f32(a.q[(uint64_t)bh * D + lane + 64]) : 0.f;
    sq[lane] = q0;
    if (v1ok) sq[lane + 64] = q1;
    float u0 = q0, u1 = q1;
    if (rotated) {
      const int8_t* sg = a.signs + (uint64_t)a.layer * D;  // K signs of this layer
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
    const float mq = wave_max(fmaxf(fabsf(q0), fabsf(q1)));
    if (lane == 0) s_scale[0] = fp16_prescale(mq);
  }
  __syncthreads();

  const float pq = s_scale[0];
  QueryPairs<D, B1> qp;
  float ur[TWO ? E : 1];
  float qsum[GPL], usum[GPL];
  {
    float v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = sq[part * E + i];
#pragma unroll
    for (int gi = 0; gi < GPL; ++gi) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += v[gi * 16 + i];
      qsum[gi] = s;
    }
    build_pairs<D, B1>(qp, v, pq);
    if constexpr (TWO) {
#pragma unroll
      for (int i = 0; i < E; ++i) ur[i] = su[part * E + i];
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s += ur[gi * 16 + i];
        usum[gi] = s;
      }
    }
  }
  const float ipq = 1.f / pq;

  float accA[E], accR[TWO ? E : 1], zA[GPL], zR[GPL];
#pragma unroll
  for (int i = 0; i < E; ++i) accA[i] = 0.f;
#pragma unroll
  for (int i = 0; i < (TWO ? E : 1); ++i) accR[i] = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPL; ++gi) zA[gi] = zR[gi] = 0.f;
  float m = kEmpty, l = 0.f;
  const float qs = a.qscale;


  for (int it = 0; it < n_tiles; ++it) {
    if (it + ST::COUNT - 1 < n_tiles) issue(it + ST::COUNT - 1);
    // wait for tile `it`: the tiles issued after it may stay in flight
    const int later = min(ST::COUNT - 1, n_tiles - 1 - it);
    if constexpr (ST::COUNT > 3) {
      if (later >= 3) wait_vm<3 * ST::N_DMA>();
    }
    if (later == 2) wait_vm<2 * ST::N_DMA>();
    else if (later == 1) wait_vm<ST::N_DMA>();
    else if (later == 0) wait_vm<0>();
    const lds_u8* st = ring + (it % ST::COUNT) * ST::BYTES;
    TokenData<D, B1, B2> cur;
    lds_plane<D, B1>(cur.k1, st + ST::k1c, st + ST::k1s, lane);
    lds_plane<D, B1>(cur.v1, st + ST::v1c, st + ST::v1s, lane);
    if constexpr (TWO) {
      lds_plane<D, B2E>(cur.k2, st + ST::k2c, st + ST::k2s, lane);
      lds_plane<D, B2E>(cur.v2, st + ST::v2c, st + ST::v2s, lane);
      typedef __attribute__((address_space(3))) const uint16_t lh;
      cur.ka = reinterpret_cast<lh*>(st + ST::ka)[2 * slot];
      cur.va = reinterpret_cast<lh*>(st + ST::va)[2 * slot];
    }
    const bool cur_ok = first + it * NW * TPW + slot < t_end;

    float part_logit = plane_logit<D, B1>(cur.k1, qp, qsum, ipq, magic);
    if constexpr (TWO)
      part_logit = fmaf(bf16_to_f32(cur.ka), plane_logit_mix<D, B2E>(cur.k2, ur, usum, magic), part_logit);
    const float logit = cur_ok ? token_sum<LPT>(part_logit) * qs : kEmpty;
    if (logit > m + kLazy) {
      const float corr = exp2f(m - logit);
      l *= corr;
#pragma unroll
      for (int i = 0; i < E; ++i) accA[i] *= corr;
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) zA[gi] *= corr;
      if constexpr (TWO) {
#pragma unroll
        for (int i = 0; i < E; ++i) accR[i] *= corr;
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) zR[gi] *= corr;
      }
      m = logit;
    }
    const float p = cur_ok ? exp2f(logit - m) : 0.f;
    l += p;
    plane_accumulate<D, B1>(cur.v1, p, accA, zA, magic);
    if constexpr (TWO) plane_accumulate<D, B2E>(cur.v2, p * bf16_to_f32(cur.va), accR, zR, magic);
  }
  __syncthreads();  // every wave is done with its ring before the epilogue reuses it

  // ---- fold the offset sums, align every slot to the wave maximum
#pragma unroll
  for (int i = 0; i < E; ++i) accA[i] += zA[i / 16];
  if constexpr (TWO) {
#pragma unroll
    for (int i = 0; i < E; ++i) accR[i] += zR[i / 16];
  }
  const float Mw = wave_max(m);
  {
    const float f = exp2f(m - Mw);
    l *= f;
#pragma unroll
    for (int i = 0; i < E; ++i) accA[i] *= f;
    if constexpr (TWO) {
#pragma unroll
      for (int i = 0; i < E; ++i) accR[i] *= f;
    }
  }
  // ---- sum the slots of each 16-lane row (lanes equal mod LPT) with row rotations
#pragma unroll
  for (int i = 0; i < E; ++i) {
    accA[i] += dpp<kRowRor8>(accA[i]);
    if constexpr (LPT == 2) accA[i] += dpp<kRowRor4>(accA[i]);
    accA[i] += dpp<(LPT == 4 ? kRowRor4 : 0x122)>(accA[i]);
  }
  if constexpr (TWO) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      accR[i] += dpp<kRowRor8>(accR[i]);
      if constexpr (LPT == 2) accR[i] += dpp<kRowRor4>(accR[i]);
      accR[i] += dpp<(LPT == 4 ? kRowRor4 : 0x122)>(accR[i]);
    }
  }
  l += dpp<kRowRor8>(l);
  if constexpr (LPT == 2) l += dpp<kRowRor4>(l);
  l += dpp<(LPT == 4 ? kRowRor4 : 0x122)>(l);
  const int row = lane >> 4;
  if ((lane & 15) < LPT) {
#pragma unroll
    for (int i = 0; i < E; ++i) sm_acc[w][row][part * E + i] = accA[i];
    if constexpr (TWO) {
#pragma unroll
      for (int i = 0; i < E; ++i) sm_acc[w][row][D + part * E + i] = accR[i];
    }
    if (part == 0) sm_acc[w][row][2 * D] = l;
  }
  if (lane == 0) sm_m[w] = Mw;
  __syncthreads();

  // ---- merge the waves: this workgroup's state for its token range
  float M = sm_m[0];
#pragma unroll
  for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm_m[ww]);
  float fw[NW];
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) fw[ww] = exp2f(sm_m[ww] - M);
  auto merged = [&](int i) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww)
      s += (sm_acc[ww][0][i] + sm_acc[ww][1][i] + sm_acc[ww][2][i] + sm_acc[ww][3][i]) * fw[ww];
    return s;
  };
  if (a.splits > 1) {
    // partial state (m, l, accA[D], accR[D]) for the combine kernel; the
    // kernel boundary orders these stores before its loads
    float* mine = a.partials + ((uint64_t)bh * a.splits + split) * (2 + 2 * D);
    for (int i = tid; i <= 2 * D; i += NW * 64) {
      const float v = (TWO || i < D || i == 2 * D) ? merged(i) : 0.f;
      if (i == 2 * D) {
        mine[0] = M;
        mine[1] = v;
      } else {
        mine[2 + i] = v;
      }
    }
    return;
  }
  // ---- a single split: finish here (first wave, two elements per lane)
  if (w != 0) return;
  const bool v1ok = (D > 64) && (lane + 64 < D);
  const float L = merged(2 * D);
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

// Merges the split partial states of one (batch row, query head) per
// workgroup (one wave, two elements per lane), applies H^T to the residual
// sum and writes the fp32 output.
template <int D, bool TWO>
__global__ void __launch_bounds__(64) combine_kernel(DecodeArgs a) {
  constexpr int W = 2 + 2 * D;
  const int bh = blockIdx.x, lane = threadIdx.x, ns = a.splits;
  const bool v1ok = (D > 64) && (lane + 64 < D);
  const float* all = a.partials + (uint64_t)bh * ns * W;
  float M = kEmpty;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) M = fmaxf(M, all[(uint64_t)(s0 + lane) * W]);
  M = wave_max(M);
  float L = 0.f, A0 = 0.f, A1 = 0.f, R0 = 0.f, R1 = 0.f;
  // eight splits per round: their loads are independent and issue together
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float ms[8], ls[8], a0[8], a1[8], r0[8], r1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sj = min(s0 + j, ns - 1);
      const float* ps = all + (uint64_t)sj * W;
      ms[j] = (s0 + j < ns) ? ps[0] : kEmpty;
      ls[j] = ps[1];
      a0[j] = ps[2 + lane];
      a1[j] = v1ok ? ps[2 + lane + 64] : 0.f;
      r0[j] = TWO ? ps[2 + D + lane] : 0.f;
      r1[j] = (TWO && v1ok) ? ps[2 + D + lane + 64] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = exp2f(ms[j] - M);
      L = fmaf(f, ls[j], L);
      A0 = fmaf(f, a0[j], A0);
      A1 = fmaf(f, a1[j], A1);
      R0 = fmaf(f, r0[j], R0);
      R1 = fmaf(f, r1[j], R1);
    }
  }
  if (TWO && a.g.rotation == RQ_ROT_HADAMARD) {
    wave_wht<D>(R0, R1, lane);
    const int8_t* sg = a.signs + ((uint64_t)a.g.layers + a.layer) * D;  // V signs
    R0 *= ((D == 128) ? 0.08838834764831845f : 0.125f) * (float)sg[lane];
    if (v1ok) R1 *= ((D == 128) ? 0.08838834764831845f : 0.17677669529663687f) * (float)sg[lane + 64];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  a.out[(uint64_t)bh * D + lane] = (A0 + R0) * inv;
  if (v1ok) a.out[(uint64_t)bh * D + lane + 64] = (A1 + R1) * inv;
}

template <int D, int B1, int B2>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<D, B1, B2>), dim3(a.splits, a.g.batch * a.q_heads), dim3(NW * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((combine_kernel<D, B2 != 0>), dim3(a.g.batch * a.q_heads), dim3(64), 0, s, a);
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
  if (ab == 4 && rb == 2) return launch_t<D, 4, 2>(a, s);
  if (ab == 4 && rb == 4) return launch_t<D, 4, 4>(a, s);
  if (ab == 2 && rb == 2) return launch_t<D, 2, 2>(a, s);
  return launch_t<D, 2, 4>(a, s);
}

}  // namespace

int decode_tile_tokens(int d) {
  switch (d) {
    case 64: return NW * Shape<64>::TPW;
    case 96: return NW * Shape<96>::TPW;
    default: return NW * Shape<128>::TPW;
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  switch (a.g.d) {
    case 64: return launch_d<64>(a, s);
    case 96: return launch_d<96>(a, s);
    default: return launch_d<128>(a, s);
  }
}

}  // namespace rq
