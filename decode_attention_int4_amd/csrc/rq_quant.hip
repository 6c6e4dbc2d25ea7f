// rq_quant.hip -- quantize-and-append of looped-Transformer K/V states.
//
// One item is one token vector of one loop group: (kv, batch row, layer, kv
// head, token, loop group).  Its anchor (last loop of the group) is quantized
// at anchor_bits; every other loop's residual against the dequantized anchor
// is rotated by H = (1/sqrt(n)) WHT diag(signs), quantized at residual_bits
// and given a BF16 least-squares scale (ai4snews summary, paragraphs 1-2;
// agihunt "Confirmed" list).
//
// Work mapping: a quad of lanes encodes one item.  Lane q of the quad holds
// the 16 elements of group q and, at d = 128 (and d = 96 for q < 2), those of
// group q + 4, so group minima and maxima, codes and code packing stay inside
// the lane.  Of the Walsh-Hadamard butterflies (index bits 1..64), bits 1-8
// and 64 are in-lane; bits 16 and 32 are lane bits 0 and 1 of the quad and
// run through DPP quad permutes.  Sixteen items per wavefront.
//
// Every value that decides a stored code, FP8 byte or BF16 alpha is computed
// in IEEE double precision, in the same operations as the definition: the
// rotation's +-1 sums, (x - z) / s rounded half-even, dequantization s*c + z,
// and the alpha sums.  The per-element quotient (x - z) / s is formed as
// q0 = d * RN(1/s), corrected once by the exact FMA residual d - q0 * s
// (Markstein's correction), which gives the correctly rounded quotient, so no
// per-element division is issued.  MI355X runs fp64 FMA at the fp32 rate.
#include <hip/hip_runtime.h>

#include "rq_device.h"
#include "rq_kernels.h"

#pragma clang fp contract(off)

namespace rq {
namespace {

// DPP quad permutes of a double: lane ^ 1 and lane ^ 2 within each quad.
template <int CTRL>
__device__ __forceinline__ double quad_perm(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
constexpr int kXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);  // quad_perm [1,0,3,2]
constexpr int kXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);  // quad_perm [2,3,0,1]

__device__ __forceinline__ double quad_sum(double v) {
  v = v + quad_perm<kXor1>(v);
  return v + quad_perm<kXor2>(v);
}

// One group of 16 in-lane values quantized at BITS bits with the group's own
// FP8 scale s and offset z (min/max asymmetric quantization); the codes come
// back packed, element k at bit k*BITS.  Minimum and maximum are those of an
// index-order scan with strict comparisons, which matters only for the sign of
// a zero extreme.  With ALPHA, the group's terms of the least-squares sums
// <v, vhat> and <vhat, vhat> (vhat = s*c + z) are added to num and den.
template <int BITS, bool ALPHA>
__device__ __forceinline__ void quant16(const double (&v)[16], uint32_t (&w)[BITS / 2], uint32_t& sz,
                                        double& s, double& z, double& num, double& den) {
  constexpr int Q = (1 << BITS) - 1, PER = 32 / BITS;
  double mn = v[0], mx = v[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) {
    mn = __builtin_fmin(mn, v[k]);
    mx = __builtin_fmax(mx, v[k]);
  }
  if (mn == 0.0 || mx == 0.0) {
    // the sign of a zero extreme is that of the first zero in index order
    mn = v[0];
    mx = v[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) {
      mn = v[k] < mn ? v[k] : mn;
      mx = v[k] > mx ? v[k] : mx;
    }
  }
  const uint32_t s8 = f64_to_fp8((mx - mn) / (double)Q);
  const uint32_t z8 = f64_to_fp8(mn);
  s = fp8_to_f64(s8);
  z = fp8_to_f64(z8);
  sz = s8 | (z8 << 8);
#pragma unroll
  for (int i = 0; i < BITS / 2; ++i) w[i] = 0u;
  // s == 0 (a constant group): r = 0 makes every quotient +-0, so code 0
  const double r = s != 0.0 ? 1.0 / s : 0.0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const double d = v[k] - z;
    const double q0 = d * r;
    const double qt = __builtin_fma(__builtin_fma(-q0, s, d), r, q0);  // == d / s
    const double c = __builtin_fmin(__builtin_fmax(__builtin_rint(qt), 0.0), (double)Q);
    w[k / PER] |= (uint32_t)c << ((k % PER) * BITS);
    if constexpr (ALPHA) {
      const double vh = __builtin_fma(s, c, z);
      num = __builtin_fma(v[k], vh, num);
      den = __builtin_fma(vh, vh, den);
    }
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t code_of(const uint32_t (&w)[BITS / 2], int k) {
  constexpr int PER = 32 / BITS;
  return (w[k / PER] >> ((k % PER) * BITS)) & ((1u << BITS) - 1u);
}

// Stores one group's packed codes and its scale | offset << 8.
template <int BITS>
__device__ __forceinline__ void store_group(uint8_t* row, int g, const uint32_t (&w)[BITS / 2],
                                            uint32_t sz, uint8_t* sz_row) {
  if constexpr (BITS == 4) {
    *reinterpret_cast<uint2*>(row + 8 * g) = make_uint2(w[0], w[1]);
  } else {
    *reinterpret_cast<uint32_t*>(row + 4 * g) = w[0];
  }
  reinterpret_cast<uint16_t*>(sz_row)[g] = (uint16_t)sz;
}

// Loads the raw BF16 words of the lane's (up to) two groups of one token row.
template <int NS>
__device__ __forceinline__ void load_raw(const uint16_t* row, int q, bool s1ok, bool v16,
                                         uint32_t (&w)[2][8]) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s == 0 || s1ok) {
      const uint16_t* p = row + 64 * s + 16 * q;
      if (v16) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
        w[s][0] = a.x; w[s][1] = a.y; w[s][2] = a.z; w[s][3] = a.w;
        w[s][4] = b.x; w[s][5] = b.y; w[s][6] = b.z; w[s][7] = b.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[s][i] = reinterpret_cast<const uint32_t*>(p)[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[s][i] = 0u;
    }
  }
}
__device__ __forceinline__ void unpack16(const uint32_t (&w)[8], double (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = (double)__uint_as_float(w[i] << 16);
    x[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// y <- WHT y over the item (unscaled), stages in index-bit order 1, 2, ..., 64.
// d = 96 transforms its 64 + 32 blocks separately: the second block (groups
// 4 and 5, slot 1 of lanes 0 and 1) has index bits 1..16 only.
template <int D>
__device__ __forceinline__ void wht_quad(double (&y)[2][16], int q) {
  constexpr int NS = D == 64 ? 1 : 2;
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k & h) continue;
        const double a = y[s][k], b = y[s][k + h];
        y[s][k] = a + b;
        y[s][k + h] = a - b;
      }
    }
  }
  // bit 16 = lane bit 0: the lower lane keeps y + p, the upper one p - y
  const double g1 = (q & 1) ? -1.0 : 1.0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      y[s][k] = __builtin_fma(g1, y[s][k], quad_perm<kXor1>(y[s][k]));
    }
  }
  const double g2 = (q & 2) ? -1.0 : 1.0;
#pragma unroll
  for (int s = 0; s < (D == 128 ? 2 : 1); ++s) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      y[s][k] = __builtin_fma(g2, y[s][k], quad_perm<kXor2>(y[s][k]));
    }
  }
  if constexpr (D == 128) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const double a = y[0][k], b = y[1][k];
      y[0][k] = a + b;
      y[1][k] = a - b;
    }
  }
}

template <int D, int AB, int RB, int MODE>
__global__ void __launch_bounds__(256) quant_append_kernel(QuantArgs a) {
  constexpr int NS = D == 64 ? 1 : 2;
  constexpr bool CHAINED = MODE == RQ_MODE_CHAINED, DIRECT = MODE == RQ_MODE_DIRECT;
  const Geometry& g = a.g;
  const int q = threadIdx.x & 3;
  const uint64_t quad0 = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 2;
  const uint64_t n_quads = ((uint64_t)gridDim.x * blockDim.x) >> 2;
  const int G = g.loops / g.P;
  const bool s1ok = D == 128 || (D == 96 && q < 2);
  const bool v16 = (reinterpret_cast<uintptr_t>(a.kv) & 15u) == 0;
  const bool rotated = !DIRECT && g.rotation == RQ_ROT_HADAMARD;
  // per-block scales of the Walsh-Hadamard transform
  const double sc0 = (D == 128) ? 1.0 / sqrt(128.0) : 1.0 / sqrt(64.0);
  const double sc1 = (D == 128) ? 1.0 / sqrt(128.0) : 1.0 / sqrt(32.0);

#pragma unroll 1
  for (uint64_t item = quad0; item < a.items; item += n_quads) {
    const int t = (int)(item % (uint64_t)a.t_new);
    uint64_t c = item / (uint64_t)a.t_new;
    const int k = (int)(c % G);
    c /= G;
    const int head = (int)(c % g.kv_heads);
    c /= g.kv_heads;
    const int layer = (int)(c % g.layers);
    c /= g.layers;
    const int b = (int)(c % a.rows);
    const int kv = (int)(c / a.rows);
    int pos = a.n_tokens + t;
    int slot_row = b;  // row of the cache geometry: the batch row, or a pool block
    if (a.paging.table) {
      // paged: the logical position picks the block from the row's table; a
      // row whose range does not fit its table, or a token whose block id is
      // outside the pool, is skipped (uniform over the quad)
      const int cap = a.paging.max_blocks << a.paging.block_shift;
      const int p0 = a.positions[b];
      if (p0 < 0 || p0 > cap - a.t_new) continue;
      const int lp = p0 + t;
      slot_row = a.paging.table[(uint64_t)b * a.paging.max_blocks + (lp >> a.paging.block_shift)];
      if (slot_row < 0 || slot_row >= g.batch) continue;
      pos = lp & ((1 << a.paging.block_shift) - 1);
    } else if (a.positions) {
      // per-row positions come from device memory: a row whose range does not
      // fit the cache is skipped
      const int p0 = a.positions[b];
      if (p0 < 0 || p0 > g.max_tokens - a.t_new) continue;
      pos = p0 + t;
    }

    auto src = [&](int loop) {
      return a.kv + ((((uint64_t)(kv * a.rows + b) * g.loops + loop) * g.layers + layer) *
                         g.kv_heads + head) * (uint64_t)a.t_new * D + (uint64_t)t * D;
    };
    auto slot_base = [&](int loop) { return a.cache + g.slot_offset(kv, slot_row, layer, loop, head); };

    // ---- anchor: codes stay packed in registers for the other loops
    const int aloop = k * g.P + g.P - 1;
    uint32_t raw[2][8];
    load_raw<NS>(src(aloop), q, s1ok, v16, raw);
    uint32_t ca[2][AB / 2];
    double sa[2], za[2];
    {
      uint8_t* base = slot_base(aloop);
      uint8_t* row = base + (uint64_t)pos * (D * AB / 8);
      uint8_t* sz_row = base + g.sz_rel(aloop) + (uint64_t)pos * (2 * D / 16);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        double x[16], n0 = 0.0, d0 = 0.0;
        unpack16(raw[s], x);
        uint32_t sz;
        quant16<AB, false>(x, ca[s], sz, sa[s], za[s], n0, d0);
        if (s == 0 || s1ok) store_group<AB>(row, q + 4 * s, ca[s], sz, sz_row);
      }
    }
    // this layer's rotation signs for the lane's elements
    uint32_t sgw[2][4];
    if (rotated) {
      const int8_t* sg = a.signs + ((uint64_t)kv * g.layers + layer) * D;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int8_t* p = sg + 64 * s + 16 * q + 4 * i;
          sgw[s][i] = (s == 0 || s1ok) ? ((uint32_t)(uint8_t)p[0] | ((uint32_t)(uint8_t)p[1] << 8) |
                                          ((uint32_t)(uint8_t)p[2] << 16) | ((uint32_t)(uint8_t)p[3] << 24))
                                       : 0x01010101u;
        }
    }

    // ---- other loops of the group.  Chained mode walks from the loop next to
    // the anchor outwards: corr = sum alpha_i yhat_i over the loops already
    // stored, so y = H (x_l - deq(A)) - corr is the rotated residual against
    // the reconstruction of loop l + 1
    double corr[CHAINED ? 2 : 1][16];
    if constexpr (CHAINED) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 16; ++e) corr[s][e] = 0.0;
    }
#pragma unroll 1
    for (int jj = 0; jj < g.P - 1; ++jj) {
      const int j = CHAINED ? g.P - 2 - jj : jj;
      const int loop = k * g.P + j;
      // the anchor's values and the signs are unpacked again per loop: hoisted
      // out of the loop they would hold 128 more registers
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int i = 0; i < AB / 2; ++i) asm volatile("" : "+v"(ca[s][i]));
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(sgw[s][i]));
      }
      load_raw<NS>(src(loop), q, s1ok, v16, raw);
      uint8_t* base = slot_base(loop);
      uint8_t* row = base + (uint64_t)pos * (D * RB / 8);
      uint8_t* sz_row = base + g.sz_rel(loop) + (uint64_t)pos * (2 * D / 16);
      if constexpr (DIRECT) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          double x[16], sr, zr, n0 = 0.0, d0 = 0.0;
          unpack16(raw[s], x);
          uint32_t sz, w[RB / 2];
          quant16<RB, false>(x, w, sz, sr, zr, n0, d0);
          if (s == 0 || s1ok) store_group<RB>(row, q + 4 * s, w, sz, sz_row);
        }
      } else {
        // r = x - deq(A); dequantization s*c + z is exact in fp64, so one FMA
        // gives the same value as the product and the sum
        double y[2][16];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          unpack16(raw[s], y[s]);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            y[s][e] = y[s][e] - __builtin_fma(sa[s], (double)code_of<AB>(ca[s], e), za[s]);
        }
        if (rotated) {
          // sign flips: bit 7 of sign byte e moved to the sign bit of y_e
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const uint64_t u = (uint64_t)__double_as_longlong(y[s][e]);
              const uint32_t f = (sgw[s][e / 4] << (24 - 8 * (e % 4))) & 0x80000000u;
              y[s][e] = __longlong_as_double((long long)(u ^ ((uint64_t)f << 32)));
            }
          wht_quad<D>(y, q);
          // + 0 (inside the FMA) turns a -0 into +0 and changes nothing else:
          // an element of H r whose exact sum is zero is +0, whatever signed
          // zeros the butterflies passed through
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            y[0][e] = __builtin_fma(y[0][e], sc0, 0.0);
            if (NS == 2) y[1][e] = __builtin_fma(y[1][e], sc1, 0.0);
          }
        }
        if constexpr (CHAINED) {
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int e = 0; e < 16; ++e) y[s][e] = y[s][e] - corr[s][e];
        }
        double num = 0.0, den = 0.0, yy = 0.0;
        double sr[2], zr[2];
        uint32_t cw[2][RB / 2];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          uint32_t sz;
          double n0 = 0.0, d0 = 0.0;
          quant16<RB, true>(y[s], cw[s], sz, sr[s], zr[s], n0, d0);
          if (s == 1 && !s1ok) continue;
          store_group<RB>(row, q + 4 * s, cw[s], sz, sz_row);
          num += n0;
          den += d0;
        }
        if (g.alpha_mode == RQ_ALPHA_NORM_RATIO) {
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (s == 1 && !s1ok) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) yy = __builtin_fma(y[s][e], y[s][e], yy);
          }
        }
        num = quad_sum(num);
        den = quad_sum(den);
        yy = quad_sum(yy);
        uint32_t al;
        if (g.alpha_mode == RQ_ALPHA_ONE)
          al = 0x3F80u;
        else if (!(den > 0.0))
          al = 0u;
        else if (g.alpha_mode == RQ_ALPHA_NORM_RATIO)
          al = f64_to_bf16(sqrt(yy) / sqrt(den));
        else
          al = f64_to_bf16(num / den);
        if (q == 0)
          reinterpret_cast<uint16_t*>(a.cache + g.alpha_offset(kv, slot_row, layer, loop, head))[pos] =
              (uint16_t)al;
        if constexpr (CHAINED) {
          // alpha (8 significant bits) times yhat is exact, so the FMA is the
          // product-then-sum of the definition
          const double ab = (double)bf16_to_f32(al);
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              corr[s][e] = __builtin_fma(
                  ab, __builtin_fma(sr[s], (double)code_of<RB>(cw[s], e), zr[s]), corr[s][e]);
        }
      }
    }
  }
}

}  // namespace

template <int D, int AB, int RB>
static hipError_t launch_quant_t(const QuantArgs& a, hipStream_t s) {
  // one quad per item, four wavefronts per block
  uint64_t blocks = (a.items + 63) / 64;
  if (blocks > 16384) blocks = 16384;
  const dim3 grid((unsigned)blocks), block(256);
  switch (a.g.mode) {
    case RQ_MODE_DIRECT:
      hipLaunchKernelGGL((quant_append_kernel<D, AB, RB, RQ_MODE_DIRECT>), grid, block, 0, s, a);
      break;
    case RQ_MODE_CHAINED:
      hipLaunchKernelGGL((quant_append_kernel<D, AB, RB, RQ_MODE_CHAINED>), grid, block, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((quant_append_kernel<D, AB, RB, RQ_MODE_RESIDUAL>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_quant_d(const QuantArgs& a, hipStream_t s) {
  const int ab = a.g.anchor_bits, rb = a.g.residual_bits;
  if (ab == 4 && rb == 2) return launch_quant_t<D, 4, 2>(a, s);
  if (ab == 4 && rb == 4) return launch_quant_t<D, 4, 4>(a, s);
  if (ab == 2 && rb == 2) return launch_quant_t<D, 2, 2>(a, s);
  return launch_quant_t<D, 2, 4>(a, s);
}

hipError_t launch_quant_append(const QuantArgs& a, hipStream_t s) {
  switch (a.g.d) {
    case 64: return launch_quant_d<64>(a, s);
    case 96: return launch_quant_d<96>(a, s);
    default: return launch_quant_d<128>(a, s);
  }
}

}  // namespace rq
