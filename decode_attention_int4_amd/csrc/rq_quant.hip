// rq_quant.hip -- quantize-and-append of looped-Transformer K/V states.
//
// One wavefront encodes one (kv, batch row, layer, kv head, token, loop group):
// lane l holds head_dim elements l and l+64.  The anchor (last loop of the
// group) is quantized at anchor_bits; every other loop's residual against the
// dequantized anchor is rotated by H = (1/sqrt(n)) WHT diag(signs), quantized
// at residual_bits and given a BF16 least-squares scale (ai4snews summary,
// paragraphs 1-2; agihunt "Confirmed" list).  Every value that decides a
// stored code, FP8 byte or BF16 alpha is computed in IEEE double precision;
// MI355X runs fp64 vector arithmetic at the fp32 rate, and this step is
// latency-bound at decode (one token per step) anyway.
//
// Group min/max and the alpha dot products are wavefront reductions over
// __shfl_xor; the Walsh-Hadamard butterflies run across lanes (index bits 1-32)
// and in-lane (bit 64).
#include <hip/hip_runtime.h>

#include "rq_device.h"
#include "rq_kernels.h"

#pragma clang fp contract(off)

namespace rq {
namespace {

struct QuantResult {
  uint32_t code0, code1;   // codes of elements lane, lane+64
  uint32_t sz0, sz1;       // scale | offset << 8 of their groups
  double deq0, deq1;       // dequantized values
};

// Asymmetric min/max quantization of the 16-lane group each element lives in.
template <int Q>
__device__ __forceinline__ void quant_elem(double x, uint32_t& code, uint32_t& sz, double& deq) {
  double mn = x, mx = x;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    mn = fmin(mn, __shfl_xor(mn, o));
    mx = fmax(mx, __shfl_xor(mx, o));
  }
  const uint32_t s8 = f64_to_fp8((mx - mn) / (double)Q);
  const uint32_t z8 = f64_to_fp8(mn);
  const double s = fp8_to_f64(s8);
  const double z = fp8_to_f64(z8);
  double c = 0.0;
  if (s != 0.0) {
    c = rint((x - z) / s);
    c = fmin(fmax(c, 0.0), (double)Q);
  }
  code = (uint32_t)c;
  sz = s8 | (z8 << 8);
  deq = s * c + z;
}

template <int D, int BITS>
__device__ __forceinline__ QuantResult quant_vec(double x0, double x1) {
  constexpr int Q = (1 << BITS) - 1;
  QuantResult r;
  quant_elem<Q>(x0, r.code0, r.sz0, r.deq0);
  if constexpr (D > 64) {
    quant_elem<Q>(x1, r.code1, r.sz1, r.deq1);
  } else {
    r.code1 = r.sz1 = 0;
    r.deq1 = 0.0;
  }
  return r;
}

// Packs the codes of one token vector into its row (element e at bit e*BITS).
template <int D, int BITS>
__device__ __forceinline__ void store_codes(uint8_t* row, uint8_t* sz_row, const QuantResult& r,
                                            int lane) {
  constexpr int PER = 32 / BITS;  // codes per dword
  uint32_t v0 = r.code0 << ((lane % PER) * BITS);
  uint32_t v1 = r.code1 << ((lane % PER) * BITS);
#pragma unroll
  for (int o = 1; o < PER; o <<= 1) {
    v0 |= __shfl_xor(v0, o);
    if constexpr (D > 64) v1 |= __shfl_xor(v1, o);
  }
  if (lane % PER == 0) {
    reinterpret_cast<uint32_t*>(row)[lane / PER] = v0;
    if (D > 64 && lane + 64 < D) reinterpret_cast<uint32_t*>(row)[(lane + 64) / PER] = v1;
  }
  if (lane % 16 == 0) {
    reinterpret_cast<uint16_t*>(sz_row)[lane / 16] = (uint16_t)r.sz0;
    if (D > 64 && lane + 64 < D) reinterpret_cast<uint16_t*>(sz_row)[(lane + 64) / 16] = (uint16_t)r.sz1;
  }
}

// y = WHT (in place over the lane-distributed vector), unscaled.
template <int D>
__device__ __forceinline__ void wht(double& y0, double& y1, int lane) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const double p0 = __shfl_xor(y0, h);
    y0 = (lane & h) ? (p0 - y0) : (y0 + p0);
    if constexpr (D == 128) {
      const double p1 = __shfl_xor(y1, h);
      y1 = (lane & h) ? (p1 - y1) : (y1 + p1);
    } else if constexpr (D == 96) {
      if (h < 32) {  // second block has 32 elements (lanes 0-31)
        const double p1 = __shfl_xor(y1, h);
        y1 = (lane & h) ? (p1 - y1) : (y1 + p1);
      }
    }
  }
  if constexpr (D == 128) {
    const double a = y0, b = y1;
    y0 = a + b;
    y1 = a - b;
  }
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

template <int D, int AB, int RB>
__global__ void __launch_bounds__(256) quant_append_kernel(QuantArgs a) {
  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const uint64_t wave_id = (uint64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const uint64_t n_waves = (uint64_t)gridDim.x * (blockDim.x / 64);
  const int G = g.loops / g.P;
  const bool v1ok = (D > 64) && (lane + 64 < D);
  // per-block scales of the Walsh-Hadamard transform
  const double sc0 = (D == 128) ? 1.0 / sqrt(128.0) : 1.0 / sqrt(64.0);
  const double sc1 = (D == 128) ? 1.0 / sqrt(128.0) : 1.0 / sqrt(32.0);

  for (uint64_t item = wave_id; item < a.items; item += n_waves) {
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
      // outside the pool, is skipped (all wave-uniform)
      const int cap = a.paging.max_blocks << a.paging.block_shift;
      const int p0 = a.positions[b];
      if (p0 < 0 || p0 > cap - a.t_new) continue;
      const int lp = p0 + t;
      slot_row = a.paging.table[(uint64_t)b * a.paging.max_blocks + (lp >> a.paging.block_shift)];
      if (slot_row < 0 || slot_row >= g.batch) continue;
      pos = lp & ((1 << a.paging.block_shift) - 1);
    } else if (a.positions) {
      // per-row positions come from device memory: a row whose range does not
      // fit the cache is skipped (the whole wave agrees, b is wave-uniform)
      const int p0 = a.positions[b];
      if (p0 < 0 || p0 > g.max_tokens - a.t_new) continue;
      pos = p0 + t;
    }

    auto src = [&](int loop) {
      return a.kv + ((((uint64_t)(kv * a.rows + b) * g.loops + loop) * g.layers + layer) *
                         g.kv_heads + head) * (uint64_t)a.t_new * D + (uint64_t)t * D;
    };
    auto load = [&](int loop, double& x0, double& x1) {
      const uint16_t* p = src(loop);
      x0 = (double)bf16_to_f32(p[lane]);
      x1 = v1ok ? (double)bf16_to_f32(p[lane + 64]) : 0.0;
    };

    // ---- anchor
    const int aloop = k * g.P + g.P - 1;
    double x0, x1;
    load(aloop, x0, x1);
    const QuantResult A = quant_vec<D, AB>(x0, x1);
    {
      uint8_t* base = a.cache + g.slot_offset(kv, slot_row, layer, aloop, head);
      store_codes<D, AB>(base + (uint64_t)pos * (D * AB / 8),
                         base + g.sz_rel(aloop) + (uint64_t)pos * (2 * D / 16), A, lane);
    }

    // ---- other loops of the group.  Chained mode walks from the loop next to
    // the anchor outwards: corr = sum alpha_i yhat_i over the loops already
    // stored, so y = H (x_l - deq(A)) - corr is the rotated residual against
    // the reconstruction of loop l + 1
    const bool chained = g.mode == RQ_MODE_CHAINED;
    double corr0 = 0.0, corr1 = 0.0;
    for (int jj = 0; jj < g.P - 1; ++jj) {
      const int j = chained ? g.P - 2 - jj : jj;
      const int loop = k * g.P + j;
      load(loop, x0, x1);
      uint8_t* base = a.cache + g.slot_offset(kv, slot_row, layer, loop, head);
      uint8_t* row = base + (uint64_t)pos * (D * RB / 8);
      uint8_t* sz_row = base + g.sz_rel(loop) + (uint64_t)pos * (2 * D / 16);
      if (g.mode == RQ_MODE_DIRECT) {
        store_codes<D, RB>(row, sz_row, quant_vec<D, RB>(x0, x1), lane);
        continue;
      }
      double y0 = x0 - A.deq0;
      double y1 = v1ok ? (x1 - A.deq1) : 0.0;
      if (g.rotation == RQ_ROT_HADAMARD) {
        const int8_t* sg = a.signs + ((uint64_t)kv * g.layers + layer) * D;
        y0 *= (double)sg[lane];
        if (v1ok) y1 *= (double)sg[lane + 64];
        wht<D>(y0, y1, lane);
        // + 0.0 turns a -0 into +0 and changes nothing else: an element of
        // H r whose exact sum is zero is +0 (a sum accumulated from zero),
        // whatever signed zeros the butterflies passed through, so the FP8
        // offset of an all-zero residual group is +0 (0x00), not 0x80
        y0 = y0 * sc0 + 0.0;
        y1 = v1ok ? y1 * sc1 + 0.0 : 0.0;
      }
      if (chained) {
        y0 -= corr0;
        y1 = v1ok ? y1 - corr1 : 0.0;
      }
      const QuantResult R = quant_vec<D, RB>(y0, y1);
      store_codes<D, RB>(row, sz_row, R, lane);
      const double yh1 = v1ok ? R.deq1 : 0.0;
      const double num = wave_sum(y0 * R.deq0 + y1 * yh1);
      const double den = wave_sum(R.deq0 * R.deq0 + yh1 * yh1);
      const double yy = wave_sum(y0 * y0 + y1 * y1);
      uint32_t al;
      if (g.alpha_mode == RQ_ALPHA_ONE)
        al = 0x3F80u;
      else if (!(den > 0.0))
        al = 0u;
      else if (g.alpha_mode == RQ_ALPHA_NORM_RATIO)
        al = f64_to_bf16(sqrt(yy) / sqrt(den));
      else
        al = f64_to_bf16(num / den);
      if (lane == 0)
        reinterpret_cast<uint16_t*>(base + g.alpha_rel(loop))[pos] = (uint16_t)al;
      if (chained) {
        const double ab = (double)bf16_to_f32((uint16_t)al);
        corr0 += ab * R.deq0;
        corr1 = v1ok ? corr1 + ab * R.deq1 : 0.0;
      }
    }
  }
}

}  // namespace

template <int D, int AB, int RB>
static hipError_t launch_quant_t(const QuantArgs& a, hipStream_t s) {
  const uint64_t waves_needed = a.items;
  uint64_t blocks = (waves_needed + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((quant_append_kernel<D, AB, RB>), dim3((unsigned)blocks), dim3(256), 0, s, a);
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
