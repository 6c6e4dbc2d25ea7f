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
// Work decomposition (gfx950, wave64):
//   grid (splits, batch * q_heads); 4 waves per workgroup.
//   LPT lanes share one token; each owns GPL consecutive groups of 16 (a
//   contiguous byte range of every plane), so a wave reads 64 lanes x 16 bytes
//   of anchor codes per instruction, contiguous across lanes.
//   Each lane slot keeps its own online-softmax state over its token stream;
//   states are merged across slots with lane shuffles, across waves in LDS,
//   and across splits by the last workgroup to finish (a per-(b,h) counter in
//   the workspace), which also applies H^T and writes the fp32 output.
#include <hip/hip_runtime.h>

#include "rq_device.h"
#include "rq_kernels.h"

namespace rq {
namespace {

constexpr int NW = 4;             // waves per workgroup
constexpr float kEmpty = -1e30f;  // running max of an empty stream (finite on purpose)

template <int D>
struct Shape {
  static constexpr int NG = D / 16;
  static constexpr int LPT = (D == 96) ? 2 : NG / 2;  // lanes per token
  static constexpr int GPL = NG / LPT;                 // groups per lane
  static constexpr int E = GPL * 16;                   // elements per lane
  static constexpr int TPW = 64 / LPT;                 // tokens per wave step
};

// Loads BYTES bytes at p (aligned to ALIGN) into 32-bit words, low bytes first.
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

// One plane (codes + sz) as seen by one lane for one token.
template <int D, int BITS>
struct PlaneView {
  using S = Shape<D>;
  static constexpr int CB = S::E * BITS / 8;          // code bytes per lane
  static constexpr int CW = CB / 4;                   // code words per lane
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

template <int BITS>
__device__ __forceinline__ float code_at(const uint32_t* c, int i) {
  constexpr uint32_t M = (1u << BITS) - 1;
  return (float)((c[(i * BITS) / 32] >> ((i * BITS) % 32)) & M);
}

__device__ __forceinline__ uint32_t sz_byte(const uint32_t* s, int b) {
  return (s[b / 4] >> (8 * (b % 4))) & 0xFFu;
}

// sum over the lane's groups of  s_g * sum_i(w_i c_i) + z_g * wsum_g
template <int D, int BITS>
__device__ __forceinline__ float plane_dot(const PlaneData<D, BITS>& pd, const float* w,
                                           const float* wsum) {
  using S = Shape<D>;
  float acc = 0.f;
#pragma unroll
  for (int gi = 0; gi < S::GPL; ++gi) {
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) dot = fmaf(w[gi * 16 + i], code_at<BITS>(pd.c, gi * 16 + i), dot);
    const float s = fp8_to_f32(sz_byte(pd.s, 2 * gi));
    const float z = fp8_to_f32(sz_byte(pd.s, 2 * gi + 1));
    acc = fmaf(s, dot, fmaf(z, wsum[gi], acc));
  }
  return acc;
}

// acc_i += p * (s_g c_i + z_g)
template <int D, int BITS>
__device__ __forceinline__ void plane_axpy(const PlaneData<D, BITS>& pd, float p, float* acc) {
  using S = Shape<D>;
#pragma unroll
  for (int gi = 0; gi < S::GPL; ++gi) {
    const float ps = p * fp8_to_f32(sz_byte(pd.s, 2 * gi));
    const float pz = p * fp8_to_f32(sz_byte(pd.s, 2 * gi + 1));
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[gi * 16 + i] = fmaf(ps, code_at<BITS>(pd.c, gi * 16 + i), acc[gi * 16 + i] + pz);
  }
}

template <int D, int B1, int B2>
struct TokenData {
  PlaneData<D, B1> k1, v1;
  PlaneData<D, (B2 ? B2 : 2)> k2, v2;
  uint32_t ka, va;  // BF16 alphas
};

// Walsh-Hadamard transform of an LDS vector of length D (block diagonal 64+32
// when D == 96), scaled to be orthonormal.  Called by the whole workgroup.
template <int D>
__device__ __forceinline__ void lds_wht(float* v) {
  const int i = threadIdx.x;
  const int blk = (D == 96 && i >= 64) ? 32 : (D == 96 ? 64 : D);
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
    float nv = 0.f;
    const bool act = i < D && h < blk;
    if (act) {
      const float a = v[i], b = v[i ^ h];
      nv = (i & h) ? (b - a) : (a + b);
    }
    __syncthreads();
    if (act) v[i] = nv;
    __syncthreads();
  }
  if (i < D) v[i] *= rsqrtf((float)blk);
  __syncthreads();
}

template <int D, int B1, int B2>
__global__ void __launch_bounds__(NW * 64) decode_kernel(DecodeArgs a) {
  using S = Shape<D>;
  constexpr int E = S::E, LPT = S::LPT, TPW = S::TPW, GPL = S::GPL;
  constexpr bool TWO = B2 != 0;
  constexpr int B2E = TWO ? B2 : 2;
  const Geometry& g = a.g;

  __shared__ float sq[D], su[D], sR[D];
  __shared__ float sm_m[NW], sm_l[NW];
  __shared__ float sm_acc[NW][2 * D];
  __shared__ int sm_last;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.q_heads, hq = bh % a.q_heads, kvh = hq / a.group_ratio;
  const int slot = lane / LPT, part = lane % LPT;
  const bool rotated = TWO && g.rotation == RQ_ROT_HADAMARD;

  // ---- query (scaled into the log2 domain) and u = H q
  if (tid < D) {
    const float qv = bf16_to_f32(a.q[(uint64_t)bh * D + tid]) * a.qscale;
    sq[tid] = qv;
    su[tid] = rotated ? qv * (float)a.signs[(uint64_t)g.layers * 0 + (uint64_t)a.layer * D + tid] : qv;
  }
  __syncthreads();
  if (rotated) lds_wht<D>(su);

  float qr[E], ur[TWO ? E : 1], qsum[GPL], usum[GPL];
#pragma unroll
  for (int i = 0; i < E; ++i) qr[i] = sq[part * E + i];
#pragma unroll
  for (int gi = 0; gi < GPL; ++gi) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += qr[gi * 16 + i];
    qsum[gi] = s;
  }
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

  auto load_tok = [&](TokenData<D, B1, B2>& td, int t) {
    load_plane<D, B1>(td.k1, k1, k1s, t, part);
    load_plane<D, B1>(td.v1, v1, v1s, t, part);
    if constexpr (TWO) {
      load_plane<D, B2E>(td.k2, k2, k2s, t, part);
      load_plane<D, B2E>(td.v2, v2, v2s, t, part);
      td.ka = k2a[t];
      td.va = v2a[t];
    }
  };

  float accA[E], accR[TWO ? E : 1];
#pragma unroll
  for (int i = 0; i < E; ++i) accA[i] = 0.f;
  if constexpr (TWO) {
#pragma unroll
    for (int i = 0; i < E; ++i) accR[i] = 0.f;
  }
  float m = kEmpty, l = 0.f;

  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(a.n_tokens, t_begin + a.tokens_per_split);

  TokenData<D, B1, B2> cur, nxt;
  int base = t_begin + w * TPW;
  bool cur_ok = base + slot < t_end;
  if (cur_ok) load_tok(cur, base + slot);
  for (; base < t_end; base += NW * TPW) {
    const int nb = base + NW * TPW;
    const bool nxt_ok = nb + slot < t_end;
    if (nxt_ok) load_tok(nxt, nb + slot);

    float part_logit = plane_dot<D, B1>(cur.k1, qr, qsum);
    if constexpr (TWO) part_logit = fmaf(bf16_to_f32(cur.ka), plane_dot<D, B2E>(cur.k2, ur, usum), part_logit);
#pragma unroll
    for (int o = 1; o < LPT; o <<= 1) part_logit += __shfl_xor(part_logit, o);
    const float logit = cur_ok ? part_logit : kEmpty;
    if (logit > m) {
      const float corr = exp2f(m - logit);
      l *= corr;
#pragma unroll
      for (int i = 0; i < E; ++i) accA[i] *= corr;
      if constexpr (TWO) {
#pragma unroll
        for (int i = 0; i < E; ++i) accR[i] *= corr;
      }
      m = logit;
    }
    const float p = cur_ok ? exp2f(logit - m) : 0.f;
    l += p;
    plane_axpy<D, B1>(cur.v1, p, accA);
    if constexpr (TWO) plane_axpy<D, B2E>(cur.v2, p * bf16_to_f32(cur.va), accR);

    cur = nxt;
    cur_ok = nxt_ok;
  }

  // ---- merge the lane slots of this wave (lanes with equal `part`)
#pragma unroll
  for (int o = LPT; o < 64; o <<= 1) {
    const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
    const float M = fmaxf(m, mo);
    const float fs = exp2f(m - M), fo = exp2f(mo - M);
    l = l * fs + lo * fo;
#pragma unroll
    for (int i = 0; i < E; ++i) accA[i] = accA[i] * fs + __shfl_xor(accA[i], o) * fo;
    if constexpr (TWO) {
#pragma unroll
      for (int i = 0; i < E; ++i) accR[i] = accR[i] * fs + __shfl_xor(accR[i], o) * fo;
    }
    m = M;
  }
  if (lane < LPT) {
#pragma unroll
    for (int i = 0; i < E; ++i) sm_acc[w][part * E + i] = accA[i];
    if constexpr (TWO) {
#pragma unroll
      for (int i = 0; i < E; ++i) sm_acc[w][D + part * E + i] = accR[i];
    }
    if (lane == 0) {
      sm_m[w] = m;
      sm_l[w] = l;
    }
  }
  __syncthreads();

  // ---- merge the waves and publish this split's partial state
  float* mine = a.partials + ((uint64_t)bh * a.splits + split) * (2 + 2 * D);
  {
    float M = sm_m[0];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm_m[ww]);
    for (int i = tid; i < 2 * D; i += NW * 64) {
      if (!TWO && i >= D) {
        mine[2 + i] = 0.f;
        continue;
      }
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) s += sm_acc[ww][i] * exp2f(sm_m[ww] - M);
      mine[2 + i] = s;
    }
    if (tid == 0) {
      float L = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) L += sm_l[ww] * exp2f(sm_m[ww] - M);
      mine[0] = M;
      mine[1] = L;
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&a.counters[bh], 1u);
    sm_last = (prev == (uint32_t)(a.splits - 1));
    __threadfence();
  }
  __syncthreads();
  if (!sm_last) return;
  __threadfence();

  // ---- last workgroup of this (b, h): merge all splits
  const float* all = a.partials + (uint64_t)bh * a.splits * (2 + 2 * D);
  float M = kEmpty;
  for (int s = 0; s < a.splits; ++s)
    M = fmaxf(M, __hip_atomic_load(all + (uint64_t)s * (2 + 2 * D), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  float L = 0.f, A = 0.f, R = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float* ps = all + (uint64_t)s * (2 + 2 * D);
    const float f = exp2f(__hip_atomic_load(ps, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - M);
    L += f * __hip_atomic_load(ps + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < D) {
      A += f * __hip_atomic_load(ps + 2 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (TWO) R += f * __hip_atomic_load(ps + 2 + D + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (rotated) {
    if (tid < D) sR[tid] = R;
    __syncthreads();
    lds_wht<D>(sR);
    if (tid < D) R = sR[tid] * (float)a.signs[((uint64_t)g.layers + a.layer) * D + tid];
  }
  if (tid < D) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    a.out[(uint64_t)bh * D + tid] = (A + R) * inv;
  }
  if (tid == 0) a.counters[bh] = 0u;
}

template <int D, int B1, int B2>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<D, B1, B2>), dim3(a.splits, a.g.batch * a.q_heads), dim3(NW * 64), 0, s, a);
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
