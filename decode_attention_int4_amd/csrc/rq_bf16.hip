// rq_bf16.hip -- split-K flash decode over an uncompressed BF16 cache: the
// baseline the packed path is compared against (ai4snews summary, paragraph 4,
// compares against BF16 attention).  Same decomposition as rq_decode.hip:
// 4 lanes per token, each lane owning d/4 contiguous elements (16-byte loads),
// per-slot online softmax, shuffle + LDS merges, and a combine kernel for the
// splits.
#include <hip/hip_runtime.h>

#include "rq_device.h"
#include "rq_kernels.h"

namespace rq {
namespace {

constexpr int NW = 4;
constexpr int LPT = 4;
constexpr int TPW = 64 / LPT;
constexpr float kEmpty = -1e30f;

template <int D>
__global__ void __launch_bounds__(NW * 64) bf16_decode_kernel(Bf16DecodeArgs a) {
  constexpr int E = D / LPT;     // elements per lane
  constexpr int W = E / 8;       // uint4 loads per lane per token
  __shared__ float sm_m[NW], sm_l[NW];
  __shared__ float sm_acc[NW][D];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.q_heads, hq = bh % a.q_heads, kvh = hq / a.group_ratio;
  const int slot = lane / LPT, part = lane % LPT;

  float qr[E];
#pragma unroll
  for (int i = 0; i < E; ++i) qr[i] = bf16_to_f32(a.q[(uint64_t)bh * D + part * E + i]) * a.qscale;

  const uint64_t head_off =
      ((((uint64_t)b * a.loops + a.loop) * a.layers + a.layer) * a.kv_heads + kvh) * (uint64_t)a.max_tokens * D;
  const uint16_t* kp = a.k + head_off + part * E;
  const uint16_t* vp = a.v + head_off + part * E;

  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  float m = kEmpty, l = 0.f;

  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(a.n_tokens, t_begin + a.tokens_per_split);

  // Slots past the end of the range load the range's last token (finite data)
  // and are masked out with p = 0.
  uint4 ck[W], cv[W], nk[W], nv[W];
  int base = t_begin + w * TPW;
  bool cur_ok = base + slot < t_end;
  if (base < t_end) {
    const int t = min(base + slot, t_end - 1);
#pragma unroll
    for (int i = 0; i < W; ++i) {
      ck[i] = reinterpret_cast<const uint4*>(kp + (uint64_t)t * D)[i];
      cv[i] = reinterpret_cast<const uint4*>(vp + (uint64_t)t * D)[i];
    }
  }
  for (; base < t_end; base += NW * TPW) {
    const int nb = base + NW * TPW;
    const bool nxt_ok = nb + slot < t_end;
    if (nb < t_end) {
      const int t = min(nb + slot, t_end - 1);
#pragma unroll
      for (int i = 0; i < W; ++i) {
        nk[i] = reinterpret_cast<const uint4*>(kp + (uint64_t)t * D)[i];
        nv[i] = reinterpret_cast<const uint4*>(vp + (uint64_t)t * D)[i];
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const uint32_t u[4] = {ck[i].x, ck[i].y, ck[i].z, ck[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dot = fmaf(qr[8 * i + 2 * j], __uint_as_float(u[j] << 16), dot);
        dot = fmaf(qr[8 * i + 2 * j + 1], __uint_as_float(u[j] & 0xFFFF0000u), dot);
      }
    }
#pragma unroll
    for (int o = 1; o < LPT; o <<= 1) dot += __shfl_xor(dot, o);
    const float logit = cur_ok ? dot : kEmpty;
    if (logit > m) {
      const float corr = exp2f(m - logit);
      l *= corr;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] *= corr;
      m = logit;
    }
    const float p = cur_ok ? exp2f(logit - m) : 0.f;
    l += p;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const uint32_t u[4] = {cv[i].x, cv[i].y, cv[i].z, cv[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[8 * i + 2 * j] = fmaf(p, __uint_as_float(u[j] << 16), acc[8 * i + 2 * j]);
        acc[8 * i + 2 * j + 1] = fmaf(p, __uint_as_float(u[j] & 0xFFFF0000u), acc[8 * i + 2 * j + 1]);
      }
    }
#pragma unroll
    for (int i = 0; i < W; ++i) {
      ck[i] = nk[i];
      cv[i] = nv[i];
    }
    cur_ok = nxt_ok;
  }

#pragma unroll
  for (int o = LPT; o < 64; o <<= 1) {
    const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
    const float M = fmaxf(m, mo);
    const float fs = exp2f(m - M), fo = exp2f(mo - M);
    l = l * fs + lo * fo;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = acc[i] * fs + __shfl_xor(acc[i], o) * fo;
    m = M;
  }
  if (lane < LPT) {
#pragma unroll
    for (int i = 0; i < E; ++i) sm_acc[w][part * E + i] = acc[i];
    if (lane == 0) {
      sm_m[w] = m;
      sm_l[w] = l;
    }
  }
  __syncthreads();
  float M = sm_m[0];
#pragma unroll
  for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm_m[ww]);
  float L = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) L += sm_l[ww] * exp2f(sm_m[ww] - M);
  float A = 0.f;
  if (tid < D) {
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) A += sm_acc[ww][tid] * exp2f(sm_m[ww] - M);
  }
  if (a.splits == 1) {
    if (tid < D) a.out[(uint64_t)bh * D + tid] = L > 0.f ? A / L : 0.f;
    return;
  }
  // partial state for the combine kernel (ordered by the kernel boundary)
  float* mine = a.partials + ((uint64_t)bh * a.splits + split) * (2 + D);
  if (tid < D) mine[2 + tid] = A;
  if (tid == 0) {
    mine[0] = M;
    mine[1] = L;
  }
}

template <int D>
__global__ void __launch_bounds__(128) bf16_combine_kernel(Bf16DecodeArgs a) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* all = a.partials + (uint64_t)bh * a.splits * (2 + D);
  float M = kEmpty, L = 0.f, A = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float* ps = all + (uint64_t)s * (2 + D);
    const float ms = ps[0];
    const float Mn = fmaxf(M, ms);
    const float fo = exp2f(M - Mn), fs = exp2f(ms - Mn);
    L = L * fo + ps[1] * fs;
    if (tid < D) A = A * fo + ps[2 + tid] * fs;
    M = Mn;
  }
  if (tid < D) a.out[(uint64_t)bh * D + tid] = L > 0.f ? A / L : 0.f;
}

template <int D>
hipError_t launch_t(const Bf16DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bf16_decode_kernel<D>), dim3(a.splits, a.batch * a.q_heads), dim3(NW * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((bf16_combine_kernel<D>), dim3(a.batch * a.q_heads), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int bf16_tile_tokens() { return NW * TPW; }

hipError_t launch_bf16_decode(const Bf16DecodeArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_t<64>(a, s);
    case 96: return launch_t<96>(a, s);
    default: return launch_t<128>(a, s);
  }
}

}  // namespace rq
