// rq_reconstruct.hip -- dequantize cached loops back to K/V vectors from two
// reads each: xhat = deq(anchor) + alpha * H^T deq(residual) (ai4snews
// summary, paragraph 3: shared-anchor reconstruction needs two cache reads).
// One wavefront per token vector, lane l holding elements l and l+64; the
// inverse rotation is diag(signs) * WHT / sqrt(n) done with lane shuffles in
// fp32.  Off the decode path: used to check the cache and to materialize it.
#include <hip/hip_runtime.h>

#include "rq_device.h"
#include "rq_kernels.h"

namespace rq {
namespace {

__device__ __forceinline__ float deq_elem(const uint8_t* slot, uint64_t sz_rel, int bits, int d,
                                          int t, int e) {
  const uint8_t* row = slot + (uint64_t)t * (d * bits / 8);
  const uint32_t byte = row[(e * bits) / 8];
  const uint32_t c = (byte >> ((e * bits) % 8)) & ((1u << bits) - 1u);
  const uint8_t* sz = slot + sz_rel + (uint64_t)t * (2 * (d / 16)) + 2 * (e / 16);
  return fp8_to_f32(sz[0]) * (float)c + fp8_to_f32(sz[1]);
}

template <int D>
__device__ __forceinline__ void wht_f32(float& y0, float& y1, int lane) {
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

template <int D>
__global__ void __launch_bounds__(256) reconstruct_kernel(ReconArgs a) {
  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const uint64_t wave_id = (uint64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const uint64_t n_waves = (uint64_t)gridDim.x * (blockDim.x / 64);
  const bool v1ok = (D > 64) && (lane + 64 < D);
  const float sc0 = (D == 128) ? 0.08838834764831845f : 0.125f;
  const float sc1 = (D == 128) ? 0.08838834764831845f : 0.17677669529663687f;

  for (uint64_t item = wave_id; item < a.vectors; item += n_waves) {
    const int tr = (int)(item % (uint64_t)a.n_out);
    uint64_t c = item / (uint64_t)a.n_out;
    const int head = (int)(c % g.kv_heads);
    c /= g.kv_heads;
    const int layer = (int)(c % g.layers);
    c /= g.layers;
    const int loop = (int)(c % g.loops);
    c /= g.loops;
    const int b = (int)(c % g.batch);
    const int kv = (int)(c / g.batch);
    const int t = a.tok_begin + tr;

    const bool direct = g.mode == RQ_MODE_DIRECT;
    const bool anchor = g.is_anchor(loop);
    const int aloop = (direct || anchor) ? loop : loop - loop % g.P + g.P - 1;
    const uint8_t* as = a.cache + g.slot_offset(kv, b, layer, aloop, head);
    const int abits = g.bits_of(aloop);
    float x0 = deq_elem(as, g.sz_rel(aloop), abits, D, t, lane);
    float x1 = v1ok ? deq_elem(as, g.sz_rel(aloop), abits, D, t, lane + 64) : 0.f;
    if (!direct && !anchor) {
      // sum alpha_i yhat_i over the residual planes this loop reads (its own;
      // chained mode: loops up to the anchor), then H^T once
      const int last = g.mode == RQ_MODE_CHAINED ? aloop - 1 : loop;
      float y0 = 0.f, y1 = 0.f;
      for (int rl = last; rl >= loop; --rl) {
        const uint8_t* rs = a.cache + g.slot_offset(kv, b, layer, rl, head);
        const float al = bf16_to_f32(
            reinterpret_cast<const uint16_t*>(a.cache + g.alpha_offset(kv, b, layer, rl, head))[t]);
        y0 = fmaf(al, deq_elem(rs, g.sz_rel(rl), g.residual_bits, D, t, lane), y0);
        if (v1ok) y1 = fmaf(al, deq_elem(rs, g.sz_rel(rl), g.residual_bits, D, t, lane + 64), y1);
      }
      if (g.rotation == RQ_ROT_HADAMARD) {
        wht_f32<D>(y0, y1, lane);
        const int8_t* sg = a.signs + ((uint64_t)kv * g.layers + layer) * D;
        y0 *= sc0 * (float)sg[lane];
        if (v1ok) y1 *= sc1 * (float)sg[lane + 64];
      }
      x0 += y0;
      x1 += y1;
    }
    const uint64_t o = item * D;
    if (a.out_bf16) {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + o;
      out[lane] = (uint16_t)f32_to_bf16(x0);
      if (v1ok) out[lane + 64] = (uint16_t)f32_to_bf16(x1);
    } else {
      float* out = reinterpret_cast<float*>(a.out) + o;
      out[lane] = x0;
      if (v1ok) out[lane + 64] = x1;
    }
  }
}

// Streaming-read probe: each workgroup reads one contiguous chunk of the
// buffer with non-temporal 16-byte loads, eight in flight per thread, and
// writes the XOR of its words to sink[blockIdx.x] (the XOR keeps the loads).
// Of the patterns measured on MI355X (grid-stride and chunked global loads,
// LDS-DMA rings, 256-2048 workgroups, 2-16 loads in flight, with and without
// the non-temporal hint), this one read fastest: about 7.0 TB/s over 8 GiB,
// and 6.4-6.5 TB/s for one decode call's 136 MB per launch.
__global__ void __launch_bounds__(256) read_probe_kernel(const uint4* buf, uint64_t n16, uint32_t* sink) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  constexpr int U = 8;
  uint32_t x = 0;
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t b0 = (uint64_t)blockIdx.x * per;
  const uint64_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint64_t i = b0 + threadIdx.x;
  for (; i + (U - 1) * 256 < b1; i += U * 256) {
    u4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(buf + i + u * 256));
    // all U loads issue before any result is used (left alone, the scheduler
    // interleaved the XORs and kept one or two loads in flight)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += 256) {
    const u4 a = __builtin_nontemporal_load(reinterpret_cast<const u4*>(buf + i));
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_reconstruct(const ReconArgs& a, hipStream_t s) {
  uint64_t blocks = (a.vectors + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  switch (a.g.d) {
    case 64: hipLaunchKernelGGL(reconstruct_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    case 96: hipLaunchKernelGGL(reconstruct_kernel<96>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(reconstruct_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace rq
