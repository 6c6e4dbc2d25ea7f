// rq_stage.h -- device helpers shared by the decode kernels: vector types, the
// buffer resources and LDS-DMA staging of cache tiles, the fp16 "magic
// number" code unpack, and wave-wide reductions.  Included inside an
// anonymous namespace by each kernel source.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int NW = 4;              // waves per workgroup
constexpr float kEmpty = -1e30f;   // running max of an empty stream (finite on purpose)
constexpr float kLazy = 8.f;       // log2-domain headroom before the running max moves
constexpr uint32_t kMagic = 0x64006400u;  // fp16 pair (1024, 1024)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// A raw (unstrided) buffer resource: base address bits 0-31, bits 32-47,
// size in bytes, and the dword format word gfx9 needs for untyped loads.
typedef u32x4 rsrc_t;

// fp16 pair of two codes: v_and_or_b32 keeps the masked code bits and ORs in
// the exponent of 1024, so each half reads 1024 + 2^p * code.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
  return r;
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

// Calls f(integral_constant<K>) for K = 0..N-1 (keeps K a compile-time constant).
template <int N, int K = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (K < N) {
    f(std::integral_constant<int, K>{});
    static_for<N, K + 1>(f);
  }
}

// ------------------------------------------------------------ LDS-DMA staging
__device__ __forceinline__ rsrc_t make_rsrc(const uint8_t* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return (rsrc_t){(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// One DMA instruction moving G bytes per lane from buffer offset vo + so to
// LDS dst + G * lane.  Written as inline asm on purpose: the compiler's wait
// insertion cannot tell which LDS bytes a buffer_load ... lds writes, so
// with the builtin every LDS read after a DMA waits for ALL DMAs in flight,
// including the tile being prefetched.  The kernels synchronize the ring
// themselves with wait_vm (no VGPR is written by these loads, and their
// address operands are read at issue).
template <int G>
__device__ __forceinline__ void dma1(rsrc_t r, lds_u8* dst, int vo, uint32_t so) {
  const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(dst);
  if constexpr (G == 16)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0), "v"(vo), "s"(r), "s"(so) : "memory", "m0");
  else if constexpr (G == 4)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(m0), "v"(vo), "s"(r), "s"(so) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ushort %1, %2, %3 offen lds"
                 :: "s"(m0), "v"(vo), "s"(r), "s"(so) : "memory", "m0");
}

// BF16 alphas of a tile, one 2-byte DMA over all lanes (lane l lands at
// dst + 4 l); lanes past the tile's in-range tokens re-read the last one.
__device__ __forceinline__ void dma_alpha(rsrc_t r, uint32_t so, int tokens, lds_u8* dst, int lane) {
  dma1<2>(r, dst, min(lane, tokens - 1) * 2, so);
}

// s_waitcnt that waits until at most N vector-memory operations are pending;
// also a compiler barrier, so no LDS read of the staged tile moves above it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt has 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_u16(const lds_u8* p) {
  typedef __attribute__((address_space(3))) const uint16_t lh;
  return *reinterpret_cast<lh*>(p);
}

// ------------------------------------------------------------ wave helpers
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

}  // namespace
}  // namespace rq
