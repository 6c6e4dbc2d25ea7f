// rq_stage.h -- device helpers shared by the decode kernels: vector types, the
// buffer resources and LDS-DMA staging of cache tiles, the fp16 "magic
// number" code unpack, and wave-wide reductions.  Included inside an
// anonymous namespace by each kernel source.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rq_kernels.h"

namespace rq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr float kEmpty = -1e30f;   // running max of an empty stream (finite on purpose)
constexpr float kLazy = 8.f;       // log2-domain headroom before the running max moves
constexpr uint32_t kMagic = 0x64006400u;  // fp16 pair (1024, 1024)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// A raw (unstrided) buffer resource: base address bits 0-31, bits 32-47,
// size in bytes, and the dword format word gfx9 needs for untyped loads.
typedef u32x4 rsrc_t;

// fp16 pair of two codes: v_and_or_b32 keeps the masked code bits and ORs in
// the exponent of 1024, so each half reads 1024 + 2^p * code.  Plain C, which
// the compiler selects as that one instruction: as inline asm its writes were
// invisible to the compiler's hazard checks, so a code operand rebuilt right
// after the matrix op reading it could change under that op, and every use
// paid a conservative wait state.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  return (x & mask) | magic;
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
// NT marks the load non-temporal: cache-plane bytes are read once per call,
// and the streaming hint raised a plain read of a decode call's bytes from
// 5.9 to 6.5 TB/s on MI355X (136 MB per launch, back-to-back launches).
template <int G, bool NT = false>
__device__ __forceinline__ void dma1(rsrc_t r, lds_u8* dst, int vo, uint32_t so) {
  const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(dst);
  if constexpr (NT) {
    if constexpr (G == 16)
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                   :: "s"(m0), "v"(vo), "s"(r), "s"(so) : "memory", "m0");
    else if constexpr (G == 4)
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen nt lds"
                   :: "s"(m0), "v"(vo), "s"(r), "s"(so) : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ushort %1, %2, %3 offen nt lds"
                   :: "s"(m0), "v"(vo), "s"(r), "s"(so) : "memory", "m0");
  } else {
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
}

// BF16 alphas of a tile, one 2-byte DMA over all lanes (lane l lands at
// dst + 4 l); lanes past the tile's in-range tokens re-read the last one.
__device__ __forceinline__ void dma_alpha(rsrc_t r, uint32_t so, int tokens, lds_u8* dst, int lane) {
  dma1<2, true>(r, dst, min(lane, tokens - 1) * 2, so);
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
__device__ __forceinline__ uint32_t lds_u32(const lds_u8* p) {
  typedef __attribute__((address_space(3))) const uint32_t lw;
  return *reinterpret_cast<lw*>(p);
}

// ------------------------------------------------------------ wave helpers
// Cross-lane moves inside 16-lane rows by DPP (a VALU modifier, no LDS round
// trip as for ds_bpermute): quad permutations, row shifts and mirrors.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowShl4 = 0x104;    // lane i reads lane i + 4 of its row
constexpr int kDppRowShr4 = 0x114;    // lane i reads lane i - 4
constexpr int kDppRowShl8 = 0x108;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppHalfMirror = 0x141;  // lane i reads lane 7 - i of its half row
constexpr int kDppRowMirror = 0x140;   // lane i reads lane 15 - i of its row
constexpr int kDppRowRor8 = 0x128;     // lane i reads lane (i + 8) mod 16 = i ^ 8

// Lanes whose source is outside the row keep their own value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  const int x = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false));
}

// Rows and halves of the wave across lanes by the gfx950 permlane swaps
// (VALU, no LDS round trip).  With both operands v, permlane16_swap returns
// rows (0, 0, 2, 2) and (1, 1, 3, 3) of v and permlane32_swap the halves
// (low, low) and (high, high): the two results at a lane are v of the lane
// and of its partner lane ^ 16 (lane ^ 32), in row (half) order.
typedef float fpair __attribute__((ext_vector_type(2)));
template <int H>
__device__ __forceinline__ fpair swap_rows(float v) {
  static_assert(H == 16 || H == 32, "row or half swap");
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = H == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return (fpair){__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}

// The value of lane (lane ^ H).  For H = 4 and 8 both row shifts run on all
// lanes before the select: a DPP read from a lane that is switched off (as
// in either arm of a branch on the lane's bit) does not return its value.
template <int H>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  if constexpr (H == 1) {
    return dpp_f<kDppQuadXor1>(v);
  } else if constexpr (H == 2) {
    return dpp_f<kDppQuadXor2>(v);
  } else if constexpr (H == 4 || H == 8) {
    const float up = dpp_f<H == 4 ? kDppRowShl4 : kDppRowShl8>(v);
    const float down = dpp_f<H == 4 ? kDppRowShr4 : kDppRowShr8>(v);
    return (lane & H) ? down : up;
  } else {
    const fpair r = swap_rows<H>(v);
    return (lane & H) ? r.x : r.y;
  }
}

// Sum and maximum of v over lanes l and l ^ H (H = 16, 32).
template <int H>
__device__ __forceinline__ float pair_add(float v) {
  const fpair r = swap_rows<H>(v);
  return r.x + r.y;
}
template <int H>
__device__ __forceinline__ float pair_max(float v) {
  const fpair r = swap_rows<H>(v);
  return fmaxf(r.x, r.y);
}

// Sum and maximum over each 16-lane row (every lane of the row gets them):
// after the two quad steps a quad holds its total, the half mirror pairs
// the quads of each half row and the mirror the two halves.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppRowMirror>(v);
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppRowMirror>(v));
}

// One butterfly stage of the transform below: lane i pairs with i ^ H.
template <int H>
__device__ __forceinline__ float wht_stage(float y, int lane) {
  const float p = xor_lane<H>(y, lane);
  return (lane & H) ? (p - y) : (y + p);
}

// Walsh-Hadamard transform of a vector held two elements per lane (l, l+64)
// by one wave; block diagonal 64+32 when D == 96.  Unscaled.
template <int D>
__device__ __forceinline__ void wave_wht(float& y0, float& y1, int lane) {
  static_for<6>([&](auto K) {
    constexpr int h = 1 << decltype(K)::value;
    y0 = wht_stage<h>(y0, lane);
    if constexpr (D == 128 || (D == 96 && h < 32)) y1 = wht_stage<h>(y1, lane);
  });
  if constexpr (D == 128) {
    const float a = y0, b = y1;
    y0 = a + b;
    y1 = a - b;
  }
}

__device__ __forceinline__ float wave_max(float v) {
  return pair_max<32>(pair_max<16>(row_max16(v)));
}

// 2^k with max|v| * 2^k in [2^13, 2^14): fp16 then holds BF16 inputs exactly.
__device__ __forceinline__ float fp16_prescale(float maxabs) {
  if (!(maxabs > 0.f)) return 1.f;
  int e;
  frexpf(maxabs, &e);
  return ldexpf(1.f, 14 - e);
}


// ------------------------------------------------------------ split-K merge
// Device-wide (agent scope) relaxed accesses.  Stores write through to the
// memory level that all XCDs share and loads read from it (global_store and
// global_load with sc1), so partial states pass between workgroups on
// different XCDs without cache write-backs or invalidations.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every thread of a workgroup once its partial states are stored
// with store_dev.  Each wave first waits until its own stores have completed,
// then one thread takes a ticket from counter `ctr`; the workgroup that
// arrives last sees every other partial already written, resets the counter
// to zero for the next call and returns true.  `ticket` is a word of LDS.
__device__ __forceinline__ bool arrive_last(const DecodeArgs& a, int ctr, int ns, int tid,
                                            uint32_t* ticket) {
  wait_vm<0>();
  __syncthreads();
  if (tid == 0)
    *ticket = __hip_atomic_fetch_add(a.counters + ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const bool last = *ticket == (uint32_t)ns - 1u;
  if (last && tid == 0) __hip_atomic_store(a.counters + ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// Merges the split partial states (m, l, accA[D], accR[D]) of one (batch row,
// query head), applies H^T to the residual sum and writes the fp32 output;
// one wave, two elements per lane.  Splits are merged online, R per round,
// so each round's loads issue together and the merge waits on memory about
// once per R splits (merge_splits picks R for the split count, so a call
// with four splits issues four splits' loads, not sixteen).
template <int D, bool TWO, int R>
__device__ __forceinline__ void merge_row(const DecodeArgs& a, int bh, int ns, int lane) {
  constexpr int W = 2 + 2 * D;
  const bool v1ok = (D > 64) && (lane + 64 < D);
  const float* all = a.partials + (uint64_t)bh * a.splits * W;   // row stride: a.splits states
  float M = kEmpty, L = 0.f, A0 = 0.f, A1 = 0.f, R0 = 0.f, R1 = 0.f;
  for (int s0 = 0; s0 < ns; s0 += R) {
    float ms[R], ls[R], a0[R], a1[R], r0[R], r1[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int sj = min(s0 + j, ns - 1);
      const float* ps = all + (uint64_t)sj * W;
      ms[j] = (s0 + j < ns) ? load_dev(ps) : kEmpty;
      ls[j] = load_dev(ps + 1);
      a0[j] = load_dev(ps + 2 + lane);
      a1[j] = v1ok ? load_dev(ps + 2 + lane + 64) : 0.f;
      r0[j] = TWO ? load_dev(ps + 2 + D + lane) : 0.f;
      r1[j] = (TWO && v1ok) ? load_dev(ps + 2 + D + lane + 64) : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < R; ++j) Mn = fmaxf(Mn, ms[j]);
    const float c = __builtin_amdgcn_exp2f(M - Mn);
    L *= c;
    A0 *= c;
    A1 *= c;
    R0 *= c;
    R1 *= c;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float f = __builtin_amdgcn_exp2f(ms[j] - Mn);
      L = fmaf(f, ls[j], L);
      A0 = fmaf(f, a0[j], A0);
      A1 = fmaf(f, a1[j], A1);
      R0 = fmaf(f, r0[j], R0);
      R1 = fmaf(f, r1[j], R1);
    }
    M = Mn;
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

template <int D, bool TWO>
__device__ __forceinline__ void merge_splits(const DecodeArgs& a, int bh, int ns, int lane) {
  if (ns <= 4) merge_row<D, TWO, 4>(a, bh, ns, lane);
  else if (ns <= 8) merge_row<D, TWO, 8>(a, bh, ns, lane);
  else merge_row<D, TWO, 16>(a, bh, ns, lane);
}

}  // namespace
}  // namespace rq
