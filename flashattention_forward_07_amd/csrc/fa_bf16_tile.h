// fa_bf16_tile.h -- device pieces shared by the bf16 forward kernels: the
// LDS layout of a K/V tile, operand reads issued by hand, lane exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_common.h"

namespace fa355 {
namespace bf16t {

template <int D, int BN_>
struct Bf16Tile {
  static constexpr int BN = BN_;
  // (32 keys: the key-split kernel, whose per-wave rings would not fit in
  // LDS with 64-key tiles)
  static_assert(BN == 64 || (BN == 128 && D == 64) || BN == 32, "keys per tile");
  static constexpr int ROWB = D * 2;              // bytes per K/V row
  static constexpr int TILE = BN * ROWB;          // bytes per K (or V) tile
  static constexpr int STAGE = 2 * TILE;          // K tile then V tile
  static constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  // K: rows read 16 at a time at one logical chunk -> spread over all slots.
  static __device__ __forceinline__ int swz_k(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
  }
  // V: four consecutive rows x 64 bytes per 32-lane transposed read.
  static __device__ __forceinline__ int swz_v(int r) {
    return D == 128 ? (10 * (r & 1) + 4 * ((r >> 1) & 1)) : (6 * ((r >> 1) & 1));
  }
};

// Workgroup barrier that also completes this wave's LDS writes first.  The
// wait is the builtin (lgkmcnt = 0, other counters untouched) rather than
// inline assembly, so the compiler's own wait insertion knows that scalar
// loads issued before it have completed and does not wait again inside the
// loop, where such a wait would also stall on this wave's LDS writes.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>).
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Operand reads of the matrix-core phase are issued by hand: the compiler
// cannot tell them apart from the LDS the in-flight global->LDS loads are
// filling and would wait for those loads before every read.  Completion is
// awaited with lgkm_wait, which is tied to the destination registers so no
// consumer can be scheduled above it.
template <int OFF>
__device__ __forceinline__ u32x4_t lds_read_b128(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x4_t d;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "i"(OFF));
  return d;
}
template <int OFF>
__device__ __forceinline__ u32x2_t lds_read_tr16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x2_t d;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "i"(OFF));
  return d;
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4_t &a, u32x2_t &b, u32x2_t &c) {
  asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a), "+v"(b), "+v"(c) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4_t &a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x2_t &a, u32x2_t &b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// v_max3_f32 / v_max_f32 without the NaN-quieting canonicalisation the
// compiler adds to fmaxf on values it cannot prove canonical (scores are
// never NaN for finite inputs).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ bf16x8_t cat_bf16(u32x2_t lo, u32x2_t hi) {
  const u32x4_t x = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8_t, x);
}

// Exchange with lane ^ 32: v_permlane32_swap swaps the upper half of its
// first operand with the lower half of its second, so with both operands
// holding x, lane l < 32 ends with (x[l], x[l+32]) and lane l >= 32 with
// (x[l-32], x[l]): the pair is {own, partner} on every lane.  Issued by hand
// on two distinct registers (the builtin, given the same value twice, is
// folded as if the swap returned its inputs).
__device__ __forceinline__ void pair_swap(float x, float &a, float &b) {
  uint32_t u = __builtin_bit_cast(uint32_t, x), w = u;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(u), "+v"(w));
  a = __builtin_bit_cast(float, u);
  b = __builtin_bit_cast(float, w);
}

__device__ __forceinline__ float pair_max(float x) {  // max with lane ^ 32
  float a, b;
  pair_swap(x, a, b);
  return max2f(a, b);
}

__device__ __forceinline__ float pair_sum(float x) {  // sum with lane ^ 32
  float a, b;
  pair_swap(x, a, b);
  return a + b;
}

}  // namespace bf16t
}  // namespace fa355
