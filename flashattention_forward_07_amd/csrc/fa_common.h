// fa_common.h -- device helpers shared by the forward kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_launch.h"

namespace fa355 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))
#define FA_GLOBAL __attribute__((address_space(1)))

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

// Row (key) of a 32 x 32 matrix-core output block held in accumulator
// register r by a lane of half h = lane / 32.
__device__ __forceinline__ int block_key(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Hardware workgroup id -> (head index bh, query-tile level qi), a bijection
// on [0, grid).  Workgroups are dispatched round-robin over the XCDs
// (hardware id i runs on XCD i % 8, as its (i / 8)-th workgroup there).  When
// the number of (sequence, head) pairs is a multiple of 8, head h is pinned
// to XCD h % 8, so all query tiles of a head share that XCD's L2 and its
// K/V stream.  Each XCD takes its heads in groups of G (G divides its head
// count; G <= 0 means all of them) and issues a group's tiles level by level,
// heaviest (highest query tile) first across the group's heads, which
// balances the causal triangle; a small group keeps several running
// workgroups on each head's K/V stream at once.  Otherwise the order is
// heaviest-first over all heads.
struct TileOrder {
  int bh;  // (sequence, head) pair
  int qi;  // 0 = heaviest query tile
};
__device__ __forceinline__ TileOrder tile_order(int i, int n_heads, int n_qtiles, int G) {
  TileOrder o;
  if (n_heads % kXcds == 0) {
    const int hx = n_heads / kXcds;  // heads per XCD
    const int x = i % kXcds, r = i / kXcds;
    if (G <= 0 || hx % G != 0) G = hx;
    const int grp = r / (G * n_qtiles), rr = r - grp * (G * n_qtiles);
    o.bh = x + kXcds * (grp * G + rr % G);
    o.qi = rr / G;
  } else {
    o.bh = i % n_heads;
    o.qi = i / n_heads;
  }
  return o;
}

__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// Where a workgroup's query tile lives.
struct TileCoords {
  int n;            // length of its sequence
  int m0;           // first query row of the tile
  long long base;   // element offset of (sequence, head) token 0
  long long lbase;  // lse offset of (sequence, head) token 0
};

// Workgroup -> (sequence, head, query tile) in the order of tile_order.
template <bool VARLEN>
__device__ __forceinline__ TileCoords tile_coords(const FwdArgs &a, int block_m) {
  const TileOrder to = tile_order(blockIdx.x, a.batch * a.H, a.n_qtiles, a.order_group);
  const int bh = to.bh;
  const int qt = a.n_qtiles - 1 - to.qi;
  const int s = bh / a.H;
  const int hd = bh - s * a.H;
  TileCoords c;
  if constexpr (VARLEN) {
    const int t0 = a.cu_seqlens[s];
    c.n = a.cu_seqlens[s + 1] - t0;
    c.base = (long long)t0 * a.row_stride;
    c.lbase = (long long)t0 * a.lse_row_stride;
  } else {
    c.n = a.n;
    c.base = (long long)s * a.seq_stride;
    c.lbase = (long long)s * a.lse_seq_stride;
  }
  c.base += (long long)hd * a.head_stride;
  c.lbase += (long long)hd * a.lse_head_stride;
  c.m0 = qt * block_m;
  return c;
}

}  // namespace fa355
