// fa_decode.hip -- split-KV attention for decode-shaped problems on gfx950.
//
// A decode step brings a few new queries per (batch, head) to a long cache of
// keys and values; the causal mask is the one autoregressive decoding uses
// ("Mini FlashAttention", section 1), here aligned so the queries are the
// newest positions: query i of nq sees keys 0 .. nk - nq + i.  The work is a
// matrix-vector product over the cache -- every K and V byte is read once for
// a few multiply-adds -- so it is bound by HBM bandwidth, not by the matrix
// cores.  These kernels therefore use vector-ALU arithmetic and spend their
// effort on the memory stream: non-temporal 16-byte loads covering 128
// contiguous bytes of a key row per 8 lanes, the next step's loads in flight
// while a step computes, start offsets staggered between waves, and enough
// waves to keep every SIMD streaming even when batch x heads is small, which
// is what the split of the key range is for.
//
//  1. decode_split: one wave per (b, h, key range, group of up to 4 queries);
//     a workgroup is 4 such waves, with the query groups of one key range
//     adjacent so they share the cache lines they read.  Lanes 8 r .. 8 r + 7
//     hold key row r of each 8-key slot; lane c of the row holds d / 8
//     elements (16-byte vectors at elements VEC (c + 8 j)).  A score is the
//     lane's partial dot product summed over the row's 8 lanes (DPP).  Each of
//     the 8 row positions keeps its own running max, sum and output
//     accumulator over the keys it sees -- the online softmax of "Mini
//     FlashAttention", section 4, per lane group -- so no step needs an
//     exchange between rows; the 8 states are merged once at the end by the
//     same rescaling rule.
//  2. decode_merge, only when the key range was split: per output element,
//     lse = ln sum_s exp(lse_s) and O = sum_s exp(lse_s - lse) O_s, the exact
//     combination of softmax results over disjoint key sets that the lse
//     output makes possible.
//
// bf16 scores use v_dot2c_f32_bf16 (bf16 pairs, fp32 accumulate); V is
// widened to fp32 and P stays fp32.  fp32 inputs use fp32 FMAs throughout.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_decode_launch.h"

namespace fa355 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;  // 4 independent waves

// The cache is streamed once: non-temporal loads keep it from displacing
// what the caches hold (measured ~12 % faster than plain loads).
__device__ __forceinline__ u32x4_t load16(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float ninf() { return -__builtin_huge_valf(); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                            0xF, 0xF, true));
}

// Sum over the 8 lanes 8 r .. 8 r + 7 (every lane gets the total).
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: lane 7 - i of the 8, i.e. the other quad
  return x;
}

// Partial dot product of one 16-byte vector of q with one of k.  Vector
// components are copied to scalars before __builtin_bit_cast: the builtin
// applied to a component expression reads component 0.
template <bool BF16>
__device__ __forceinline__ float dot_vec(u32x4_t q, u32x4_t k, float acc) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t qw = q[w], kw = k[w];
    if constexpr (BF16)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw),
                                            __builtin_bit_cast(bf16x2_t, kw), acc, false);
    else
      acc = __builtin_fmaf(__builtin_bit_cast(float, qw), __builtin_bit_cast(float, kw), acc);
  }
  return acc;
}

template <bool BF16, int D, int NQ, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void decode_split(DecodeArgs a) {
  constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte vector
  constexpr int NV = D / (8 * VEC);  // vectors per lane per key row
  constexpr int EPL = NV * VEC;      // elements per lane
  constexpr int U = BF16 ? 2 : 1;    // 8-key slots per step (8 KB of K and V per wave at d = 128)
  constexpr int STEP = 8 * U;
  using E = typename std::conditional<BF16, uint16_t, float>::type;

  const long long task = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (task >= a.tasks) return;  // wave-uniform; no barriers below
  const int lane = threadIdx.x & 63, r = lane >> 3, c = lane & 7;
  const int qc = static_cast<int>(task % a.qchunks);
  const long long rest = task / a.qchunks;
  const int split = static_cast<int>(rest % a.splits);
  const long long bh = rest / a.splits;
  const int nq = a.nq, nk = a.nk;
  const int k_begin = split * a.chunk;
  const int k_end = min(nk, k_begin + a.chunk);
  const int q0 = qc * NQ;
  const E *kbase = static_cast<const E *>(a.k) + bh * nk * D;
  const E *vbase = static_cast<const E *>(a.v) + bh * nk * D;

  u32x4_t qv[NQ][NV];
  int last[NQ];  // last key each query sees
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    const int qi = q0 + qq;
    last[qq] = CAUSAL ? nk - nq + qi : nk - 1;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      qv[qq][j] = u32x4_t{0u, 0u, 0u, 0u};
      if (qi < nq)
        qv[qq][j] = *reinterpret_cast<const u32x4_t *>(static_cast<const E *>(a.q) +
                                                       (bh * nq + qi) * D + VEC * (c + 8 * j));
    }
  }

  // running state of this lane's row position, scores in log2 units
  float m[NQ], l[NQ], o[NQ][EPL];
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    m[qq] = ninf();
    l[qq] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[qq][e] = 0.f;
  }

  u32x4_t k0v[U][NV], v0v[U][NV], k1v[U][NV], v1v[U][NV];
  auto load = [&](u32x4_t (&kx)[U][NV], u32x4_t (&vx)[U][NV], int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = k0 + 8 * u + r;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        kx[u][j] = u32x4_t{0u, 0u, 0u, 0u};
        vx[u][j] = u32x4_t{0u, 0u, 0u, 0u};
        if (key < k_end) {
          const long long off = (long long)key * D + VEC * (c + 8 * j);
          kx[u][j] = load16(kbase + off);
          vx[u][j] = load16(vbase + off);
        }
      }
    }
  };
  auto step = [&](const u32x4_t (&kx)[U][NV], const u32x4_t (&vx)[U][NV], int k0) {
    float p[NQ][U];
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = k0 + 8 * u + r;
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) acc = dot_vec<BF16>(qv[qq][j], kx[u][j], acc);
        acc = sum8(acc);
        s[u] = (key < k_end && key <= last[qq]) ? acc * a.scale_log2 : ninf();
      }
      float mx = m[qq];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u]);
      const float mu = (mx == ninf()) ? 0.f : mx;  // no key seen yet: keep exp2 finite
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[qq][u] = __builtin_amdgcn_exp2f(s[u] - mu);
        ps += p[qq][u];
      }
      const float alpha = __builtin_amdgcn_exp2f(m[qq] - mu);
      l[qq] = l[qq] * alpha + ps;
      if (__builtin_amdgcn_ballot_w64(mx > m[qq])) {  // some row's max grew: rescale
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[qq][e] *= alpha;
      }
      m[qq] = mx;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (BF16) {
            const float lo = __builtin_bit_cast(float, vx[u][j][w] << 16);
            const float hi = __builtin_bit_cast(float, vx[u][j][w] & 0xffff0000u);
#pragma unroll
            for (int qq = 0; qq < NQ; ++qq) {
              o[qq][j * VEC + 2 * w] = __builtin_fmaf(p[qq][u], lo, o[qq][j * VEC + 2 * w]);
              o[qq][j * VEC + 2 * w + 1] = __builtin_fmaf(p[qq][u], hi, o[qq][j * VEC + 2 * w + 1]);
            }
          } else {
            const uint32_t bits = vx[u][j][w];
            const float x = __builtin_bit_cast(float, bits);
#pragma unroll
            for (int qq = 0; qq < NQ; ++qq)
              o[qq][j * VEC + w] = __builtin_fmaf(p[qq][u], x, o[qq][j * VEC + w]);
          }
        }
  };

  // Each wave starts its range at its own step and wraps around (the order
  // of the steps does not matter: every row position's state is merged
  // exactly at the end), so the waves do not all stream the same address
  // offsets of their ranges at the same time.
  if (k_begin < k_end) {  // wave-uniform
    const int nsteps = (k_end - k_begin + STEP - 1) / STEP;
    const int rot = static_cast<int>((task * 37) % nsteps);
    auto kat = [&](int i) {
      const int t = rot + i;
      return k_begin + STEP * (t >= nsteps ? t - nsteps : t);
    };
    load(k0v, v0v, kat(0));
    int i = 0;
    while (true) {
      if (i + 1 < nsteps) load(k1v, v1v, kat(i + 1));
      step(k0v, v0v, kat(i));
      if (++i >= nsteps) break;
      if (i + 1 < nsteps) load(k0v, v0v, kat(i + 1));
      step(k1v, v1v, kat(i));
      if (++i >= nsteps) break;
    }
  }

  // merge the 8 row positions (lanes c, c + 8, ..., c + 56) and store
  const long long rows = a.bh * nq;
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    float M = m[qq];
    M = fmaxf(M, __shfl_xor(M, 8));
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float w = __builtin_amdgcn_exp2f(m[qq] - ((M == ninf()) ? 0.f : M));
    float L = l[qq] * w;
    L += __shfl_xor(L, 8);
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = o[qq][e] * w;
      x += __shfl_xor(x, 8);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      o[qq][e] = x;
    }
    const int qi = q0 + qq;
    if (r != qq || qi >= nq) continue;  // row position qq stores query qq
    const long long row = bh * nq + qi;
    const float lse = (L > 0.f) ? (M + __log2f(L)) * kLn2 : ninf();
    if (a.splits == 1) {
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      E *orow = static_cast<E *>(a.o) + row * D;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        if constexpr (BF16) {
          bf16x8_t x;
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = (__bf16)(o[qq][j * VEC + t] * inv);
          *reinterpret_cast<bf16x8_t *>(orow + VEC * (c + 8 * j)) = x;
        } else {
          *reinterpret_cast<f32x4_t *>(orow + VEC * (c + 8 * j)) =
              f32x4_t{o[qq][j * VEC] * inv, o[qq][j * VEC + 1] * inv, o[qq][j * VEC + 2] * inv,
                      o[qq][j * VEC + 3] * inv};
        }
      }
      if (c == 0 && a.lse != nullptr) a.lse[row] = lse;
    } else {
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      const long long prow = (long long)split * rows + row;
      float *po = a.part_o + prow * D;
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int t = 0; t < VEC; t += 4)
          *reinterpret_cast<f32x4_t *>(po + VEC * (c + 8 * j) + t) =
              f32x4_t{o[qq][j * VEC + t] * inv, o[qq][j * VEC + t + 1] * inv,
                      o[qq][j * VEC + t + 2] * inv, o[qq][j * VEC + t + 3] * inv};
      if (c == 0) a.part_lse[prow] = lse;
    }
  }
}

// One thread per output element: combine the key ranges' normalised
// partial outputs by their lse.  The loops over the ranges issue 8
// independent loads at a time, since with few rows (one long sequence) a
// thread walks many ranges and would otherwise wait on each load in turn.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void decode_merge(DecodeArgs a) {
  using E = typename std::conditional<BF16, __bf16, float>::type;
  constexpr int G = 8;
  const long long rows = a.bh * a.nq;
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = idx / D;
  const int e = static_cast<int>(idx % D);
  if (row >= rows) return;
  const int ns = a.splits;
  const float *pl = a.part_lse + row;      // stride rows
  const float *po = a.part_o + row * D + e;  // stride rows * D
  float M = ninf();
  int s = 0;
  for (; s + G <= ns; s += G) {
    float x[G];
#pragma unroll
    for (int t = 0; t < G; ++t) x[t] = pl[(s + t) * rows];
#pragma unroll
    for (int t = 0; t < G; ++t) M = fmaxf(M, x[t]);
  }
  for (; s < ns; ++s) M = fmaxf(M, pl[s * rows]);
  float out = 0.f, lse = ninf();
  if (M != ninf()) {  // some key range saw a key
    float L = 0.f, acc = 0.f;
    s = 0;
    for (; s + G <= ns; s += G) {
      float x[G], y[G];
#pragma unroll
      for (int t = 0; t < G; ++t) {
        x[t] = pl[(s + t) * rows];
        y[t] = po[(s + t) * rows * D];
      }
#pragma unroll
      for (int t = 0; t < G; ++t) {
        const float w = __expf(x[t] - M);  // exp(-inf) = 0
        L += w;
        acc = __builtin_fmaf(w, y[t], acc);
      }
    }
    for (; s < ns; ++s) {
      const float w = __expf(pl[s * rows] - M);
      L += w;
      acc = __builtin_fmaf(w, po[s * rows * D], acc);
    }
    out = acc / L;
    lse = M + __logf(L);
  }
  static_cast<E *>(a.o)[row * D + e] = (E)out;
  if (e == 0 && a.lse != nullptr) a.lse[row] = lse;
}

template <bool BF16, int D, bool CAUSAL>
hipError_t run(const DecodeArgs &a, hipStream_t st) {
  const long long blocks = (a.tasks + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks <= 0 || blocks > 0x7fffffffll) return hipErrorInvalidValue;
  switch (decode_queries_per_wave(a.nq)) {
    case 1:
      hipLaunchKernelGGL((decode_split<BF16, D, 1, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads),
                         0, st, a);
      break;
    case 2:
      hipLaunchKernelGGL((decode_split<BF16, D, 2, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads),
                         0, st, a);
      break;
    default:
      hipLaunchKernelGGL((decode_split<BF16, D, 4, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads),
                         0, st, a);
      break;
  }
  if (a.splits > 1) {
    const long long mblocks = (a.bh * a.nq * D + kThreads - 1) / kThreads;
    if (mblocks > 0x7fffffffll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_merge<BF16, D>), dim3((unsigned)mblocks), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t run_c(const DecodeArgs &a, bool causal, hipStream_t st) {
  return causal ? run<BF16, D, true>(a, st) : run<BF16, D, false>(a, st);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int dtype, int d, bool causal, hipStream_t stream) {
  if (a.tasks <= 0 || a.splits <= 0 || a.chunk <= 0 || a.qchunks <= 0) return hipErrorInvalidValue;
  if (a.splits > 1 && (a.part_o == nullptr || a.part_lse == nullptr)) return hipErrorInvalidValue;
  const bool bf16 = dtype == 1;
  if (d == 64) return bf16 ? run_c<true, 64>(a, causal, stream) : run_c<false, 64>(a, causal, stream);
  if (d == 128)
    return bf16 ? run_c<true, 128>(a, causal, stream) : run_c<false, 128>(a, causal, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa355
