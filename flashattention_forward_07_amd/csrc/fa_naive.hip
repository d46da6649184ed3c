// fa_naive.hip -- the unfused three-step attention forward on gfx950.
//
// The standard method the pages start from, before fusion (wpnews, "How
// Did I Write My First FlashAttention Kernel in CUDA?", the three passes of
// softmax; "Mini FlashAttention", section 2): per (batch, head)
//   1. S = scale Q K^T, written to a caller-provided N x N fp32 workspace;
//   2. each row of S: its max and sum of exp (one pass, the sum rebased as
//      the max grows), then P = exp(S - max) / sum written back over the
//      row in the input dtype (bf16 P takes the first half of the row's
//      bytes), and lse = max + ln(sum);
//   3. O = P V.
// The N x N matrix goes through HBM twice, which is what the fused kernel
// avoids.  Causal: key j > query i is masked; score tiles entirely above
// the diagonal are not computed and P.V stops at each tile's diagonal, but
// every allowed score still makes the round trip.
//
// bf16 uses v_mfma_f32_32x32x16_bf16 for both products (fp32 accumulate);
// fp32 uses plain FMA loops (it serves the small fp32 workloads).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.h"
#include "fa_naive_launch.h"

namespace fa355 {
namespace {

constexpr int kNT = 256;  // threads per workgroup (4 waves)

// ---- 1. scores (bf16) ------------------------------------------------------
// Workgroup: 128 queries x 128 keys of one (b, h); wave w owns queries
// 32 w .. 32 w + 31 and computes S = Q K^T in four 32-key blocks (lane l
// holds key l % 32 and queries 8 (r / 4) + 4 (l / 32) + r % 4 of a block in
// register r, so each store writes 128 contiguous bytes of a row per
// half-wave).  Operands come straight from global memory (L2): the K rows
// and the wave's resident Q rows are 16-byte reads.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNT) void scores_bf16(NaiveArgs a) {
  const int bh = blockIdx.z;
  const int q0 = blockIdx.y * 128, k0 = blockIdx.x * 128;
  if (CAUSAL && k0 > q0 + 127) return;  // tile entirely above the diagonal
  const int n = a.n;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q) + (long long)bh * n * D;
  const uint16_t *kb = reinterpret_cast<const uint16_t *>(a.k) + (long long)bh * n * D;
  float *sb = a.s + (long long)bh * n * a.ld;
  const int qw = q0 + 32 * wv;  // the wave's first query
  const int qi = qw + l32;      // query row this lane reads for the A operand
  bf16x8_t qr[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (qi < n) x = *reinterpret_cast<const u32x4_t *>(qb + (long long)qi * D + 16 * c + 8 * h);
    qr[c] = __builtin_bit_cast(bf16x8_t, x);
  }
  // K rows of block kb32 + 1 are loaded while block kb32's products run
  u32x4_t kx[D / 16];
  auto load_k = [&](int kb32) {
    const int key = k0 + 32 * kb32 + l32;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      kx[c] = u32x4_t{0u, 0u, 0u, 0u};
      if (key < n) kx[c] = *reinterpret_cast<const u32x4_t *>(kb + (long long)key * D + 16 * c + 8 * h);
    }
  };
  load_k(0);
#pragma unroll
  for (int kb32 = 0; kb32 < 4; ++kb32) {
    const int key = k0 + 32 * kb32 + l32;  // key row this lane read, and its output column
    u32x4_t kc[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) kc[c] = kx[c];
    if (kb32 + 1 < 4) load_k(kb32 + 1);
    f32x16_t acc = {};
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qr[c], __builtin_bit_cast(bf16x8_t, kc[c]), acc,
                                                    0, 0, 0);
    if (key < n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = qw + 8 * (r / 4) + 4 * h + r % 4;
        if (qrow < n)
          sb[(long long)qrow * a.ld + key] = (CAUSAL && key > qrow) ? neg_inf() : acc[r] * a.scale;
      }
    }
  }
}

// ---- 1. scores (fp32) ------------------------------------------------------
// One thread per score, 16 x 16 threads per 16 x 16 tile.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNT) void scores_f32(NaiveArgs a) {
  const int bh = blockIdx.z, n = a.n;
  const int i = blockIdx.y * 16 + (threadIdx.x >> 4), j = blockIdx.x * 16 + (threadIdx.x & 15);
  if (i >= n || j >= n) return;
  float *row = a.s + (long long)bh * n * a.ld + (long long)i * a.ld;
  if (CAUSAL && j > i) {
    row[j] = neg_inf();
    return;
  }
  const float *qr = reinterpret_cast<const float *>(a.q) + ((long long)bh * n + i) * D;
  const float *kr = reinterpret_cast<const float *>(a.k) + ((long long)bh * n + j) * D;
  float acc = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; ++c) acc = __builtin_fmaf(qr[c], kr[c], acc);
  row[j] = acc * a.scale;
}

// ---- 2. row softmax (both dtypes) ------------------------------------------
// One wave per row, two passes over the allowed keys: pass 1 keeps a running
// max and a sum of exp rebased to it (each lane over its own 4-key chunks,
// then merged across the wave); pass 2 writes P = exp(s - m) / l in the
// input dtype from the start of the row, with zeros after the allowed keys up
// to the last key P.V reads (the end of the causal diagonal's 64-key block,
// or N; bf16 rounds that up to the 8-key chunk P.V loads).  Pass 2 reads a
// chunk of 64 lanes x 4 scores before it writes that chunk's P, and P bytes
// never reach scores not yet read (2 bytes per bf16 P sit below 4 bytes per
// score).  Rows start 16-byte aligned (ld % 4 == 0), so full chunks are
// single 16-byte loads.
__device__ __forceinline__ void load4(const float *s, int j, int len, float (&x)[4]) {
  if (j + 3 < len) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t *>(s + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (j + e < len) ? s[j + e] : neg_inf();
  }
}

template <bool BF16, bool CAUSAL>
__global__ __launch_bounds__(kNT) void softmax_rows(NaiveArgs a) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = a.n;
  if (row >= (long long)a.bh * n) return;
  const int lane = threadIdx.x & 63;
  const int i = static_cast<int>(row % n);
  const int len = CAUSAL ? i + 1 : n;  // allowed keys
  // P.V reads keys up to the end of the diagonal's 64-key block
  int ext = CAUSAL ? ((i / 64 + 1) * 64 < n ? (i / 64 + 1) * 64 : n) : n;
  if (BF16) ext = (ext + 7) & ~7;  // <= 2 ld: inside the row's bytes
  float *s = a.s + row * a.ld;
  float m = neg_inf(), l = 0.f;
  for (int j = 4 * lane; j < len; j += 256) {
    float x[4];
    load4(s, j, len, x);
    const float mn = fmaxf(m, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));  // finite: j < len
    l = l * __expf(m - mn) + (__expf(x[0] - mn) + __expf(x[1] - mn)) +
        (__expf(x[2] - mn) + __expf(x[3] - mn));
    m = mn;
  }
  float mw = m;
  for (int off = 32; off > 0; off >>= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
  l = (l > 0.f) ? l * __expf(m - mw) : 0.f;  // lanes without keys hold m = -inf, l = 0
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  m = mw;
  const float inv = 1.f / l;
  for (int j0 = 0; j0 < ext; j0 += 256) {
    const int j = j0 + 4 * lane;
    float x[4], p[4];
    load4(s, j, len, x);  // keys past len read as -inf and are never loaded
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = (j + e < len) ? __expf(x[e] - m) * inv : 0.f;
    __builtin_amdgcn_wave_barrier();  // the whole chunk is read before any of it is written
    if constexpr (BF16) {
      uint16_t *pr = reinterpret_cast<uint16_t *>(s);
      if (j + 3 < ext) {  // ext % 8 == 0 here, so this is every chunk below ext
        const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)p[0]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[1]) << 16);
        const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)p[2]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)p[3]) << 16);
        *reinterpret_cast<u32x2_t *>(pr + j) = u32x2_t{lo, hi};  // 8-byte aligned: j % 4 == 0
      }
    } else {
      if (j + 3 < ext) {
        *reinterpret_cast<f32x4_t *>(s + j) = f32x4_t{p[0], p[1], p[2], p[3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < ext) s[j + e] = p[e];
      }
    }
  }
  if (a.lse != nullptr && lane == 0) a.lse[row] = m + __logf(l);
}

// ---- 3. O = P V (bf16) -----------------------------------------------------
// Workgroup: 128 queries of one (b, h), wave w owns 32 of them and computes
// O^T = V^T P^T in 32-column blocks of d.  Key tiles of 64 rows of V are
// staged in LDS (rows padded by 32 bytes, so the transposing reads are free
// of bank conflicts) and read as the A operand with ds_read_b64_tr_b16; the
// B operand is 8 consecutive P values of the lane's query row (16 bytes).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNT) void pv_bf16(NaiveArgs a) {
  constexpr int RS = D + 16;  // LDS row stride in elements
  __shared__ __attribute__((aligned(16))) uint16_t vt[64 * RS];
  const int bh = blockIdx.y, q0 = blockIdx.x * 128, n = a.n;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int qi = q0 + 32 * wv + l32;
  const uint16_t *vb = reinterpret_cast<const uint16_t *>(a.v) + (long long)bh * n * D;
  // P row of this lane's query: bf16, row stride 2 ld elements (it sits over
  // the fp32 scores)
  const uint16_t *pr = reinterpret_cast<const uint16_t *>(a.s + (long long)bh * n * a.ld) +
                       (long long)(qi < n ? qi : n - 1) * 2 * a.ld;
  const int n_keys = CAUSAL ? ((q0 + 127) < n - 1 ? q0 + 128 : n) : n;
  const int T = (n_keys + 63) / 64;
  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
  // transposing-read address: 16-lane group g = lane / 16 covers d columns
  // 16 (g % 2) .. +15 of the 32-column block and keys 8 (g / 2) .. +7 of a
  // 16-key step; lane j of the group addresses key row j / 4 (+4 for the
  // second read) at columns 4 (j % 4) .. +3
  const int g = lane >> 4, j = lane & 15;
  const uint32_t vbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS uint16_t *)vt));
  const uint32_t vaddr = vbase + 2u * ((8 * (g >> 1) + (j >> 2)) * RS + 16 * (g & 1) + 4 * (j & 3));
  const int wave_keys = CAUSAL ? (q0 + 32 * wv + 32 < n ? q0 + 32 * wv + 32 : n) : n;
  // the next tile's V chunks and P vectors are loaded into registers while
  // this tile's products run
  constexpr int NV = 64 * D / 8 / kNT;  // 16-byte V chunks per thread per tile
  u32x4_t vx[NV], pn[4];
  auto load_tile = [&](int t) {
    const int key0 = 64 * t;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int c = threadIdx.x + u * kNT;
      const int r = c / (D / 8), col = 8 * (c % (D / 8));
      vx[u] = u32x4_t{0u, 0u, 0u, 0u};  // rows past n read as zeros
      if (key0 + r < n) vx[u] = *reinterpret_cast<const u32x4_t *>(vb + (long long)(key0 + r) * D + col);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = key0 + 16 * ks + 8 * h;
      pn[ks] = u32x4_t{0u, 0u, 0u, 0u};
      if (key0 < wave_keys && kk < n) pn[ks] = *reinterpret_cast<const u32x4_t *>(pr + kk);
    }
  };
  load_tile(0);
  for (int t = 0; t < T; ++t) {
    const int key0 = 64 * t;
    __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int c = threadIdx.x + u * kNT;
      *reinterpret_cast<u32x4_t *>(vt + (c / (D / 8)) * RS + 8 * (c % (D / 8))) = vx[u];
    }
    u32x4_t pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pb[ks] = pn[ks];
    __syncthreads();
    if (t + 1 < T) load_tile(t + 1);
    if (key0 >= wave_keys) continue;  // wave-uniform; P is zero there anyway
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {  // 16-key steps
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint32_t ad = vaddr + 2u * (16 * ks * RS + 32 * db);
        u32x2_t lo, hi;
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(ad));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(ad), "i"(2 * 4 * RS));
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(lo), "+v"(hi));
        const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                        __builtin_bit_cast(bf16x8_t, pb[ks]), o[db],
                                                        0, 0, 0);
      }
    }
  }
  if (qi < n) {
    uint16_t *orow = reinterpret_cast<uint16_t *>(a.o) + ((long long)bh * n + qi) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const bf16x4_t x = {(__bf16)o[db][4 * gq], (__bf16)o[db][4 * gq + 1],
                            (__bf16)o[db][4 * gq + 2], (__bf16)o[db][4 * gq + 3]};
        *reinterpret_cast<bf16x4_t *>(orow + 32 * db + 8 * gq + 4 * h) = x;
      }
  }
}

// ---- 3. O = P V (fp32) -----------------------------------------------------
// One thread per output element.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNT) void pv_f32(NaiveArgs a) {
  const int bh = blockIdx.y, n = a.n;
  const long long idx = (long long)blockIdx.x * kNT + threadIdx.x;
  if (idx >= (long long)n * D) return;
  const int i = static_cast<int>(idx / D), c = static_cast<int>(idx % D);
  const float *p = a.s + (long long)bh * n * a.ld + (long long)i * a.ld;
  const float *v = reinterpret_cast<const float *>(a.v) + (long long)bh * n * D + c;
  const int len = CAUSAL ? i + 1 : n;
  float acc = 0.f;
  for (int j = 0; j < len; ++j) acc = __builtin_fmaf(p[j], v[(long long)j * D], acc);
  reinterpret_cast<float *>(a.o)[((long long)bh * n + i) * D + c] = acc;
}

template <int D, bool CAUSAL>
hipError_t run(const NaiveArgs &a, bool bf16, hipStream_t st) {
  const int n = a.n;
  const long long rows = (long long)a.bh * n;
  if (bf16) {
    const dim3 g1((n + 127) / 128, (n + 127) / 128, a.bh);
    hipLaunchKernelGGL((scores_bf16<D, CAUSAL>), g1, dim3(kNT), 0, st, a);
    hipLaunchKernelGGL((softmax_rows<true, CAUSAL>), dim3((unsigned)((rows + 3) / 4)), dim3(kNT),
                       0, st, a);
    hipLaunchKernelGGL((pv_bf16<D, CAUSAL>), dim3((n + 127) / 128, a.bh), dim3(kNT), 0, st, a);
  } else {
    const dim3 g1((n + 15) / 16, (n + 15) / 16, a.bh);
    hipLaunchKernelGGL((scores_f32<D, CAUSAL>), g1, dim3(kNT), 0, st, a);
    hipLaunchKernelGGL((softmax_rows<false, CAUSAL>), dim3((unsigned)((rows + 3) / 4)), dim3(kNT),
                       0, st, a);
    hipLaunchKernelGGL((pv_f32<D, CAUSAL>), dim3((unsigned)(((long long)n * D + kNT - 1) / kNT), a.bh),
                       dim3(kNT), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_naive(const NaiveArgs &a, int dtype, int d, bool causal, hipStream_t stream) {
  const bool bf16 = dtype == 1;
  if (a.n <= 0 || a.bh <= 0) return hipErrorInvalidValue;
  if ((long long)(a.n + 127) / 128 > 65535 || a.bh > 65535) return hipErrorInvalidValue;
  if (d == 64) return causal ? run<64, true>(a, bf16, stream) : run<64, false>(a, bf16, stream);
  if (d == 128) return causal ? run<128, true>(a, bf16, stream) : run<128, false>(a, bf16, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa355
