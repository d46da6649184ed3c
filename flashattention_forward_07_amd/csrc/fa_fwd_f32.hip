// fa_fwd_f32.hip -- attention forward for fp32 inputs on gfx950.
//
// fp32 keeps every operand in fp32 (v_mfma_f32_32x32x2_f32, P not rounded),
// so it has its own operand plumbing; it serves small fp32 problems and is
// not tuned for throughput.  Structure: a workgroup of 4 wave64s owns 128
// query rows (32 per wave, resident in registers); K/V tiles of 32 keys are
// staged global -> registers -> LDS (double buffered, one barrier per tile).
// Each wave computes the transposed score block S^T = K . Q^T, so an output
// lane holds one query and 16 keys (keys 8*(r/4) + 4*(lane/32) + r%4 for
// accumulator register r): the row max is in-register plus one exchange
// with lane ^ 32 and the rescale factor is a per-lane scalar.  The same
// registers are the B operand of O^T += V^T . P^T with the contraction index
// relabelled to the keys the lane holds (lane l holds B[l / 32][l % 32] and
// A[l % 32][l / 32] for this instruction), so V is read row-major from LDS.
//
// The method is the resident-query flash loop ("Mini FlashAttention",
// section 4; grasp.study, "The Complete Kernel: Initialization, Loop, and
// Finalization"): m = -inf, l = 0, O = 0; per tile m_new = max(m, rowmax S),
// alpha = exp(m - m_new), P = exp(S - m_new), l = alpha l + rowsum P,
// O = alpha O + P V; O / l at the end.  Keys past the sequence end and, when
// causal, keys after the query score -inf; a -inf running max is replaced by
// 0 before use (the ghost-row guard of the same section 4).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.h"
#include "fa_fwd_launch.h"

namespace fa355 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kBlockM = 32 * kWaves;
constexpr int kBN = 32;

template <int D>
struct F32Tile {
  static constexpr int KSTR = D + 4;  // LDS row stride (floats)
  static constexpr int K_ELEMS = kBN * KSTR;
  static constexpr int STAGE_BYTES = 2 * kBN * KSTR * 4;
  static constexpr int CHUNKS = kBN * D / 4 / kThreads;  // 16-byte chunks per thread, per tensor
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads) void fa_fwd_f32_kernel(const FwdArgs a) {
  using C = F32Tile<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const TileCoords tc = tile_coords<VARLEN>(a, kBlockM);
  const int n = tc.n, m0 = tc.m0;
  if (m0 >= n) return;  // uniform over the workgroup, before any barrier

  const float *qb = reinterpret_cast<const float *>(a.q) + tc.base;
  const float *kb = reinterpret_cast<const float *>(a.k) + tc.base;
  const float *vb = reinterpret_cast<const float *>(a.v) + tc.base;
  const long long rs = a.row_stride;

  const int n_kv = CAUSAL ? (n < m0 + kBlockM ? n : m0 + kBlockM) : n;
  const int nt = (n_kv + kBN - 1) / kBN;
  const int qw0 = m0 + 32 * wv;
  const int qrow = qw0 + l32;
  const bool wave_live = qw0 < n;

  // resident Q^T as the B operand: lane holds Q[qrow][2t + h]
  float q[D / 2];
  {
    const float *p = qb + (long long)qrow * rs + h;
#pragma unroll
    for (int t = 0; t < D / 2; ++t) q[t] = qrow < n ? p[2 * t] : 0.f;
  }
  float m_run = neg_inf();
  float l_run = 0.f;
  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
  const float sl2 = a.scale_log2;

  u32x4_t rk[C::CHUNKS], rv[C::CHUNKS];
  auto gload = [&](int key0) {
#pragma unroll
    for (int i = 0; i < C::CHUNKS; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 4), col = (c % (D / 4)) * 4;
      const int key = key0 + row;
      u32x4_t x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (key < n) {
        x = *reinterpret_cast<const u32x4_t *>(kb + (long long)key * rs + col);
        y = *reinterpret_cast<const u32x4_t *>(vb + (long long)key * rs + col);
      }
      rk[i] = x;
      rv[i] = y;
    }
  };
  auto lstore = [&](char *stage) {
    float *lk = reinterpret_cast<float *>(stage);
    float *lv = lk + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::CHUNKS; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 4), col = (c % (D / 4)) * 4;
      *reinterpret_cast<u32x4_t *>(lk + row * C::KSTR + col) = rk[i];
      *reinterpret_cast<u32x4_t *>(lv + row * C::KSTR + col) = rv[i];
    }
  };

  gload(0);
  lstore(smem);
  for (int kt = 0; kt < nt; ++kt) {
    const bool more = kt + 1 < nt;
    if (more) gload((kt + 1) * kBN);
    __syncthreads();
    const char *stage = smem + (kt & 1) * C::STAGE_BYTES;
    const int key0 = kt * kBN;
    if (wave_live && (!CAUSAL || key0 <= qw0 + 31)) {
      // S^T = K . Q^T
      f32x16_t s = {};
      {
        const float *kr = reinterpret_cast<const float *>(stage) + l32 * C::KSTR + h;
#pragma unroll
        for (int t = 0; t < D / 2; ++t)
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[2 * t], q[t], s, 0, 0, 0);
      }
      if ((key0 + kBN > n) || (CAUSAL && key0 + kBN - 1 > qw0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + block_key(r, h);
          if (!(key < n && (!CAUSAL || key <= qrow))) s[r] = neg_inf();
        }
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_ref = (m_new == neg_inf()) ? 0.f : m_new;  // ghost-row guard
      const float alpha = exp2_fast((m_run - m_ref) * sl2);
      const float mb = m_ref * sl2;
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(__builtin_fmaf(s[r], sl2, -mb));
        s[r] = p;
        ps += p;
      }
      l_run = l_run * alpha + ps;
      m_run = m_new;
      // O^T = alpha O^T + V^T . P^T
      const float *lv = reinterpret_cast<const float *>(stage) + C::K_ELEMS;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        o[db] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float av = lv[block_key(r, h) * C::KSTR + 32 * db + l32];
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, s[r], o[db], 0, 0, 0);
        }
      }
    }
    if (more) lstore(smem + ((kt + 1) & 1) * C::STAGE_BYTES);
  }

  // finalise: O / l, lse = scale * m + ln l
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < n) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float *orow = reinterpret_cast<float *>(a.o) + tc.base + (long long)qrow * rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t x = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                     o[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4_t *>(orow + 32 * db + 8 * g + 4 * h) = x;
      }
    if (a.lse != nullptr && h == 0) {
      const float m_fin = (m_run == neg_inf()) ? 0.f : m_run;
      a.lse[tc.lbase + (long long)qrow * a.lse_row_stride] =
          l_tot > 0.f ? m_fin * a.scale + __logf(l_tot) : neg_inf();
    }
  }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL, VARLEN>), dim3(a.grid), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs &a, bool causal, bool varlen, hipStream_t stream) {
  if (causal)
    return varlen ? launch<D, true, true>(a, stream) : launch<D, true, false>(a, stream);
  return varlen ? launch<D, false, true>(a, stream) : launch<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_f32(FwdArgs a, int d, bool causal, bool varlen, hipStream_t stream) {
  a.n_qtiles = (a.max_len + kBlockM - 1) / kBlockM;
  const long long grid = (long long)a.batch * a.H * a.n_qtiles;
  if (grid > 0x7fffffffll || grid <= 0) return hipErrorInvalidValue;
  a.grid = (int)grid;
  if (d == 64) return launch_d<64>(a, causal, varlen, stream);
  if (d == 128) return launch_d<128>(a, causal, varlen, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa355
