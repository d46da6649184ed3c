// fa_fwd_ksplit.hip -- attention forward for bf16 inputs at d = 64 and 128
// on gfx950 (MI355X), for problems too small to fill the GPU with query
// tiles: a handful of heads at a sequence length of a few thousand at most.
//
// There the time of a launch is the serial key loop of its heaviest query
// tile, not throughput.  So each workgroup takes only 32 query rows, and
// its W waves (eight at d = 64, two per SIMD; four at d = 128) split the
// key range of those rows among them: wave w streams 32-key chunks w,
// w + W, w + 2W, ... through a two-stage LDS ring of its own, keeps a
// partial softmax state for all 32 rows, and needs no barrier until the
// end.  Then the W partial states are merged
// through LDS, each term weighted by 2^(its reference - the largest), which
// is the exact combination of partial softmax sums, and O / l is written.
//
// Per chunk, one wave runs the steps of
// the resident-query loop of "Mini FlashAttention", section 4: S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 (one query per lane, 16 keys of each 32-key block
// per lane half), the causal and sequence-end mask (section 1), the chunk's
// row max against the running one, the rescale of O and l by
// exp2(old reference - new) and the weights exp2(s - reference), then
// O^T += V^T P^T with P rounded to bf16.  The reference is the running row
// max itself, replaced by 0 while a row has seen no key (the ghost-row guard
// of section 4).  O is divided by the sum of the bf16-rounded weights that
// the P.V products used; lse takes the fp32 sum.
//
// LDS layout and staging follow the streaming kernels: K and V rows
// row-major with XOR-swizzled 16-byte chunks (Bf16Tile), filled by direct
// global->LDS loads.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_bf16_tile.h"
#include "fa_common.h"
#include "fa_fwd_launch.h"

namespace fa355 {
namespace {

using namespace bf16t;

constexpr int kKsRows = 32;                   // query rows per workgroup

template <int D>
struct KsShape {
  static constexpr int W = D == 64 ? 8 : 4;       // waves: two per SIMD at d = 64
  static constexpr int THREADS = W * kWave;
  static constexpr int BN = 32;                   // keys per chunk
  using Tile = Bf16Tile<D, BN>;
  static constexpr int RING = 2 * Tile::STAGE;    // two stages per wave: 16 or 32 KB
  static constexpr int DPW = Tile::TILE / 1024;  // staging loads per tensor and chunk
  static constexpr int NV = (D / 32) * 4 + 1;       // float4 slots per lane of a partial state
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(KsShape<D>::THREADS) void fa_fwd_ksplit(const FwdArgs a) {
  using S = KsShape<D>;
  constexpr int kKsWaves = S::W;
  using C = typename S::Tile;
  constexpr int BN = S::BN;
  constexpr int KB = BN / 32;       // 32-key blocks per chunk
  constexpr int KC = D / 16;        // 16-wide d chunks (S products per block)
  constexpr int VC = BN / 16;       // 16-key steps (P.V products per d block)
  constexpr int DPW = S::DPW;
  static_assert(DPW * 1024 == C::TILE, "staging split");
  // s_waitcnt immediate for vmcnt(2 DPW) (low four bits, then bits 14-15),
  // lgkmcnt and expcnt at their maxima
  constexpr int kVmcntNext = ((2 * DPW) & 15) | (((2 * DPW) >> 4) << 14) | 0x0F70;
  static_assert(kKsWaves * S::NV * kWave * 16 <= kKsWaves * S::RING, "merge area");
  __shared__ __attribute__((aligned(1024))) char smem[kKsWaves * S::RING];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const TileCoords tc = tile_coords<VARLEN>(a, kKsRows);
  const int n = tc.n, m0 = tc.m0;
  if (m0 >= n) return;  // uniform over the workgroup, before any barrier

  const uint16_t *qg = reinterpret_cast<const uint16_t *>(a.q) + tc.base;
  const uint16_t *kg = reinterpret_cast<const uint16_t *>(a.k) + tc.base;
  const uint16_t *vg = reinterpret_cast<const uint16_t *>(a.v) + tc.base;
  const long long rs = a.row_stride;
  const uint32_t rsb = static_cast<uint32_t>(rs) * 2u;  // bytes per key row

  const int qrow = m0 + l32;  // this lane's query
  // keys the workgroup needs: all, or (causal) up to its last query
  const int n_kv = CAUSAL ? (n < m0 + kKsRows ? n : m0 + kKsRows) : n;
  const int T = (n_kv + BN - 1) / BN;                            // chunks
  const int Tw = T > w ? (T - 1 - w) / kKsWaves + 1 : 0;         // chunks of this wave

  // ---- resident Q^T (B operand): lane holds Q[qrow][16c + 8h .. +7] ---------
  bf16x8_t q[KC];
  {
    // rows past the end load row n - 1 and are zeroed (never stored)
    const uint16_t *p = qg + (long long)(qrow < n ? qrow : n - 1) * rs + 8 * h;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4_t x = *reinterpret_cast<const u32x4_t *>(p + 16 * c);
      if (qrow >= n) x = u32x4_t{0u, 0u, 0u, 0u};
      q[c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // ---- staging: global -> LDS, this wave's ring only -------------------------
  // Load j of a tensor fills LDS slots p = 64 j + lane (row p / CPR, slot
  // p % CPR) of the chunk; the lane fetches the logical 16-byte chunk the
  // swizzle places in its slot: a chunk base in scalar registers plus a fixed
  // byte offset per lane.  In the workgroup's last chunk, rows past its last
  // key load that key's row again (finite data; their scores are masked).
  int d_row[DPW];
  uint32_t c_k[DPW], c_v[DPW];  // byte offset of the slot's column within a row
  uint32_t o_k[DPW], o_v[DPW];  // ... and of its source within a whole chunk
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int p = j * kWave + lane;
    const int row = p / C::CPR, slot = p % C::CPR;
    d_row[j] = row;
    c_k[j] = 16u * (slot ^ C::swz_k(row));
    c_v[j] = 16u * (slot ^ C::swz_v(row));
    o_k[j] = c_k[j] + row * rsb;
    o_v[j] = c_v[j] + row * rsb;
  }
  char *ring = smem + w * S::RING;
  // global chunk g (its keys g BN ..) into stage st of this wave's ring
  auto dma_chunk = [&](int g_, int st) {
    const int g = __builtin_amdgcn_readfirstlane(g_);
    const int key0 = g * BN;
    const char *kt = reinterpret_cast<const char *>(kg + (long long)key0 * rs);
    const char *vt = reinterpret_cast<const char *>(vg + (long long)key0 * rs);
    char *dst = ring + st * C::STAGE;
    if (key0 + BN <= n_kv) {
#pragma unroll
      for (int j = 0; j < DPW; ++j) {
        __builtin_amdgcn_global_load_lds((const FA_GLOBAL void *)(kt + o_k[j]),
                                         (FA_LDS void *)(dst + j * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const FA_GLOBAL void *)(vt + o_v[j]),
                                         (FA_LDS void *)(dst + C::TILE + j * 1024), 16, 0, 0);
      }
    } else {
      const int last = n_kv - 1 - key0;  // >= 0 for a chunk of the workgroup
#pragma unroll
      for (int j = 0; j < DPW; ++j) {
        const uint32_t rb = static_cast<uint32_t>(d_row[j] < last ? d_row[j] : last) * rsb;
        __builtin_amdgcn_global_load_lds((const FA_GLOBAL void *)(kt + (rb + c_k[j])),
                                         (FA_LDS void *)(dst + j * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const FA_GLOBAL void *)(vt + (rb + c_v[j])),
                                         (FA_LDS void *)(dst + C::TILE + j * 1024), 16, 0, 0);
      }
    }
  };

  // ---- LDS operand addresses (byte offsets within a stage) -------------------
  uint32_t kofs[KC];  // K operand (kb, c): row 32 kb + l32, logical chunk 2c + h
  {
    const int sw = C::swz_k(l32);
#pragma unroll
    for (int c = 0; c < KC; ++c) kofs[c] = l32 * C::ROWB + 16 * ((2 * c + h) ^ sw);
  }
  uint32_t vofs[D / 32];  // V^T operand (db, step): key row 16 step (+8) + 4h + e4
  {
    const int j = lane & 15, e4 = j >> 2, g = (lane >> 4) & 1;
    const int sw = C::swz_v(e4);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      vofs[db] = C::TILE + (4 * h + e4) * C::ROWB +
                 16 * ((4 * db + 2 * g + ((j & 3) >> 1)) ^ sw) + 8 * (j & 1);
  }
  const uint32_t ring_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS char *)ring));

  // ---- running state (per lane: its query, its half of each block's keys) ----
  float mref = neg_inf();  // running row max, exp2 domain (-inf: no key yet)
  float l_run = 0.f;       // this lane's partial row sum
  float lr_run = 0.f;      // the same over the bf16-rounded weights
  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
  const float sl2 = a.scale_log2;
  const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};

  // prologue: this wave's first two chunks in flight at once
  if (Tw > 0) dma_chunk(w, 0);
  if (Tw > 1) dma_chunk(w + kKsWaves, 1);

  for (int i = 0; i < Tw; ++i) {
    const int g = w + kKsWaves * i;  // global chunk index
    const int key0 = g * BN;
    const uint32_t sbase = ring_base + (i & 1) * C::STAGE;
    // this chunk's loads have landed (the next chunk's may still fly)
    if (i + 1 < Tw)
      __builtin_amdgcn_s_waitcnt(kVmcntNext);  // vmcnt(2 DPW)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // S^T = K Q^T: all K operands read at once, each product waits for its own
    u32x4_t kr[KB * KC];
    static_for<KB * KC>([&](auto I) {
      constexpr int ii = decltype(I)::value, kb = ii / KC, c = ii % KC;
      kr[ii] = lds_read_b128<kb * 32 * C::ROWB>(sbase + kofs[c]);
    });
    f32x16_t sc[KB];
    static_for<KB * KC>([&](auto I) {
      constexpr int ii = decltype(I)::value, kb = ii / KC, c = ii % KC;
      lgkm_wait<KB * KC - 1 - ii>(kr[ii]);
      sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kr[ii]), q[c],
                                                       c == 0 ? f32x16_t{} : sc[kb], 0, 0, 0);
    });
    // the V operands go out behind the score products; their latency hides
    // under the softmax
    u32x2_t vr[D / 32][VC][2];
    static_for<(D / 32) * VC>([&](auto I) {
      constexpr int ii = decltype(I)::value, db = ii / VC, c = ii % VC;
      vr[db][c][0] = lds_read_tr16<16 * c * C::ROWB>(sbase + vofs[db]);
      vr[db][c][1] = lds_read_tr16<(16 * c + 8) * C::ROWB>(sbase + vofs[db]);
    });
    constexpr int kVReads = 2 * (D / 32) * VC;
    static_assert(kVReads <= 16 && KB * KC <= 16, "outstanding LDS reads");

    // scores in the exp2 domain; keys past the end and (causal) after the
    // query are -inf
    const bool edge = (key0 + BN > n) || (CAUSAL && key0 + BN - 1 > m0);
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sc[b][r] * sl2;
        if (edge) {
          const int key = key0 + 32 * b + block_key(r, h);
          if (!(key < n && (!CAUSAL || key <= qrow))) x = neg_inf();
        }
        sc[b][r] = x;
      }
    float mx = neg_inf();
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sc[b][r]);
    mx = pair_max(mx);
    const float mnew = __builtin_fmaxf(mref, mx);
    const float ref = (mnew == neg_inf()) ? 0.f : mnew;  // ghost-row guard
    const float alpha = exp2_fast(mref - ref);             // 0 while there was no key
    mref = mnew;

    // weights: fp32 sum for lse, bf16 P and the sum of its rounded values
    bf16x8_t pb[VC];
    float ps = 0.f, psr = 0.f;
#pragma unroll
    for (int c = 0; c < VC; ++c)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = exp2_fast(sc[c >> 1][8 * (c & 1) + e] - ref);
        const float p1 = exp2_fast(sc[c >> 1][8 * (c & 1) + e + 1] - ref);
        pb[c][e] = (__bf16)p0;
        pb[c][e + 1] = (__bf16)p1;
        ps += p0 + p1;
        const bf16x2_t pr = {pb[c][e], pb[c][e + 1]};
        psr = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, psr, false);
      }
    l_run = l_run * alpha + ps;
    lr_run = lr_run * alpha + psr;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;

    // O^T += V^T P^T
    static_for<(D / 32) * VC>([&](auto I) {
      constexpr int ii = decltype(I)::value, db = ii / VC, c = ii % VC;
      lgkm_wait<kVReads - 2 * (ii + 1)>(vr[db][c][0], vr[db][c][1]);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_bf16(vr[db][c][0], vr[db][c][1]), pb[c],
                                                      o[db], 0, 0, 0);
    });
    // every read of this stage has returned: chunk i + 2 may overwrite it
    asm volatile("" ::: "memory");
    if (i + 2 < Tw) dma_chunk(g + 2 * kKsWaves, i & 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: no staging load outlives the loop

  // ---- merge the W partial states through LDS --------------------------------
  wg_barrier();  // every wave is done with its ring
  // per wave and lane: O in float4 slots (d block db, quarter j at slot
  // 4 db + j) and (max, l, rounded-weight sum) in the last slot; slot s of
  // wave v at f32x4 index (v NV + s) 64 + lane, so that every access is one
  // 16-byte read or write per lane over consecutive lanes
  f32x4_t *part = reinterpret_cast<f32x4_t *>(smem);
  constexpr int NV = S::NV;
  {
    f32x4_t *mine = part + (w * NV) * kWave + lane;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        mine[(db * 4 + j) * kWave] =
            f32x4_t{o[db][4 * j], o[db][4 * j + 1], o[db][4 * j + 2], o[db][4 * j + 3]};
    mine[(NV - 1) * kWave] = f32x4_t{mref, l_run, lr_run, 0.f};
  }
  wg_barrier();
  // wave w finishes d block w (d = 64: waves 0 and 1); wave 0 also writes lse
  if (w >= D / 32) return;
  f32x4_t sv[kKsWaves];
  float mm = neg_inf();
#pragma unroll
  for (int v = 0; v < kKsWaves; ++v) {
    sv[v] = part[(v * NV + NV - 1) * kWave + lane];
    mm = __builtin_fmaxf(mm, sv[v][0]);
  }
  f32x16_t acc = f32x16_t{};
  float l_tot = 0.f, lr_tot = 0.f;
#pragma unroll
  for (int v = 0; v < kKsWaves; ++v) {
    const float f = sv[v][0] == neg_inf() ? 0.f : exp2_fast(sv[v][0] - mm);
    const f32x4_t *pv = part + (v * NV + 4 * w) * kWave + lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4_t x = pv[j * kWave];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * j + e] += f * x[e];
    }
    l_tot += f * sv[v][1];
    lr_tot += f * sv[v][2];
  }
  l_tot = pair_sum(l_tot);
  lr_tot = pair_sum(lr_tot);
  if (qrow < n) {
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    uint16_t *orow = reinterpret_cast<uint16_t *>(a.o) + tc.base + (long long)qrow * rs;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const bf16x4_t x = {(__bf16)(acc[4 * gq] * inv), (__bf16)(acc[4 * gq + 1] * inv),
                          (__bf16)(acc[4 * gq + 2] * inv), (__bf16)(acc[4 * gq + 3] * inv)};
      *reinterpret_cast<bf16x4_t *>(orow + 32 * w + 8 * gq + 4 * h) = x;
    }
    if (w == 0 && h == 0 && a.lse != nullptr) {  // lse = ln 2 (m + log2 l)
      const float m_fin = (mm == neg_inf()) ? 0.f : mm;
      a.lse[tc.lbase + (long long)qrow * a.lse_row_stride] =
          l_tot > 0.f ? (m_fin + __log2f(l_tot)) * 0.693147180559945309f : neg_inf();
    }
  }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_ks(const FwdArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_ksplit<D, CAUSAL, VARLEN>), dim3(a.grid), dim3(KsShape<D>::THREADS), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_ks_d(const FwdArgs &a, bool causal, bool varlen, hipStream_t stream) {
  if (causal)
    return varlen ? launch_ks<D, true, true>(a, stream) : launch_ks<D, true, false>(a, stream);
  return varlen ? launch_ks<D, false, true>(a, stream) : launch_ks<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_ksplit(const FwdArgs &a, int d, bool causal, bool varlen,
                             hipStream_t stream) {
  if (d == 64) return launch_ks_d<64>(a, causal, varlen, stream);
  if (d == 128) return launch_ks_d<128>(a, causal, varlen, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa355
