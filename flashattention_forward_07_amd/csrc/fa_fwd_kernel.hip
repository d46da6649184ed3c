// fa_fwd_kernel.hip -- attention forward for bf16 inputs on gfx950 (MI355X).
//
// The method is the resident-query flash loop of "Mini FlashAttention",
// section 4 (with the initialise / loop / finalise structure of the
// grasp.study lesson "The Complete Kernel: Initialization, Loop, and
// Finalization"): per query row a running max m, denominator l and fp32
// output accumulator O; each K/V tile (64 keys at d = 128, 128 at d = 64)
// gives scores S, the state is
// rescaled by exp(m_old - m_new), P = exp(S - m) is added into l and P.V into
// O, and O / l is formed once at the end.  Scores and P never leave
// registers.
//
// Workgroup: 8 wave64s, 256 query rows, 32 per wave, held in registers as
// the B operand of the matrix-core products.  The waves form two groups of
// four (waves 0-3 and 4-7); a CU runs one workgroup, so every SIMD hosts one
// wave of each group.  The groups run the same loop half a step apart and
// alternate between two phases separated by workgroup barriers:
//   M(t): S_t = K_t . Q^T  and  O^T += V_{t-1}^T . P_{t-1}^T   (matrix cores)
//   V(t): mask S_t, row max, P_t = exp2(...), l, rescale O       (VALU)
// so while one wave of a SIMD issues matrix-core work the other issues the
// softmax, and the two overlap.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, D = A.B + C, A 32x16, B
// 16x32; lane l holds A[l%32][8(l/32)..+7], B[8(l/32)..+7][l%32] and output
// rows 8(r/4) + 4(l/32) + r%4 of column l%32 in register r).  The kernel
// forms the TRANSPOSED score block S^T = K . Q^T: output column = query, so
// a lane owns one query and 16 keys of each 32-key block; the row max is 15
// in-register maxima plus one v_permlane32_swap with lane l ^ 32, and the
// rescale factor is a per-lane scalar.  Those registers, rounded to bf16,
// are the B operand of O^T += V^T . P^T after relabelling the contraction
// index: in 16-key chunk c, operand index 8(l/32) + e stands for key
// 16c + 8(e/4) + 4(l/32) + e%4, which is what lane l holds.
//
// LDS: K and V tiles stay row-major ([key][d], as in memory) in a 4-stage
// ring.  Each wave moves 1/8 of every tile with direct global->LDS loads
// (global_load_lds_dwordx4, 16 bytes per lane into consecutive LDS slots),
// issued in its softmax phase V(t) for tile t + 2 and awaited (vmcnt) at the
// end of its next matrix phase, before the barrier that precedes the first
// read: no staging registers, no LDS write instructions, and the matrix
// phase issues no memory traffic at all.  (An earlier probe measured ~100
// stall cycles per such load; those came from a compiler-inserted vmcnt(0)
// before every later LDS read the compiler could not prove disjoint.  Here
// all operand reads are inline assembly, which that pass does not track,
// and the only waits are the explicit ones.)  K operands are read with one
// ds_read_b128 per lane (the LDS serves 16 lanes of a b128 read per cycle;
// a pair of ds_read_b64 was measured to conflict two ways, because a b64
// read is served 32 lanes at a time and lanes l and l + 16 then share
// banks), V^T operands with ds_read_b64_tr_b16, which hands each lane one d
// column of four key rows (lanes 4e..4e+3 of a 16-lane group address row e,
// lane i receives element i of each row).  16-byte chunks are XOR-swizzled
// per row so that every read is free of bank conflicts: K chunk j of row r
// sits at slot j ^ sk(r), V chunk j at j ^ sv(r).
//
// Lazy rescaling: the exponent reference is a past row max, and a tile is
// first weighted against it without computing its own row max.  The tile is
// kept if no lane's weights sum above 2^32; only otherwise is the row max
// taken and the reference raised to a fixed margin above it (O and l scaled
// by exp2(old - new)).
// The result is unchanged in exact arithmetic (any reference cancels in
// O / l), the weights stay <= 2^32, far from fp32 overflow even summed over
// millions of keys, and most tiles skip both the row max and the rescale.
//
// Masking: keys at or past the sequence end score -inf (the pages fill
// padded key rows with zeros, which would give them score 0; the definition
// sums over real keys only), in causal mode key j > query i scores -inf
// ("Mini FlashAttention", section 1), tiles entirely above a wave's diagonal
// are skipped, and a -inf reference is replaced by 0 before use, the
// ghost-row guard of "Mini FlashAttention", section 4.  Query rows past the
// sequence end compute on zeros and are never stored.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_bf16_tile.h"
#include "fa_common.h"
#include "fa_fwd_launch.h"

namespace fa355 {
namespace {

// Tuning knobs (compile-time): wave priority during the matrix and softmax
// phases, and how many matrix steps ahead operands are read.
#ifndef FA_PRIO_M
#define FA_PRIO_M 3
#endif
#ifndef FA_PRIO_V
#define FA_PRIO_V 0
#endif
#ifndef FA_LOOKAHEAD
#define FA_LOOKAHEAD 4
#endif
// When the softmax rebases its exponent reference on a row max, the new
// reference sits FA_REF_MARGIN log2 units above the max, and a tile stays on
// the fast path while every lane's weights sum to at most FA_FAST_BOUND, so
// scores may grow ~80 log2 units past a rebased max before the next rebase:
// rows whose scores keep creeping up (wide score ranges) rarely pay the
// second pass.  The reference cancels in O / l and in lse; weights start at
// 2^-48, so only terms more than ~78 log2 units below the row max (relative
// weight < 2^-78) underflow, and no weight exceeds 2^32.
#ifndef FA_REF_MARGIN
#define FA_REF_MARGIN 48.f
#endif
#ifndef FA_FAST_BOUND
#define FA_FAST_BOUND 4294967296.f
#endif


constexpr int kWaves = 8;
constexpr int kThreads = kWave * kWaves;  // 512
constexpr int kBlockM = 32 * kWaves;      // 256 query rows
constexpr int kStages = 4;

using namespace bf16t;

// Keys per K/V tile: 64 at d = 128.  At d = 64 the registers also allow
// 128, which gives the matrix phase 32 products as at d = 128 and halves the
// per-key share of the per-tile costs (barriers, staging issue, loop
// control); it is taken when the longest sequence has at least
// kWideMinLen tokens, since shorter sequences would mostly compute masked
// keys of a wide tile.
constexpr int kWideMinLen = 256;

// SPLIT: the key range is split instead of the query rows.  The workgroup
// owns 128 query rows; waves w and w + 4 hold the same 32 rows, group 0
// streams the first half of the K/V tiles and group 1 the second half, each
// through an LDS ring of its own, and at the end group 1 hands its O, l and
// exponent reference to group 0 through LDS, which merges the two partial
// results (each term weighted by 2^(its reference - the larger one)) before
// the final O / l.  It halves the serial key loop of a workgroup, for
// problems whose grid would leave most compute units idle.
template <int D, int BN, bool CAUSAL, bool VARLEN, bool SPLIT = false>
__global__ __launch_bounds__(kThreads) void fa_fwd_bf16_kernel(const FwdArgs a) {
  using C = Bf16Tile<D, BN>;
  constexpr int kLds = kStages * C::STAGE;  // one ring of K/V tiles
  constexpr int kBN = C::BN;    // keys per tile
  constexpr int KB = kBN / 32;  // 32-key blocks per tile
  constexpr int kRows = SPLIT ? kBlockM / 2 : kBlockM;  // query rows of the workgroup
  constexpr int kCopyWaves = SPLIT ? kWaves / 2 : kWaves;  // waves that stage one ring
  constexpr int DPW = C::TILE / (1024 * kCopyWaves);  // staging loads per wave per tensor
  static_assert(DPW >= 1 && C::TILE % (1024 * kCopyWaves) == 0, "tile / workgroup mismatch");
  __shared__ __attribute__((aligned(1024))) char smem[SPLIT ? 2 * kLds : kLds];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int grp = wv >> 2;  // ping-pong group
  const int rw = SPLIT ? (wv & 3) : wv;  // row slot (and staging slot) of this wave
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const TileCoords tc = tile_coords<VARLEN>(a, kRows);
  const int n = tc.n, m0 = tc.m0;
  if (m0 >= n) return;  // uniform over the workgroup, before any barrier

  const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q) + tc.base;
  const uint16_t *kb = reinterpret_cast<const uint16_t *>(a.k) + tc.base;
  const uint16_t *vb = reinterpret_cast<const uint16_t *>(a.v) + tc.base;
  const long long rs = a.row_stride;

  const int n_kv = CAUSAL ? (n < m0 + kRows ? n : m0 + kRows) : n;
  const int T = (n_kv + kBN - 1) / kBN;  // K/V tiles of the workgroup
  // The loop counts steps: step t of a group is K/V tile lo + t.  Without
  // the split both groups step through all T tiles.
  const int T0 = SPLIT ? (T + 1) / 2 : T;  // steps of group 0 (the longer share)
  const int lo = (SPLIT && grp) ? T0 : 0;
  const int Tg = SPLIT ? (grp ? T - T0 : T0) : T;  // steps of this wave's group
  const int qw0 = m0 + 32 * rw;          // first query row of this wave
  const int qrow = qw0 + l32;            // this lane's query row
  // steps this wave works on (causal: no tile entirely above its diagonal)
  int Tw = 0;
  if (qw0 < n) {
    const int last = CAUSAL ? ((qw0 + 31) / kBN + 1 < T ? (qw0 + 31) / kBN + 1 : T) : T;
    if constexpr (SPLIT)
      Tw = last - lo < 0 ? 0 : (last - lo < Tg ? last - lo : Tg);
    else
      Tw = last;
  }
  const int ring = SPLIT ? grp * kLds : 0;  // this group's LDS ring

  // ---- resident Q^T (B operand): lane holds Q[qrow][16c + 8h .. +7] ---------
  bf16x8_t q[D / 16];
  {
    const uint16_t *p = qb + (long long)qrow * rs + 8 * h;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (qrow < n) x = *reinterpret_cast<const u32x4_t *>(p + 16 * c);
      q[c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // ---- K/V tile staging: global -> LDS directly -------------------------
  // A tile is 2 * TILE bytes of LDS in 16-byte slots.  Load i of wave wv
  // fills the 1 KB of slots p = (wv * DPW + i) * 64 + lane (row p / CPR,
  // slot p % CPR) of the K tile and of the V tile, one slot per lane, so each
  // lane fetches the logical chunk that the XOR swizzle places in its slot:
  // chunk (p % CPR) ^ swz(row).  Every lane of a row still reads that row's
  // 256 bytes (a permutation of its chunks).
  // Source addresses: a wave-uniform tile base (key0 rows down, in scalar
  // registers) plus a fixed 32-bit byte offset per lane; the host bounds the
  // row stride so that 64 or 128 rows stay below 2^31 bytes.
  int d_row[DPW];
  uint32_t o_k[DPW], o_v[DPW];  // byte offset of the slot's source in a whole tile
  uint32_t c_k[DPW], c_v[DPW];  // byte offset of its column within a row (ragged path)
  const uint32_t rsb = static_cast<uint32_t>(a.row_stride) * 2u;  // bytes per key row
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int p = (rw * DPW + i) * kWave + lane;
    const int row = p / C::CPR, slot = p % C::CPR;
    d_row[i] = row;
    c_k[i] = 16u * (slot ^ C::swz_k(row));
    c_v[i] = 16u * (slot ^ C::swz_v(row));
    o_k[i] = c_k[i] + row * rsb;
    o_v[i] = c_v[i] + row * rsb;
  }
  auto dma_tile = [&](int t_) {
    const int t = __builtin_amdgcn_readfirstlane(t_);
    const int key0 = (lo + t) * kBN;
    char *st = smem + ring + (t & (kStages - 1)) * C::STAGE;
    const char *kt = reinterpret_cast<const char *>(kb + (long long)key0 * rs);
    const char *vt = reinterpret_cast<const char *>(vb + (long long)key0 * rs);
    if (key0 + kBN <= n) {
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int reg = (rw * DPW + i) * 1024;
        __builtin_amdgcn_global_load_lds((const FA_GLOBAL void *)(kt + o_k[i]),
                                         (FA_LDS void *)(st + reg), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const FA_GLOBAL void *)(vt + o_v[i]),
                                         (FA_LDS void *)(st + C::TILE + reg), 16, 0, 0);
      }
    } else {
      const int last = n - 1 - key0;
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const uint32_t rb = static_cast<uint32_t>(d_row[i] < last ? d_row[i] : last) * rsb;
        const int reg = (rw * DPW + i) * 1024;
        __builtin_amdgcn_global_load_lds((const FA_GLOBAL void *)(kt + (rb + c_k[i])),
                                         (FA_LDS void *)(st + reg), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const FA_GLOBAL void *)(vt + (rb + c_v[i])),
                                         (FA_LDS void *)(st + C::TILE + reg), 16, 0, 0);
      }
    }
  };

  // ---- LDS operand addresses (byte offsets within a stage) ----------------
  // K operand (kb, c): row 32 kb + l32, logical chunk 2c + h.
  uint32_t kofs[D / 16];
  {
    const int sw = C::swz_k(l32);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) kofs[c] = l32 * C::ROWB + 16 * ((2 * c + h) ^ sw);
  }
  // V^T operand (db, c): this lane addresses key row 16c (+8) + 4h + e4 at
  // d = 32 db + 16 g + 4 (j % 4) .. +3 (j = lane % 16, e4 = j / 4, g = lane / 16 % 2).
  uint32_t vofs[D / 32];
  {
    const int j = lane & 15, e4 = j >> 2, g = (lane >> 4) & 1;
    const int sw = C::swz_v(e4);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      vofs[db] = C::TILE + (4 * h + e4) * C::ROWB +
                 16 * ((4 * db + 2 * g + ((j & 3) >> 1)) ^ sw) + 8 * (j & 1);
  }
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS char *)smem));

  // ---- running state ------------------------------------------------------
  float mbl = neg_inf();    // exponent reference, exp2 domain
  float l_run = 0.f;        // this lane's partial row sum (its half of the keys)
  float lr_run = 0.f;       // the same over the bf16-rounded weights
  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
  f32x16_t sc[KB];
  bf16x8_t pb[kBN / 16];
  const float sl2 = a.scale_log2;

  // M(t): S_t = K_t Q^T and O^T += V_{t-1}^T P_{t-1}^T, interleaved.  Step i
  // does S product (kb = i % 2, c = i / 2) and P.V product (db = i / 4,
  // c = i % 4); operands are read kLook steps ahead into a ring of buffers.
  constexpr int NSTEP = KB * (D / 16);  // = (D / 32) (kBN / 16) P.V products
  constexpr int kLook = FA_LOOKAHEAD;
  constexpr int NB = kLook + 1;
  auto m_body = [&](auto do_s, auto do_pv, uint32_t kbase, uint32_t vbase) {
    constexpr bool S = decltype(do_s)::value, PV = decltype(do_pv)::value;
    constexpr int RPS = (S ? 1 : 0) + (PV ? 2 : 0);  // LDS reads per step
    uint32_t ka[D / 16], va[D / 32];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) ka[c] = kbase + kofs[c];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) va[db] = vbase + vofs[db];
    u32x4_t kr[NB];
    u32x2_t vr[NB][2];
    auto issue = [&](auto I) {
      constexpr int i = decltype(I)::value, b = i % NB;
      if constexpr (S) {
        constexpr int kbk = i % KB, c = i / KB;
        kr[b] = lds_read_b128<kbk * 32 * C::ROWB>(ka[c]);
      }
      if constexpr (PV) {
        constexpr int db = i / (kBN / 16), c = i % (kBN / 16);
        vr[b][0] = lds_read_tr16<16 * c * C::ROWB>(va[db]);
        vr[b][1] = lds_read_tr16<(16 * c + 8) * C::ROWB>(va[db]);
      }
    };
    static_for<(kLook < NSTEP ? kLook : NSTEP)>([&](auto I) { issue(I); });
    static_for<NSTEP>([&](auto I) {
      constexpr int i = decltype(I)::value, b = i % NB;
      if constexpr (i + kLook < NSTEP) issue(std::integral_constant<int, i + kLook>{});
      constexpr int ahead = (NSTEP - 1 - i) < kLook ? (NSTEP - 1 - i) : kLook;
      if constexpr (S && PV)
        lgkm_wait<RPS * ahead>(kr[b], vr[b][0], vr[b][1]);
      else if constexpr (S)
        lgkm_wait<RPS * ahead>(kr[b]);
      else
        lgkm_wait<RPS * ahead>(vr[b][0], vr[b][1]);
      if constexpr (S) {
        constexpr int kbk = i % KB, c = i / KB;
        sc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kr[b]), q[c],
                                                          c == 0 ? f32x16_t{} : sc[kbk], 0, 0, 0);
      }
      if constexpr (PV) {
        constexpr int db = i / (kBN / 16), c = i % (kBN / 16);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_bf16(vr[b][0], vr[b][1]), pb[c], o[db],
                                                        0, 0, 0);
      }
    });
  };
  auto m_phase = [&](int t) {
    const bool do_s = t < Tw;
    const bool do_pv = t >= 1 && t <= Tw;
    if (!do_s && !do_pv) return;
    const uint32_t kbase = lds_base + ring + (t & (kStages - 1)) * C::STAGE;
    const uint32_t vbase = lds_base + ring + ((t - 1) & (kStages - 1)) * C::STAGE;
    __builtin_amdgcn_s_setprio(FA_PRIO_M);
    if (do_s && do_pv)
      m_body(std::true_type{}, std::true_type{}, kbase, vbase);
    else if (do_s)
      m_body(std::true_type{}, std::false_type{}, kbase, vbase);
    else
      m_body(std::false_type{}, std::true_type{}, kbase, vbase);
    __builtin_amdgcn_s_setprio(FA_PRIO_V);
  };

  // V(t): softmax update of S_t -> P_t (bf16), l, rescaled O.
  //
  // The reference is kept in the exp2 domain (mbl = scale log2(e) times a
  // past row max).  Every tile is first tried against the current reference
  // (fast path: no row max at all); it is accepted when no lane's weights sum
  // above 2^32, so every weight stays <= 2^32.  Otherwise (scores outgrew the
  // reference, or no reference yet) the row max is taken and the reference
  // rebased on it, with O and l rescaled by exp2(old - new).
  // P = exp2(x - d) into pb.  Returns this lane's sum of the fp32 weights
  // (for l and lse) and, in *rsum, its sum of the bf16-rounded weights that
  // the P.V product actually uses (for the division O / l): normalising by
  // the rounded weights keeps each output row an exact convex combination of
  // the V rows it uses, so a row dominated by one key returns that key's V
  // row unchanged whatever the rounding of its weight.
  auto weights = [&](float d, float *rsum) {
    float pq[4];
    float rq[2] = {0.f, 0.f};
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int c = 0; c < kBN / 16; ++c)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = exp2_fast(sc[c >> 1][8 * (c & 1) + e] - d);
        const float p1 = exp2_fast(sc[c >> 1][8 * (c & 1) + e + 1] - d);
        pb[c][e] = (__bf16)p0;
        pb[c][e + 1] = (__bf16)p1;
        const int j = (c & 1) + 2 * (e >> 2);  // four partial sums: short add chains
        if (c < 2 && (e & 3) == 0)
          pq[j] = p0 + p1;
        else
          pq[j] += p0 + p1;
        const bf16x2_t pr = {pb[c][e], pb[c][e + 1]};
        rq[e >> 2] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rq[e >> 2], false);
      }
    *rsum = rq[0] + rq[1];
    return (pq[0] + pq[1]) + (pq[2] + pq[3]);
  };
  auto v_softmax = [&](int t) {
    const int key0 = (lo + t) * kBN;
    const float g = (mbl == neg_inf()) ? 0.f : mbl;  // ghost-row guard
    // x = S scale log2(e) - g; keys past the end and (causal) after the query
    // are -inf
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[b][r] = __builtin_fmaf(sc[b][r], sl2, -g);
    if ((key0 + kBN > n) || (CAUSAL && key0 + kBN - 1 > qw0)) {
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * b + block_key(r, h);
          if (!(key < n && (!CAUSAL || key <= qrow))) sc[b][r] = neg_inf();
        }
    }
    float ps = 0.f, psr = 0.f, alpha = 1.f;
    bool slow = __builtin_amdgcn_ballot_w64(mbl == neg_inf()) != 0;
    if (!slow) {
      ps = weights(0.f, &psr);
      slow = __builtin_amdgcn_ballot_w64(!(ps <= FA_FAST_BOUND)) != 0;  // NaN / inf fail too
    }
    if (slow) {
      // row max of x: four independent max3 chains over 8 values, then combined
      float mq[2 * KB];
#pragma unroll
      for (int j = 0; j < 2 * KB; ++j) {
        const int b = j >> 1, r0 = 8 * (j & 1);
        float m = max3f(sc[b][r0], sc[b][r0 + 1], sc[b][r0 + 2]);
        m = max3f(m, sc[b][r0 + 3], sc[b][r0 + 4]);
        m = max3f(m, sc[b][r0 + 5], sc[b][r0 + 6]);
        mq[j] = max2f(m, sc[b][r0 + 7]);
      }
      float mx;
      if constexpr (KB == 1) {
        mx = max2f(mq[0], mq[1]);
      } else {
        mx = max2f(max3f(mq[0], mq[1], mq[2]), mq[3]);
#pragma unroll
        for (int j = 4; j < 2 * KB; j += 2) mx = max3f(mx, mq[j], mq[j + 1]);
      }
      mx = pair_max(mx);
      // rebase when the row grew past the reference, or on its first finite score
      const bool bump = (mbl == neg_inf()) ? (mx > neg_inf()) : (mx > 0.f);
      const float delta = bump ? mx + FA_REF_MARGIN : 0.f;
      if (bump) {
        const float mbl_new = g + mx + FA_REF_MARGIN;
        alpha = exp2_fast(mbl - mbl_new);  // 0 when there was no reference
        mbl = mbl_new;
      }
      ps = weights(delta, &psr);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    }
    l_run = l_run * alpha + ps;
    lr_run = lr_run * alpha + psr;
  };
  // V(t) also sends tile t + 2 into its LDS stage, whose previous tile t - 2
  // was last read two phases earlier: before the softmax at d = 128, after
  // it at d = 64 (where the softmax phase is the longer of the two; measured
  // either way).
  auto v_phase = [&](int t) {
    if constexpr (D >= 128)
      if (t + 2 < Tg) dma_tile(t + 2);
    if (t < Tw) v_softmax(t);
    if constexpr (D < 128)
      if (t + 2 < Tg) dma_tile(t + 2);
  };

  // ---- prologue: tiles 0 and 1 in LDS (both in flight at once) -------------
  if (!SPLIT || Tg > 0) dma_tile(0);
  if (Tg > 1) dma_tile(1);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: both tiles have landed
  wg_barrier();

  // ---- ping-pong loop: phase ph; group g runs step ph - g ------------------
  for (int ph = 0; ph <= 2 * T0 + 1; ++ph) {
    const int step = ph - grp;
    if (step >= 0) {
      if (!(step & 1)) {
        m_phase(step >> 1);
        // the tile this wave sent in V(t - 1) must be in LDS before this
        // barrier: group 0 reads it in the phase after next
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0
      } else {
        v_phase(step >> 1);
      }
    }
    wg_barrier();
  }

  if constexpr (SPLIT) {
    // group 1 leaves O, l and its reference in LDS (the rings are no longer
    // read: the loop ended with a barrier); group 0 merges them into its own
    constexpr int NW = (D / 32) * 16 + 3;  // floats per lane
    float *xb = reinterpret_cast<float *>(smem) + (rw * NW) * kWave + lane;
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xb[(db * 16 + r) * kWave] = o[db][r];
      xb[(NW - 3) * kWave] = lr_run;
      xb[(NW - 2) * kWave] = mbl;
      xb[(NW - 1) * kWave] = l_run;
    }
    wg_barrier();
    if (grp == 1) return;
    const float m1 = xb[(NW - 2) * kWave], l1 = xb[(NW - 1) * kWave];
    const float mm = mbl > m1 ? mbl : m1;  // -inf only if neither half saw a key
    const float f0 = mbl == neg_inf() ? 0.f : exp2_fast(mbl - mm);
    const float f1 = m1 == neg_inf() ? 0.f : exp2_fast(m1 - mm);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * f0 + xb[(db * 16 + r) * kWave] * f1;
    l_run = l_run * f0 + l1 * f1;
    lr_run = lr_run * f0 + xb[(NW - 3) * kWave] * f1;
    mbl = mm;
  }

  // ---- finalise: O / l, lse = scale * m + ln l --------------------------------
  // (O is divided by the sum of the rounded weights it was built from, lse
  // takes the fp32 sum)
  const float l_tot = pair_sum(l_run);
  const float lr_tot = pair_sum(lr_run);
  if (qrow < n) {
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    uint16_t *orow = reinterpret_cast<uint16_t *>(a.o) + tc.base + (long long)qrow * rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const bf16x4_t x = {(__bf16)(o[db][4 * gq] * inv), (__bf16)(o[db][4 * gq + 1] * inv),
                            (__bf16)(o[db][4 * gq + 2] * inv), (__bf16)(o[db][4 * gq + 3] * inv)};
        *reinterpret_cast<bf16x4_t *>(orow + 32 * db + 8 * gq + 4 * h) = x;
      }
    if (a.lse != nullptr && h == 0) {  // lse = ln 2 (mbl + log2 l)
      const float m_fin = (mbl == neg_inf()) ? 0.f : mbl;
      a.lse[tc.lbase + (long long)qrow * a.lse_row_stride] =
          l_tot > 0.f ? (m_fin + __log2f(l_tot)) * 0.693147180559945309f : neg_inf();
    }
  }
}

template <int D, int BN, bool CAUSAL, bool VARLEN, bool SPLIT>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, BN, CAUSAL, VARLEN, SPLIT>), dim3(a.grid),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BN, bool SPLIT = false>
hipError_t launch_d(const FwdArgs &a, bool causal, bool varlen, hipStream_t stream) {
  if (causal)
    return varlen ? launch<D, BN, true, true, SPLIT>(a, stream)
                  : launch<D, BN, true, false, SPLIT>(a, stream);
  return varlen ? launch<D, BN, false, true, SPLIT>(a, stream)
                : launch<D, BN, false, false, SPLIT>(a, stream);
}

// The key-split mode (two LDS rings of 4 stages: 64-key tiles at d = 64,
// 32-key tiles at d = 128), when
// the longest sequence has at least kSplitMinLen tokens and the grid of
// 256-row workgroups is small: at most 128 workgroups (the split then fills
// the 256 CUs), or, causal, at most 256 (one round, whose time is the key
// loop of the heaviest, last query tile).  Measured at d = 64: causal grids
// of 256 gain 27-37 % from the split and of 512 lose 13-15 %; non-causal
// grids of 256 lose 20 %.
constexpr long long kSplitMaxGrid = 128;
// Grid bound of the four-way key split (32-row blocks), from an interleaved
// A/B against the two-way split above: B1 H8 N1000 d64 causal (256 blocks)
// 18.6 -> 9.7 us, B2 H4 N1500 d128 causal (376) 34.5 -> 19.3 us, B1 H1
// N16384 d64 (512) 190 -> 175 us; grids of 1024 and 2048 blocks ran
// 1.6-1.75x slower with it.
#ifndef FA_KSPLIT_MAX_GRID
#define FA_KSPLIT_MAX_GRID 512
#endif
constexpr long long kKsplitMaxGrid = FA_KSPLIT_MAX_GRID;
constexpr long long kSplitMaxGridCausal = 256;
constexpr int kSplitMinLen = 512;

// Heads of one XCD scheduled together (tile_order): the largest divisor of
// its head count up to kGroupHeads, so that the 32 CUs of an XCD run about
// eight workgroups on each head's K/V stream at once.  Interleaved A/B of
// the group size on B4 H32 N4096 d128 causal (16 heads per XCD), with the
// K/V bytes fetched from beyond L2 (FETCH_SIZE, per launch, against the
// compulsory Q + K + V):
//   group 1: 617 us, 1.00x;  2: 545 us, 1.32x;  4: 545 us, 1.38x;
//   8: 560 us, 2.15x;        16: 569 us, 3.59x.
// On the packed 16-sequence causal workload (64 heads per XCD) groups of 4
// and 8 tie (3560 and 3568 us), 2 is 3 % slower and 1 is 8 % slower.
constexpr int kGroupHeads = 4;
int head_group(int n_heads) {
  if (n_heads % kXcds != 0) return 0;
  const int hx = n_heads / kXcds;
  int g = hx < kGroupHeads ? hx : kGroupHeads;
  while (hx % g != 0) --g;
  return g;
}

}  // namespace

hipError_t launch_fwd(FwdArgs a, int dtype, int d, bool causal, bool varlen,
                      hipStream_t stream) {
  if (dtype == 0) return launch_fwd_f32(a, d, causal, varlen, stream);
  if (dtype != 1) return hipErrorInvalidValue;
  a.n_qtiles = (a.max_len + kBlockM - 1) / kBlockM;
  a.order_group = head_group(a.batch * a.H);
  long long grid = (long long)a.batch * a.H * a.n_qtiles;
  const bool split = a.max_len >= kSplitMinLen &&
                     grid <= (causal ? kSplitMaxGridCausal : kSplitMaxGrid);
  // Problems that give at most two 32-row query blocks per compute unit run
  // the four-way key split of fa_fwd_ksplit.hip instead: there the serial key
  // loop of the heaviest block, not throughput, sets the time.
  const long long ks_grid =
      (long long)a.batch * a.H * ((a.max_len + kKsplitBlockM - 1) / kKsplitBlockM);
  if (ks_grid <= kKsplitMaxGrid) {
    a.n_qtiles = (a.max_len + kKsplitBlockM - 1) / kKsplitBlockM;
    a.grid = (int)ks_grid;
    return launch_fwd_ksplit(a, d, causal, varlen, stream);
  }
  if (split) {
    a.n_qtiles = (a.max_len + kBlockM / 2 - 1) / (kBlockM / 2);
    grid = (long long)a.batch * a.H * a.n_qtiles;
  }
  if (grid > 0x7fffffffll || grid <= 0) return hipErrorInvalidValue;
  a.grid = (int)grid;
  if (split) {
    if (d == 64) return launch_d<64, 64, true>(a, causal, varlen, stream);
    if (d == 128) return launch_d<128, 32, true>(a, causal, varlen, stream);
    return hipErrorInvalidValue;
  }
  if (d == 64)
    return a.max_len >= kWideMinLen ? launch_d<64, 128>(a, causal, varlen, stream)
                                    : launch_d<64, 64>(a, causal, varlen, stream);
  if (d == 128) return launch_fwd_pipe(a, causal, varlen, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa355
