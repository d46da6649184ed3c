// fa_small.hip -- one-tile attention forward for short sequences (N <= 128)
// on gfx950: bf16 on the matrix cores, fp32 on the vector ALU.
//
// When a whole sequence fits in one key tile, the streaming loop of the
// general kernel has nothing to stream: "Mini FlashAttention", section 3
// ("Part A", one-shot fused attention) computes S, the softmax and P V for
// the entire tile at once, with no running max to rescale.  This kernel does
// that, sized for many short sequences: the general kernel gives every
// (batch, head) a 256-row query tile and a software pipeline whose start-up
// dominates at N <= 128, so with thousands of short heads it ran slower
// than even the unfused method.
//
// Workgroup: 4 waves and G = 4 / ceil(N / 32) heads (4 heads of N <= 32,
// 2 of N <= 64, one otherwise); wave i owns 32 queries of head i / (waves
// per head).  The workgroup stages the K and V rows of its heads in LDS once
// (16-byte coalesced loads, zero rows past N; a compile-time number per
// thread, all issued before the first LDS write, so that one load latency
// covers them all), synchronises once, and then every wave works alone:
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (lane l holds query l % 32 and
//       keys 8 (r / 4) + 4 (l / 32) + r % 4 of each 32-key block in register
//       r), K rows read from LDS with ds_read_b128 (reading K straight
//       from L2 instead, to halve the LDS and double the workgroups per CU
//       at d = 128, measured slower);
//   the row max and sum over at most 128 keys in the lane plus one exchange
//   with lane l ^ 32 (the other half of the same query); keys >= N and,
//   causal, keys after the query score -inf;
//   O^T = V^T P^T with the unnormalised weights, rounded to bf16, taken
//   straight from the score registers as the B operand; the A operand is
//   read with ds_read_b64_tr_b16 from the V rows in the order the score
//   registers hold their keys (rows 4 h + 0..3 and 8 + 4 h + 0..3 of each
//   16-key step);
//   O = O^T / l in bf16 (round to nearest even), lse = m + ln l.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fa_bf16_tile.h"
#include "fa_common.h"
#include "fa_small_launch.h"

namespace fa355 {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = 128;
constexpr float kLn2 = 0.6931471805599453f;

typedef short i16x4v_t __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 through its builtin, so the compiler schedules the
// reads and their waits: within each 16-lane group, lane i receives column i
// of the four rows the group's lanes address (lane j of the group reads row
// j / 4, columns 4 (j % 4) .. + 3).
__device__ __forceinline__ u32x2_t tr_read(const uint16_t *p) {
  const i16x4v_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4v_t *)(p));
  return __builtin_bit_cast(u32x2_t, x);
}

// (sequence, head) pair bh -> its length and element / lse offsets, for a
// fixed-length batch or (VARLEN) a packed one
template <bool VARLEN>
__device__ __forceinline__ void pair_coords(const FwdArgs &a, int bh, int &n, long long &base,
                                            long long &lbase) {
  const int s = bh / a.H, hd = bh - s * a.H;
  if constexpr (VARLEN) {
    const int t0 = a.cu_seqlens[s];
    n = a.cu_seqlens[s + 1] - t0;
    base = (long long)t0 * a.row_stride + (long long)hd * a.head_stride;
    lbase = (long long)t0 * a.lse_row_stride + (long long)hd * a.lse_head_stride;
  } else {
    n = a.n;
    base = (long long)s * a.seq_stride + (long long)hd * a.head_stride;
    lbase = (long long)s * a.lse_seq_stride + (long long)hd * a.lse_head_stride;
  }
}

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads) void small_bf16(FwdArgs a, int heads_per_wg, int nb) {
  constexpr int RSK = D + 8;   // K row stride in LDS (elements): 16-byte pad, conflict-free b128 reads
  constexpr int RSV = D + 16;  // V row stride: 32-byte pad, conflict-free transposing reads
  __shared__ __attribute__((aligned(16))) uint16_t ks[kMaxN * RSK];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kMaxN * RSV];

  const int n_heads = a.batch * a.H;
  const int h0 = blockIdx.x * heads_per_wg;  // first (sequence, head) of this workgroup
  const int rows = heads_per_wg * nb;        // staged rows (nb = longest N rounded up to 32)
  const uint16_t *kg = static_cast<const uint16_t *>(a.k);
  const uint16_t *vg = static_cast<const uint16_t *>(a.v);
  // length and offset of each of the (at most 4) heads of the workgroup
  int sn[4];
  long long sb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    long long lb;
    sn[i] = 0;
    sb[i] = 0;
    if (i < heads_per_wg && h0 + i < n_heads) pair_coords<VARLEN>(a, h0 + i, sn[i], sb[i], lb);
  }

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int wph = nb / 32;  // waves per head
  const int slot = wv / wph, qb = wv - slot * wph;
  const int bh = h0 + slot;
  const bool active = slot < heads_per_wg && bh < n_heads;  // wave-uniform
  const int qi = 32 * qb + l32;                             // this lane's query
  long long base = 0, lbase = 0;
  int n = 0;  // this wave's sequence length
  if (active) pair_coords<VARLEN>(a, bh, n, base, lbase);

  // ---- all loads first: this wave's query rows, then the K and V rows of the
  // workgroup's heads (a compile-time count per thread, so that every load is
  // in flight before the first LDS write waits for one) ------------------------
  u32x4_t qx[D / 16];
  {
    const uint16_t *qg = static_cast<const uint16_t *>(a.q) + base;
    // (unconditional loads from a valid row, zeroed afterwards: no branches
    // around the loads)
    const bool qok = active && qi < n;
    const uint16_t *qp = qg + (qok ? (long long)qi * a.row_stride : 0) + 8 * h;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t *>(qp + 16 * c);
      qx[c] = qok ? x : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  constexpr int PER = kMaxN * (D / 8) / kThreads;  // 16-byte pieces per thread and tensor, at most
  u32x4_t kx[PER], vx[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = threadIdx.x + j * kThreads;
    const int row = c / (D / 8), col = 8 * (c % (D / 8));
    const int sl = row / nb, key = row - sl * nb;
    const int n_s = sl == 0 ? sn[0] : sl == 1 ? sn[1] : sl == 2 ? sn[2] : sn[3];
    const long long b_s = sl == 0 ? sb[0] : sl == 1 ? sb[1] : sl == 2 ? sb[2] : sb[3];
    // n_s = 0 for slots past the last head; zeros past N (the load then reads
    // the first row of the tensor and is discarded)
    const bool ok = row < rows && key < n_s;
    const long long off = ok ? b_s + (long long)key * a.row_stride + col : col;
    const u32x4_t kk = *reinterpret_cast<const u32x4_t *>(kg + off);
    const u32x4_t vv = *reinterpret_cast<const u32x4_t *>(vg + off);
    kx[j] = ok ? kk : u32x4_t{0u, 0u, 0u, 0u};
    vx[j] = ok ? vv : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = threadIdx.x + j * kThreads;
    const int row = c / (D / 8), col = 8 * (c % (D / 8));
    if (row < rows) {
      *reinterpret_cast<u32x4_t *>(ks + row * RSK + col) = kx[j];
      *reinterpret_cast<u32x4_t *>(vs + row * RSV + col) = vx[j];
    }
  }
  bf16x8_t qr[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) qr[c] = __builtin_bit_cast(bf16x8_t, qx[c]);
  __syncthreads();

  const int krow0 = slot * nb;  // first LDS row of this head
  f32x16_t o[D / 32];
  float m = neg_inf(), l = 0.f;
  if (active) {
    // key blocks this wave needs: all of the head's, or (causal) up to its own
    const int nkb = CAUSAL ? qb + 1 : wph;

    // ---- S^T blocks, masked, in log2 units ----
    f32x16_t sc[kMaxN / 32];
#pragma unroll
    for (int kb = 0; kb < kMaxN / 32; ++kb) {
      if (kb >= nkb) break;  // wave-uniform
      f32x16_t acc = {};
      const uint16_t *krow = ks + (krow0 + 32 * kb + l32) * RSK + 8 * h;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4_t kx = *reinterpret_cast<const u32x4_t *>(krow + 16 * c);  // ds_read_b128
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qr[c], acc,
                                                      0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + block_key(r, h);
        const bool vis = key < n && (!CAUSAL || key <= qi);
        acc[r] = vis ? acc[r] * a.scale_log2 : neg_inf();
        m = fmaxf(m, acc[r]);
      }
      sc[kb] = acc;
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    const float mu = (m == neg_inf()) ? 0.f : m;  // a query with no visible key
#pragma unroll
    for (int kb = 0; kb < kMaxN / 32; ++kb) {
      if (kb >= nkb) break;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[kb][r] = exp2_fast(sc[kb][r] - mu);
        l += sc[kb][r];
      }
    }
    l += __shfl_xor(l, 32);

    // ---- O^T = V^T P^T ----
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
    const int g = lane >> 4, j = lane & 15;
    // first transposing read: rows 4 (g / 2) + j / 4 of the 16-key step,
    // columns 16 (g % 2) + 4 (j % 4); the second read is 8 rows further
    const uint16_t *va = vs + (krow0 + 4 * (g >> 1) + (j >> 2)) * RSV + 16 * (g & 1) + 4 * (j & 3);
#pragma unroll
    for (int kb = 0; kb < kMaxN / 32; ++kb) {
      if (kb >= nkb) break;
#pragma unroll
      for (int st = 0; st < 2; ++st) {  // 16-key steps: score registers 8 st .. 8 st + 7
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sc[kb][8 * st + e];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const uint16_t *ad = va + (32 * kb + 16 * st) * RSV + 32 * db;
          const u32x2_t lo = tr_read(ad), hi = tr_read(ad + 8 * RSV);
          const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av), pb, o[db],
                                                          0, 0, 0);
        }
      }
    }
  }

  // ---- O = O^T / l through LDS, lse ----
  // Once every wave is done with K and V, each wave stages its 32 output
  // rows in its own 32 staged K rows and reads them back as whole 16-byte
  // row chunks, so that the stores cover whole rows (the score layout would
  // give every store 32 row pieces of 16 bytes).
  __syncthreads();
  if (!active) return;
  {
    uint16_t *const st = ks + (krow0 + 32 * qb) * RSK;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const bf16x4_t x = {(__bf16)(o[db][4 * gq] * inv), (__bf16)(o[db][4 * gq + 1] * inv),
                            (__bf16)(o[db][4 * gq + 2] * inv), (__bf16)(o[db][4 * gq + 3] * inv)};
        *reinterpret_cast<bf16x4_t *>(st + l32 * RSK + 32 * db + 8 * gq + 4 * h) = x;
      }
  }
  if (h == 0 && a.lse != nullptr && qi < n)
    a.lse[lbase + (long long)qi * a.lse_row_stride] = (l > 0.f) ? (m + __log2f(l)) * kLn2 : neg_inf();
  {
    constexpr int CH = D / 8;                // 16-byte chunks per row
    constexpr int OL = 32 * CH / kWave;      // per lane
    const uint16_t *const st = ks + (krow0 + 32 * qb) * RSK;
    uint16_t *const og = static_cast<uint16_t *>(a.o) + base;
#pragma unroll
    for (int j = 0; j < OL; ++j) {
      const int p = j * kWave + lane, r = p / CH, c = p % CH;
      const u32x4_t y = *reinterpret_cast<const u32x4_t *>(st + r * RSK + 8 * c);
      if (32 * qb + r < n)
        *reinterpret_cast<u32x4_t *>(og + (long long)(32 * qb + r) * a.row_stride + 8 * c) = y;
    }
  }
}

// ---- bf16, N = 97 .. 128, more heads than compute units: staged ahead ------
// small_bf16 loads a head, computes it and stores it; with two workgroups
// per compute unit the memory pipe idles whenever both compute, and short
// heads are bound by that pipe.  Here one workgroup per compute unit (two at
// d = 64) walks its heads (blockIdx.x, then every gridDim.x-th) and keeps the
// next heads' loads in flight while it computes:
//   LDS: a two-head ring of K and V (rows of 64-key blocks, XOR-swizzled as
//        in the streaming kernels, filled by direct global -> LDS loads) and
//        one head's query rows, each wave's 32 rows written and read by that
//        wave alone;
//   head i: its query rows go to registers and the wave's rows of head
//        i + 1 to LDS in their place; S, the softmax and P V as in
//        small_bf16 from ring half i % 2; a barrier; O through the free ring
//        half to whole-row stores; a barrier; K and V of head i + 2 into ring
//        half i % 2; a wait for head i + 1's loads; a barrier.
// Rows past a head's length are loaded as zeros (buffer loads whose range
// ends with the last row), their scores masked, their outputs not stored.
// One 16-byte-per-lane global -> LDS load (a plain function: inside a
// template over the head dimension the builtin leaves the kernel without its
// host-side stub).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, FA_LDS void *dst,
                                      uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, 0, 0, 0);
}

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 1) void small_bf16_stream(FwdArgs a) {
  using TT = bf16t::Bf16Tile<D, 64>;
  constexpr int ROWB = TT::ROWB, TILE = TT::TILE, CPR = TT::CPR;
  constexpr int KV = 2 * TILE;      // 128 rows of K or of V
  constexpr int BUF = 2 * KV;       // K then V of one head
  constexpr int QOFF = 2 * BUF;     // one head's query rows
  constexpr int LDS = QOFF + KV;    // 160 KB at d = 128, 80 KB at d = 64
  constexpr int M = TILE / 4096;    // loads per wave per 64-row block of K or V
  constexpr int QL = TILE / 2048;   // loads of a wave's 32 query rows
  constexpr int NL = 4 * M;         // loads per wave of a head's K and V
  static_assert(kThreads == 256 && kMaxN == 128, "four waves, 128 rows");
  __shared__ __attribute__((aligned(1024))) char smem[LDS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int n_heads = a.batch * a.H;
  const int G = static_cast<int>(gridDim.x);
  int head = blockIdx.x;
  if (head >= n_heads) return;  // uniform, before any barrier

  const long long rs = a.row_stride;
  const uint32_t rsb = static_cast<uint32_t>(a.row_stride) * 2u;
  const uint16_t *const qg = static_cast<const uint16_t *>(a.q);
  const uint16_t *const kg = static_cast<const uint16_t *>(a.k);
  const uint16_t *const vg = static_cast<const uint16_t *>(a.v);
  // a head's length and offsets (packed batches read the sequence offsets
  // with scalar loads, which the staging loads in flight do not hold up)
  auto coords = [&](int bh, int &n, long long &base, long long &lbase) {
    const int s = bh / a.H, hd = bh - s * a.H;
    if constexpr (VARLEN) {
      using CInt = __attribute__((address_space(4))) const int;
      CInt *cs = (CInt *)(a.cu_seqlens);
      const int t0 = cs[s];
      n = cs[s + 1] - t0;
      base = (long long)t0 * a.row_stride + (long long)hd * a.head_stride;
      lbase = (long long)t0 * a.lse_row_stride + (long long)hd * a.lse_head_stride;
    } else {
      n = a.n;
      base = (long long)s * a.seq_stride + (long long)hd * a.head_stride;
      lbase = (long long)s * a.lse_seq_stride + (long long)hd * a.lse_head_stride;
    }
  };
  auto rows_rec = [&](int valid, int cap) {
    valid = valid < cap ? valid : cap;
    return valid > 0 ? (valid - 1) * static_cast<int>(rsb) + ROWB : 0;
  };

  // ---- staging -------------------------------------------------------------
  // Load m of wave w in a 64-row block fills the 1 KB of 16-byte slots
  // p = (w + 4m) * 64 + lane (row p / CPR, slot p % CPR); a wave's query
  // load j fills slots p = j * 64 + lane of its 32 rows.  Each lane fetches
  // the logical chunk the swizzle places in its slot.
  uint32_t o_k[M], o_v[M], o_q[QL];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int p = (w + 4 * m) * kWave + lane, row = p / CPR, slot = p % CPR;
    o_k[m] = row * rsb + 16u * (slot ^ TT::swz_k(row));
    o_v[m] = row * rsb + 16u * (slot ^ TT::swz_v(row));
  }
#pragma unroll
  for (int j = 0; j < QL; ++j) {
    const int p = j * kWave + lane, row = p / CPR, slot = p % CPR;
    o_q[j] = row * rsb + 16u * (slot ^ TT::swz_k(row));  // (rows 32 w + row: same swizzle)
  }
  auto dma_kv = [&](long long base, int n, int buf) {  // n = 0: nothing is read, zeros land
#pragma unroll
    for (int b = 0; b < 4; ++b) {  // K rows 0..63, 64..127, then V's
      const uint16_t *src = (b < 2 ? kg : vg) + base + (long long)(64 * (b & 1)) * rs;
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t *>(src), (short)0, rows_rec(n - 64 * (b & 1), 64), 0x00020000);
#pragma unroll
      for (int m = 0; m < M; ++m)
        dma16(rsrc, (FA_LDS void *)(smem + buf * BUF + b * TILE + (w + 4 * m) * 1024),
              b < 2 ? o_k[m] : o_v[m]);
    }
  };
  auto dma_q = [&](long long base, int n) {  // this wave's 32 query rows
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(qg + base + (long long)(32 * w) * rs), (short)0,
        rows_rec(n - 32 * w, 32), 0x00020000);
#pragma unroll
    for (int j = 0; j < QL; ++j)
      dma16(rsrc, (FA_LDS void *)(smem + QOFF + 32 * w * ROWB + j * 1024), o_q[j]);
  };

  // ---- LDS operand addresses ------------------------------------------------
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS char *)smem));
  uint32_t kofs[D / 16];  // K rows l32 of a 32-key block, chunk 2c + h (also the Q rows)
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    kofs[c] = l32 * ROWB + 16 * ((2 * c + h) ^ TT::swz_k(l32));
  uint32_t vofs[D / 32];  // V^T operand: rows 4h + e4 (+ 8) of a 16-key step, d 32 db + ..
  {
    const int j = lane & 15, e4 = j >> 2, gq = (lane >> 4) & 1;
    const int sw = TT::swz_v(e4);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      vofs[db] = KV + (4 * h + e4) * ROWB + 16 * ((4 * db + 2 * gq + ((j & 3) >> 1)) ^ sw) +
                 8 * (j & 1);
  }

  // ---- prologue: head 0's query rows and K/V, head 1's K/V --------------------
  int n0, n1 = 0, n2 = 0;
  long long b0, lb0, b1 = 0, lb1 = 0, b2 = 0, lb2 = 0;
  coords(head, n0, b0, lb0);
  bool ok1 = head + G < n_heads;
  if (ok1) coords(head + G, n1, b1, lb1);
  dma_q(b0, n0);
  dma_kv(b0, n0, 0);
  dma_kv(b1, ok1 ? n1 : 0, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (NL & 15) | ((NL >> 4) << 14));  // all but head 1's K/V
  bf16t::wg_barrier();

  const int qi = 32 * w + l32;  // this lane's query
  for (int it = 0;; ++it) {
    const uint32_t kvb = lds_base + (it & 1) * BUF;
    // this head's query rows (Q^T operand chunks) into registers, then the
    // next head's rows to the same LDS
    bf16x8_t qr[D / 16];
    {
      u32x4_t qx[D / 16];
      const uint32_t qa = lds_base + QOFF + 32 * w * ROWB;
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        asm volatile("ds_read_b128 %0, %1" : "=v"(qx[c]) : "v"(qa + kofs[c]));
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(qx[0]));
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        if (c > 0) asm volatile("" : "+v"(qx[c]));
        qr[c] = __builtin_bit_cast(bf16x8_t, qx[c]);
      }
    }
    dma_q(b1, ok1 ? n1 : 0);

    const int n = n0;
    const bool active = 32 * w < n;  // wave-uniform
    f32x16_t o[D / 32];
    float m = neg_inf(), l = 0.f;
    if (active) {
      const int nkb = CAUSAL ? w + 1 : (n + 31) / 32;  // key blocks this wave reads
      // last visible key of this lane's query, less the lane's key offset
      // 4h (opaque: otherwise the compiler keeps a lane mask per score
      // register from before the loop)
      int lim = n - 1;
      if constexpr (CAUSAL) lim = lim < qi ? lim : qi;
      lim -= 4 * h;
      asm volatile("" : "+v"(lim));
      // ---- S^T blocks, masked, in log2 units ----
      f32x16_t sc[kMaxN / 32];
#pragma unroll
      for (int kb = 0; kb < kMaxN / 32; ++kb) {
        if (kb >= nkb) break;  // wave-uniform
        u32x4_t kx[D / 16];
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
          asm volatile("ds_read_b128 %0, %1" : "=v"(kx[c]) : "v"(kvb + kofs[c] + 32 * kb * ROWB));
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kx[0]));
        f32x16_t acc = {};
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          if (c > 0) asm volatile("" : "+v"(kx[c]));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx[c]),
                                                        qr[c], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + 8 * (r >> 2) + (r & 3);  // key - 4h
          acc[r] = off <= lim ? acc[r] * a.scale_log2 : neg_inf();
          m = fmaxf(m, acc[r]);
        }
        sc[kb] = acc;
      }
      m = bf16t::pair_max(m);
      const float mu = (m == neg_inf()) ? 0.f : m;  // a query with no visible key
#pragma unroll
      for (int kb = 0; kb < kMaxN / 32; ++kb) {
        if (kb >= nkb) break;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[kb][r] = exp2_fast(sc[kb][r] - mu);
          l += sc[kb][r];
        }
      }
      l = bf16t::pair_sum(l);
      // ---- O^T = V^T P^T ----
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
#pragma unroll
      for (int kb = 0; kb < kMaxN / 32; ++kb) {
        if (kb >= nkb) break;
#pragma unroll
        for (int st = 0; st < 2; ++st) {  // 16-key steps: score registers 8 st .. 8 st + 7
          const uint32_t vb = kvb + (32 * kb + 16 * st) * ROWB;
          u32x2_t lo[D / 32], hi[D / 32];
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo[db]) : "v"(vb + vofs[db]));
            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                         : "=v"(hi[db]) : "v"(vb + vofs[db]), "i"(8 * ROWB));
          }
          bf16x8_t pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sc[kb][8 * st + e];
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(lo[0]), "+v"(hi[0]));
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            if (db > 0) asm volatile("" : "+v"(lo[db]), "+v"(hi[db]));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf16t::cat_bf16(lo[db], hi[db]), pb,
                                                            o[db], 0, 0, 0);
          }
        }
      }
    }
    bf16t::wg_barrier();  // every wave is done with this ring half
    // ---- O = O^T / l through LDS, lse ----
    // The wave's 32 output rows go to its quarter of the free ring half's K
    // rows (row-major, 16-byte chunk c of row r in slot c ^ (r % CPR)), then
    // back as whole 16-byte chunks, so that the stores cover whole rows
    // (the score layout would give every store 32 row pieces of 16 bytes).
    if (active) {
      const uint32_t ob = kvb + 32 * w * ROWB;
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const bf16x4_t x = {(__bf16)(o[db][4 * gq] * inv), (__bf16)(o[db][4 * gq + 1] * inv),
                              (__bf16)(o[db][4 * gq + 2] * inv), (__bf16)(o[db][4 * gq + 3] * inv)};
          const uint32_t ad = ob + l32 * ROWB + 16 * ((4 * db + gq) ^ (l32 % CPR)) + 8 * h;
          asm volatile("ds_write_b64 %0, %1" ::"v"(ad), "v"(__builtin_bit_cast(u32x2_t, x))
                       : "memory");
        }
      if (h == 0 && a.lse != nullptr && qi < n)
        a.lse[lb0 + (long long)qi * a.lse_row_stride] =
            (l > 0.f) ? (m + __log2f(l)) * kLn2 : neg_inf();
      uint16_t *const og = static_cast<uint16_t *>(a.o) + b0;
      constexpr int OL = 32 * CPR / kWave;  // 16-byte chunks per lane
      u32x4_t y[OL];
#pragma unroll
      for (int j = 0; j < OL; ++j) {
        const int p = j * kWave + lane, r = p / CPR, c = p % CPR;
        asm volatile("ds_read_b128 %0, %1" : "=v"(y[j]) : "v"(ob + r * ROWB + 16 * (c ^ (r % CPR))));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(y[0]));
#pragma unroll
      for (int j = 0; j < OL; ++j) {
        if (j > 0) asm volatile("" : "+v"(y[j]));
        const int p = j * kWave + lane, r = p / CPR, c = p % CPR;
        if (32 * w + r < n)
          *reinterpret_cast<u32x4_t *>(og + (long long)(32 * w + r) * rs + 8 * c) = y[j];
      }
    }
    bf16t::wg_barrier();  // every wave has read its rows back

    // K and V of the head after next into the ring half just freed, then wait
    // for the next head's loads (the wait also covers this head's stores,
    // issued before them)
    const bool ok2 = ok1 && head + 2 * G < n_heads;
    if (ok2) coords(head + 2 * G, n2, b2, lb2);
    dma_kv(b2, ok2 ? n2 : 0, it & 1);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NL & 15) | ((NL >> 4) << 14));
    bf16t::wg_barrier();
    if (!ok1) break;
    head += G;
    n0 = n1; b0 = b1; lb0 = lb1;
    n1 = n2; b1 = b2; lb1 = lb2;
    ok1 = ok2;
  }
  // no staging load outlives the workgroup (the last ones, past the last
  // head, move no memory)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// ---- fp32 ------------------------------------------------------------------
// fp32 has no fast matrix path worth its set-up at this size (the fp32
// matrix cores and the vector ALU have the same peak), so this variant
// spends its effort on latency instead: a workgroup of 256 threads takes 16
// queries of one head (a one-head N = 128 problem spreads over 8 CUs), and
// all arithmetic is plain fp32 FMA, which keeps the fp32 result within 1e-5.
//   1. K rows (N <= 128, rows padded by 4 floats so 16 lanes reading 16 rows
//      with 16-byte reads hit distinct banks) go to LDS; thread t owns query
//      t / 16 and keys t % 16 + 16 i, i < 8, and forms their scores from its
//      query row (registers) and the K rows;
//   2. the row max and sum over the 16 threads of a query (shuffles), the
//      weights into LDS;
//   3. V replaces K in LDS; thread t forms O[q][4 (t % 16) .. + 3] (d = 64)
//      or two such groups (d = 128) as the weighted sum over the keys.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void small_f32(FwdArgs a, int qblocks) {
  constexpr int QB = 16;       // queries per workgroup
  constexpr int RS = D + 4;    // LDS row stride (floats)
  constexpr int CPT = D / 64;  // 4-column groups per thread in step 3
  __shared__ __attribute__((aligned(16))) float kv[kMaxN * RS];
  __shared__ __attribute__((aligned(16))) float pw[QB * kMaxN];

  const int n = a.n;
  const int bh = blockIdx.x / qblocks, qb = blockIdx.x - bh * qblocks;
  const int s = bh / a.H, hd = bh - s * a.H;
  const long long base = (long long)s * a.seq_stride + (long long)hd * a.head_stride;
  const long long lbase = (long long)s * a.lse_seq_stride + (long long)hd * a.lse_head_stride;
  const float *qg = static_cast<const float *>(a.q) + base;
  const float *kg = static_cast<const float *>(a.k) + base;
  const float *vg = static_cast<const float *>(a.v) + base;
  const int t = threadIdx.x, ql = t >> 4, jj = t & 15;
  const int qi = qb * QB + ql;  // this thread's query

  // The loads go out in rounds of at most 8 per thread: this thread's query
  // row, then its pieces of the K rows (one round at d = 64, two at d = 128)
  // and, at d = 64, of the V rows, a compile-time count from valid rows (rows
  // past n stage duplicates that are never read).  K goes to LDS first; at
  // d = 64, V waits in registers until the scores are done with K.
  constexpr int PER = kMaxN * (D / 4) / kThreads;  // 16-byte pieces per thread and tensor
  constexpr int RND = 8;                            // pieces per round
  constexpr bool kVEarly = D == 64;
  static_assert(PER % RND == 0, "rounds");
  f32x4_t qr[D / 4];
  {
    const bool qok = qi < n;
    const float *qp = qg + (qok ? (long long)qi * a.row_stride : 0);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t *>(qp + 4 * c);
      qr[c] = qok ? x : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
  // pieces per thread that hold rows below n (uniform: the rest are skipped)
  const int need = (n * (D / 4) + kThreads - 1) / kThreads;
  auto load = [&](const float *src, f32x4_t *x, int r) {
#pragma unroll
    for (int i = 0; i < RND; ++i) {
      if (r * RND + i >= need) break;
      const int c = t + (r * RND + i) * kThreads;
      const int row = c / (D / 4), col = 4 * (c % (D / 4));
      x[i] = *reinterpret_cast<const f32x4_t *>(src + (long long)(row < n ? row : n - 1) *
                                                           a.row_stride + col);
    }
  };
  auto store = [&](const f32x4_t *x, int r) {
#pragma unroll
    for (int i = 0; i < RND; ++i) {
      if (r * RND + i >= need) break;
      const int c = t + (r * RND + i) * kThreads;
      const int row = c / (D / 4), col = 4 * (c % (D / 4));
      *reinterpret_cast<f32x4_t *>(kv + row * RS + col) = x[i];
    }
  };
  f32x4_t px[RND], vx[RND];
#pragma unroll
  for (int r = 0; r < PER / RND; ++r) {
    load(kg, px, r);
    if (kVEarly && r == 0) load(vg, vx, 0);
    store(px, r);
  }
  __syncthreads();

  // 1. scores of keys jj + 16 i
  float sc[8];
  float m = neg_inf();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = jj + 16 * i;
    float acc = 0.f;
    if (j < n) {
      const float *kr = kv + j * RS;
#pragma unroll
      for (int c = 0; c < D / 4; ++c) {
        const f32x4_t kx = *reinterpret_cast<const f32x4_t *>(kr + 4 * c);
        acc = __builtin_fmaf(qr[c][0], kx[0], acc);
        acc = __builtin_fmaf(qr[c][1], kx[1], acc);
        acc = __builtin_fmaf(qr[c][2], kx[2], acc);
        acc = __builtin_fmaf(qr[c][3], kx[3], acc);
      }
    }
    const bool vis = j < n && (!CAUSAL || j <= qi);
    sc[i] = vis ? acc * a.scale_log2 : neg_inf();
    m = fmaxf(m, sc[i]);
  }
  // 2. max and sum over the query's 16 threads
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float mu = (m == neg_inf()) ? 0.f : m;
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = exp2_fast(sc[i] - mu);
    l += p;
    pw[ql * kMaxN + jj + 16 * i] = p;
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) l += __shfl_xor(l, off);
  __syncthreads();  // every thread is done with K
#pragma unroll
  for (int r = 0; r < PER / RND; ++r) {
    if (!kVEarly || r > 0) load(vg, vx, r);
    store(vx, r);
  }
  __syncthreads();

  // 3. O[q][cols] = sum_j p_j V[j][cols]
  f32x4_t o[CPT];
#pragma unroll
  for (int g = 0; g < CPT; ++g) o[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nj = CAUSAL ? (qb * QB + QB < n ? qb * QB + QB : n) : n;  // keys any query here sees
  const float *pr = pw + ql * kMaxN;
  for (int j = 0; j < nj; ++j) {
    const float p = pr[j];
#pragma unroll
    for (int g = 0; g < CPT; ++g) {
      const f32x4_t vx = *reinterpret_cast<const f32x4_t *>(kv + j * RS + 64 * g + 4 * jj);
      o[g][0] = __builtin_fmaf(p, vx[0], o[g][0]);
      o[g][1] = __builtin_fmaf(p, vx[1], o[g][1]);
      o[g][2] = __builtin_fmaf(p, vx[2], o[g][2]);
      o[g][3] = __builtin_fmaf(p, vx[3], o[g][3]);
    }
  }
  if (qi >= n) return;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  float *orow = static_cast<float *>(a.o) + base + (long long)qi * a.row_stride;
#pragma unroll
  for (int g = 0; g < CPT; ++g)
    *reinterpret_cast<f32x4_t *>(orow + 64 * g + 4 * jj) =
        f32x4_t{o[g][0] * inv, o[g][1] * inv, o[g][2] * inv, o[g][3] * inv};
  if (jj == 0 && a.lse != nullptr)
    a.lse[lbase + (long long)qi * a.lse_row_stride] = (l > 0.f) ? (m + __log2f(l)) * kLn2 : neg_inf();
}

template <int D>
hipError_t run_f32(const FwdArgs &a, bool causal, hipStream_t st) {
  const int qblocks = (a.n + 15) / 16;
  const long long grid = (long long)a.batch * a.H * qblocks;
  if (grid <= 0 || grid > 0x7fffffffll) return hipErrorInvalidValue;
  if (causal)
    hipLaunchKernelGGL((small_f32<D, true>), dim3((unsigned)grid), dim3(kThreads), 0, st, a, qblocks);
  else
    hipLaunchKernelGGL((small_f32<D, false>), dim3((unsigned)grid), dim3(kThreads), 0, st, a, qblocks);
  return hipGetLastError();
}

// Compute units of the current device (cached per device; 0 if unknown,
// which keeps the plain one-tile kernel).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <int D, bool VARLEN>
hipError_t run(const FwdArgs &a, bool causal, hipStream_t st) {
  const int nb = (a.max_len + 31) & ~31;
  const int heads_per_wg = 4 / (nb / 32);  // 4, 2, 1, 1
  const long long n_heads = (long long)a.batch * a.H;
  // Heads of 97 .. 128 rows, more of them than the workgroups a GPU holds at
  // once: the staged-ahead variant, one workgroup per compute unit (two at
  // d = 64) working through its heads.
  const long long resident = (long long)device_cus() * (D == 64 ? 2 : 1);
  if (nb == kMaxN && resident > 0 && n_heads > resident) {
    if (causal)
      hipLaunchKernelGGL((small_bf16_stream<D, true, VARLEN>), dim3((unsigned)resident),
                         dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((small_bf16_stream<D, false, VARLEN>), dim3((unsigned)resident),
                         dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  const long long grid = (n_heads + heads_per_wg - 1) / heads_per_wg;
  if (grid <= 0 || grid > 0x7fffffffll) return hipErrorInvalidValue;
  if (causal)
    hipLaunchKernelGGL((small_bf16<D, true, VARLEN>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                       a, heads_per_wg, nb);
  else
    hipLaunchKernelGGL((small_bf16<D, false, VARLEN>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                       a, heads_per_wg, nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_small_f32(const FwdArgs &a, int d, bool causal, hipStream_t stream) {
  if (a.n <= 0 || a.n > kSmallMaxN) return hipErrorInvalidValue;
  if (d == 64) return run_f32<64>(a, causal, stream);
  if (d == 128) return run_f32<128>(a, causal, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_small_bf16(const FwdArgs &a, int d, bool causal, bool varlen,
                             hipStream_t stream) {
  if (a.max_len <= 0 || a.max_len > kSmallMaxN) return hipErrorInvalidValue;
  if (d == 64) return varlen ? run<64, true>(a, causal, stream) : run<64, false>(a, causal, stream);
  if (d == 128)
    return varlen ? run<128, true>(a, causal, stream) : run<128, false>(a, causal, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa355
