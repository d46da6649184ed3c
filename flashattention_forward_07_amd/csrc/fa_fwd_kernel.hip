// fa_fwd_kernel.hip -- attention forward kernels for gfx950 (MI355X, CDNA4).
//
// One workgroup owns a block of kBlockM = 128 query rows of one (sequence,
// head): four wave64s, each with 32 rows held in registers for the whole
// kernel.  K/V tiles of BN keys stream through double-buffered LDS; for
// every tile a wave computes its 32 x BN scores on the matrix cores, runs
// the online-softmax update on them in registers, and adds P.V into an fp32
// accumulator on the matrix cores.  This is the resident-query loop order
// of "Mini FlashAttention", section 4 (and the initialise / loop / finalise
// structure of the grasp.study lesson "The Complete Kernel: Initialization,
// Loop, and Finalization"): state m = -inf, l = 0, O = 0; per tile
//     m_new = max(m, rowmax S),  alpha = exp(m - m_new),
//     P = exp(S - m_new),  l = alpha l + rowsum P,  O = alpha O + P V;
// and O / l once at the end.  The score matrix never leaves registers.
//
// Matrix-core layout (gfx950 v_mfma_f32_32x32x16_bf16, D = A.B + C with
// A 32x16, B 16x32): the kernel computes the TRANSPOSED score block
// S^T = K . Q^T, so that the 32 output columns are the wave's 32 queries.
// An output lane l then holds query (l % 32) and 16 keys of a 32-key block,
// keys 8*(r/4) + 4*(l/32) + r%4 for accumulator register r.  Row max and row
// sum are therefore 15 in-register operations plus one exchange with lane
// l ^ 32, and the per-row rescale factor is a per-lane scalar.  The same
// registers, rounded to bf16, are the B operand of O^T += V^T . P^T once the
// contraction index is re-labelled: in the 16-key chunk c the operand's
// k = 8*(l/32) + e is taken to be key 16c + 8*(e/4) + 4*(l/32) + e%4, which
// is exactly what lane l already holds.  V is therefore stored TRANSPOSED in
// LDS ([d][key]) with bits 2 and 3 of the key position swapped, so every
// A operand of the P.V product is one 16-byte LDS read.
//
// fp32 inputs use v_mfma_f32_32x32x2_f32 with the same output layout (one
// element per lane per operand, so K and V stay row-major in LDS and P stays
// fp32); only the operand plumbing differs, the tile loop, masking,
// softmax and finalisation are shared.
//
// Masking: keys at or past the sequence end score -inf (the pages fill
// padded key rows with zeros, which would give them score 0; the definition
// sums over real keys only), and in causal mode key j > query i scores -inf
// ("Mini FlashAttention", section 1).  Tiles entirely above a wave's
// diagonal are skipped.  The running max is replaced by 0 whenever it is
// still -inf before it is used as the exponent shift, the ghost-row guard of
// "Mini FlashAttention", section 4, so no row can produce NaN; query rows
// past the sequence end compute on zeros and are never stored.
//
// Work order: workgroups are dispatched round-robin over the 8 XCDs of the
// chip (hardware id i runs on XCD i % 8).  The id is remapped so that each
// XCD receives a contiguous range of logical tiles, i.e. all query tiles of
// a (sequence, head) share one XCD and its L2, which then serves their
// repeated K/V reads.  Within a head, causal tiles are issued heaviest
// (last rows, most keys) first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_launch.h"

namespace fa355 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kWaves = kBlockM / 32;
constexpr int kThreads = kWave * kWaves;
constexpr int kXcds = 8;

// Key (row of the 32 x 32 output block) held in accumulator register r by
// a lane of half h = lane / 32.
__device__ __forceinline__ int block_key(int r, int h) {
  return 8 * (r >> 2) + 4 * h + (r & 3);
}

// Hardware workgroup id -> logical id such that each XCD gets one
// contiguous logical range (a bijection on [0, grid)).
__device__ __forceinline__ int xcd_remap(int i, int grid) {
  const int q = grid / kXcds, r = grid % kXcds;
  const int x = i % kXcds, k = i / kXcds;
  return x * q + (x < r ? x : r) + k;
}

__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// ---------------------------------------------------------------------------
// bf16 operand plumbing.  BN = 64 keys per tile.
//   LDS stage: K [BN][D + 8] row-major, V^T [D][BN + 8] with swapped key
//   bits 2 and 3 (see the file header).  The +8 pads break bank conflicts
//   between the 32 rows one 16-byte operand read touches.
// ---------------------------------------------------------------------------
template <int D>
struct Bf16Path {
  static constexpr int BN = 64;
  static constexpr int KSTR = D + 8;
  static constexpr int VSTR = BN + 8;
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int STAGE_BYTES = (BN * KSTR + D * VSTR) * 2;
  static constexpr int CHUNKS = BN * D / 8 / kThreads;  // 16-byte K chunks per thread
  static constexpr int KPT = CHUNKS;                    // V keys per thread (x 8 dims)
  static_assert(KPT == 2 || KPT == 4, "unsupported tile shape");

  struct QRegs { bf16x8_t q[D / 16]; };
  struct Regs { u32x4_t k[CHUNKS]; u32x4_t v[KPT]; };

  // Q^T as the B operand: lane holds query `row`, dims 16c + 8h .. +7.
  static __device__ __forceinline__ void load_q(QRegs &qr, const uint16_t *qb,
                                                long long rs, int row, int n, int h) {
    const uint16_t *p = qb + (long long)row * rs + 8 * h;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (row < n) x = *reinterpret_cast<const u32x4_t *>(p + 16 * c);
      qr.q[c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // Global -> registers for the tile starting at key0; keys >= n read as 0.
  static __device__ __forceinline__ void gload(Regs &rg, const uint16_t *kb,
                                               const uint16_t *vb, long long rs,
                                               int key0, int n, int tid) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = key0 + row;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (key < n) x = *reinterpret_cast<const u32x4_t *>(kb + (long long)key * rs + col);
      rg.k[i] = x;
    }
    const int dch = tid % (D / 8), kg = tid / (D / 8);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int key = key0 + kg * KPT + j;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (key < n) x = *reinterpret_cast<const u32x4_t *>(vb + (long long)key * rs + dch * 8);
      rg.v[j] = x;
    }
  }

  // Registers -> LDS stage.  K row-major; V transposed with the key
  // permutation pos(key) = key with bits 2 and 3 swapped.
  static __device__ __forceinline__ void lstore(const Regs &rg, char *stage, int tid) {
    uint16_t *lk = reinterpret_cast<uint16_t *>(stage);
    uint16_t *lv = lk + K_ELEMS;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4_t *>(lk + row * KSTR + col) = rg.k[i];
    }
    const int dch = tid % (D / 8), kg = tid / (D / 8);
    const int key = kg * KPT;
    const int pos = (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint16_t *dst = lv + (dch * 8 + e) * VSTR + pos;
      if constexpr (KPT == 4) {
        u32x2_t w;
        w[0] = __builtin_amdgcn_perm(rg.v[1][e >> 1], rg.v[0][e >> 1], sel);
        w[1] = __builtin_amdgcn_perm(rg.v[3][e >> 1], rg.v[2][e >> 1], sel);
        *reinterpret_cast<u32x2_t *>(dst) = w;
      } else {
        *reinterpret_cast<uint32_t *>(dst) =
            __builtin_amdgcn_perm(rg.v[1][e >> 1], rg.v[0][e >> 1], sel);
      }
    }
  }

  // S^T (two 32-key blocks) = K . Q^T, fp32.
  static __device__ __forceinline__ void scores(f32x16_t (&s)[2], const char *stage,
                                                const QRegs &qr, int l32, int h) {
    const uint16_t *lk = reinterpret_cast<const uint16_t *>(stage);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t acc = {};
      const uint16_t *kr = lk + (32 * kb + l32) * KSTR + 8 * h;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(kr + 16 * c);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr.q[c], acc, 0, 0, 0);
      }
      s[kb] = acc;
    }
  }

  // O^T += V^T . P^T with P (already exponentiated) rounded to bf16.
  static __device__ __forceinline__ void pv(f32x16_t (&o)[D / 32], const f32x16_t (&p)[2],
                                            const char *stage, int l32, int h) {
    const uint16_t *lv = reinterpret_cast<const uint16_t *>(stage) + K_ELEMS;
    bf16x8_t pb[BN / 16];
#pragma unroll
    for (int c = 0; c < BN / 16; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[c][e] = (__bf16)p[c >> 1][8 * (c & 1) + e];
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint16_t *vr = lv + (32 * db + l32) * VSTR + 8 * h;
#pragma unroll
      for (int c = 0; c < BN / 16; ++c) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(vr + 16 * c);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], o[db], 0, 0, 0);
      }
    }
  }

  // Four consecutive output dims d0..d0+3 of one row.
  static __device__ __forceinline__ void store4(uint16_t *dst, float a, float b, float c,
                                                float d) {
    bf16x4_t x = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    *reinterpret_cast<bf16x4_t *>(dst) = x;
  }
};

// ---------------------------------------------------------------------------
// fp32 operand plumbing.  BN = 32 keys per tile, K and V row-major in LDS.
// v_mfma_f32_32x32x2_f32: lane l holds A[l % 32][l / 32] and B[l / 32][l % 32].
// ---------------------------------------------------------------------------
template <int D>
struct F32Path {
  static constexpr int BN = 32;
  static constexpr int KSTR = D + 4;
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int STAGE_BYTES = 2 * BN * KSTR * 4;
  static constexpr int CHUNKS = BN * D / 4 / kThreads;  // 16-byte chunks per thread, per tensor

  struct QRegs { float q[D / 2]; };
  struct Regs { u32x4_t k[CHUNKS]; u32x4_t v[CHUNKS]; };

  static __device__ __forceinline__ void load_q(QRegs &qr, const float *qb, long long rs,
                                                int row, int n, int h) {
    const float *p = qb + (long long)row * rs + h;
#pragma unroll
    for (int t = 0; t < D / 2; ++t) qr.q[t] = row < n ? p[2 * t] : 0.f;
  }

  static __device__ __forceinline__ void gload(Regs &rg, const float *kb, const float *vb,
                                               long long rs, int key0, int n, int tid) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 4), col = (c % (D / 4)) * 4;
      const int key = key0 + row;
      u32x4_t x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (key < n) {
        x = *reinterpret_cast<const u32x4_t *>(kb + (long long)key * rs + col);
        y = *reinterpret_cast<const u32x4_t *>(vb + (long long)key * rs + col);
      }
      rg.k[i] = x;
      rg.v[i] = y;
    }
  }

  static __device__ __forceinline__ void lstore(const Regs &rg, char *stage, int tid) {
    float *lk = reinterpret_cast<float *>(stage);
    float *lv = lk + K_ELEMS;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 4), col = (c % (D / 4)) * 4;
      *reinterpret_cast<u32x4_t *>(lk + row * KSTR + col) = rg.k[i];
      *reinterpret_cast<u32x4_t *>(lv + row * KSTR + col) = rg.v[i];
    }
  }

  static __device__ __forceinline__ void scores(f32x16_t (&s)[1], const char *stage,
                                                const QRegs &qr, int l32, int h) {
    const float *kr = reinterpret_cast<const float *>(stage) + l32 * KSTR + h;
    f32x16_t acc = {};
#pragma unroll
    for (int t = 0; t < D / 2; ++t)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[2 * t], qr.q[t], acc, 0, 0, 0);
    s[0] = acc;
  }

  static __device__ __forceinline__ void pv(f32x16_t (&o)[D / 32], const f32x16_t (&p)[1],
                                            const char *stage, int l32, int h) {
    const float *lv = reinterpret_cast<const float *>(stage) + K_ELEMS;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float a = lv[block_key(r, h) * KSTR + 32 * db + l32];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[0][r], o[db], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void store4(float *dst, float a, float b, float c, float d) {
    f32x4_t x = {a, b, c, d};
    *reinterpret_cast<f32x4_t *>(dst) = x;
  }
};

template <class T> struct PathFor;
template <> struct PathFor<uint16_t> { template <int D> using type = Bf16Path<D>; };
template <> struct PathFor<float> { template <int D> using type = F32Path<D>; };

// ---------------------------------------------------------------------------
// The forward kernel.
// ---------------------------------------------------------------------------
template <class T, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_kernel(const FwdArgs a) {
  using P = typename PathFor<T>::template type<D>;
  constexpr int BN = P::BN;
  constexpr int KB = BN / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * P::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // --- work decomposition: (sequence, head, query tile) -------------------
  const int L = xcd_remap(blockIdx.x, a.grid);
  const int bh = L / a.n_qtiles;
  const int qt = a.n_qtiles - 1 - (L - bh * a.n_qtiles);  // heaviest first
  const int s = bh / a.H;
  const int hd = bh - s * a.H;
  int n;
  long long base, lbase;
  if constexpr (VARLEN) {
    const int t0 = a.cu_seqlens[s];
    n = a.cu_seqlens[s + 1] - t0;
    base = (long long)t0 * a.row_stride;
    lbase = (long long)t0 * a.lse_row_stride;
  } else {
    n = a.n;
    base = (long long)s * a.seq_stride;
    lbase = (long long)s * a.lse_seq_stride;
  }
  base += (long long)hd * a.head_stride;
  lbase += (long long)hd * a.lse_head_stride;

  const int m0 = qt * kBlockM;
  if (m0 >= n) return;  // uniform over the workgroup, before any barrier

  const T *qb = reinterpret_cast<const T *>(a.q) + base;
  const T *kb = reinterpret_cast<const T *>(a.k) + base;
  const T *vb = reinterpret_cast<const T *>(a.v) + base;
  const long long rs = a.row_stride;

  const int n_kv = CAUSAL ? (n < m0 + kBlockM ? n : m0 + kBlockM) : n;
  const int nt = (n_kv + BN - 1) / BN;
  const int qw0 = m0 + 32 * wv;  // first query row of this wave
  const int qrow = qw0 + l32;    // this lane's query row
  const bool wave_live = qw0 < n;

  // --- initialise: resident Q, m = -inf, l = 0, O = 0 -----------------------
  typename P::QRegs qr;
  P::load_q(qr, qb, rs, qrow, n, h);
  float m_run = -__builtin_huge_valf();
  float l_run = 0.f;  // this lane's partial row sum (its half of the keys)
  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
  const float sl2 = a.scale_log2;

  typename P::Regs rg;
  P::gload(rg, kb, vb, rs, 0, n, tid);
  P::lstore(rg, smem, tid);

  // --- main loop over K/V tiles --------------------------------------------
  for (int kt = 0; kt < nt; ++kt) {
    const bool more = kt + 1 < nt;
    if (more) P::gload(rg, kb, vb, rs, (kt + 1) * BN, n, tid);
    __syncthreads();
    const char *stage = smem + (kt & 1) * P::STAGE_BYTES;
    const int key0 = kt * BN;
    const bool active = wave_live && (!CAUSAL || key0 <= qw0 + 31);
    if (active) {
      f32x16_t sc[KB];
      P::scores(sc, stage, qr, l32, h);

      // mask keys past the end and, in causal mode, keys after the query
      const bool need_mask = (key0 + BN > n) || (CAUSAL && key0 + BN - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * b + block_key(r, h);
            const bool ok = key < n && (!CAUSAL || key <= qrow);
            if (!ok) sc[b][r] = -__builtin_huge_valf();
          }
      }

      // online softmax: row max over this tile (in-lane, then lane ^ 32)
      float mx = sc[0][0];
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[b][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_ref = (m_new == -__builtin_huge_valf()) ? 0.f : m_new;  // ghost-row guard
      const float alpha = exp2_fast((m_run - m_ref) * sl2);
      const float mb = m_ref * sl2;
      float ps = 0.f;
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(__builtin_fmaf(sc[b][r], sl2, -mb));
          sc[b][r] = p;
          ps += p;
        }
      l_run = l_run * alpha + ps;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;

      P::pv(o, sc, stage, l32, h);
    }
    if (more) P::lstore(rg, smem + ((kt + 1) & 1) * P::STAGE_BYTES, tid);
  }

  // --- finalise: O / l, lse = scale * m + ln l --------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < n) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *orow = reinterpret_cast<T *>(a.o) + base + (long long)qrow * rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        P::store4(orow + 32 * db + 8 * g + 4 * h, o[db][4 * g] * inv, o[db][4 * g + 1] * inv,
                  o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
    if (a.lse != nullptr && h == 0) {
      const float m_fin = (m_run == -__builtin_huge_valf()) ? 0.f : m_run;
      a.lse[lbase + (long long)qrow * a.lse_row_stride] =
          l_tot > 0.f ? m_fin * a.scale + __logf(l_tot) : -__builtin_huge_valf();
    }
  }
}

template <class T, int D, bool CAUSAL, bool VARLEN>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL, VARLEN>), dim3(a.grid), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch_d(const FwdArgs &a, bool causal, bool varlen, hipStream_t stream) {
  if (causal)
    return varlen ? launch<T, D, true, true>(a, stream) : launch<T, D, true, false>(a, stream);
  return varlen ? launch<T, D, false, true>(a, stream) : launch<T, D, false, false>(a, stream);
}

template <class T>
hipError_t launch_t(const FwdArgs &a, int d, bool causal, bool varlen, hipStream_t stream) {
  if (d == 64) return launch_d<T, 64>(a, causal, varlen, stream);
  if (d == 128) return launch_d<T, 128>(a, causal, varlen, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, int dtype, int d, bool causal, bool varlen,
                      hipStream_t stream) {
  if (dtype == 0) return launch_t<float>(a, d, causal, varlen, stream);
  if (dtype == 1) return launch_t<uint16_t>(a, d, causal, varlen, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa355
