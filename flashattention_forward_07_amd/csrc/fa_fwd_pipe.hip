// fa_fwd_pipe.hip -- attention forward for bf16 inputs at d = 128 on gfx950
// (MI355X): one wave per SIMD, each feeding the matrix core from its own
// instruction stream.
//
// The method is the resident-query flash loop of "Mini FlashAttention",
// section 4, in the initialise / loop / finalise structure of the grasp.study
// lesson "The Complete Kernel: Initialization, Loop, and Finalization": per
// query row a running exponent reference m, denominator l and fp32 output
// accumulator O; each 64-key K/V tile gives scores S, the state is rescaled
// by exp(m_old - m_new) when the reference moves, P = exp(S - m) is added
// into l and P.V into O, and O is divided once at the end.  The N x N scores
// never leave registers.
//
// Workgroup: 4 wave64s, one per SIMD, 256 query rows.  Wave w owns rows
// 64w .. 64w + 63 as two 32-row blocks, a and b, that move through the key
// tiles together, so every K or V operand read from LDS feeds the products of
// both blocks.  Iteration t is one software-pipelined body:
//   matrix core:  O += P(t-1) V(t-1)   (40 products, 8 of them row sums)
//                 S(t+1) = K(t+1) Q^T  (32 products)
//   vector ALU:   the softmax of S(t) into P(t), spread over the same slots
// One product per slot.  A product's operand reads go out right behind the
// product issued before it, and the vector work is spread over all 72 slots.
// The scores live in two register sets, even tiles in set 0 and odd tiles in
// set 1 (the loop runs two bodies per trip), so S(t+1) never overwrites the
// S(t) that the same body is still turning into weights.  P(t) reuses the
// registers of P(t-1): a 16-key chunk of P(t) is written only after the
// products that read that chunk of P(t-1).
//
// A single wave per SIMD issues everything in order, so the body's length is
// set by its instruction count as much as by the matrix core: the loop keeps
// scalar work (staging addresses, edge tests) out of the body where it can.
//
// Lazy rescaling, decided before any weight is formed: the lane's max of the
// raw scores is compared with the largest score the current reference lets
// through with every weight <= 2^52.  Only when some lane is over does the
// wave rebase (row maxima, a reference 48 above them in the exp2 domain, l
// scaled at once, O and the row sums scaled after the body's P.V products,
// which still add weights of the old reference).  The weights are then formed
// once, against the final reference.  The first tile always rebases (there
// is no reference yet).  In exact arithmetic the reference cancels in O / l.
// The bound leaves fp32 room: at most 2^31 weights of at most 2^52 sum below
// 2^83, and O stays finite while every |v| is below 2^45.  A wider bound
// means fewer rebases where the scores spread over many log2 units (2^32 ran
// packed Q, K x 8 inputs 3 % slower), but margin plus bound must stay at or
// below 102: a rebase's factor 2^(g_old - g_new) flushes to zero once the
// references differ by more than 126, and the old weights it then drops lie
// below 2^(margin + bound - 126) of the new row max, which must stay under
// 2^-24 (the fp32 rounding of the sums).  Margin 48 with bound 64 could drop
// terms of 2^-14; 56 + 64 and 48 + 80 measurably lost dominant terms.
//
// Registers: the two score sets and P of both blocks in VGPRs; O (2 x 64) and the
// rounded-weight row sums (2 x 4) in AGPRs; the resident Q (2 x 32) and the
// LDS operands in fixed AGPRs named by the inline v_mfma instructions that
// use them.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16): the score block is
// S^T = K Q^T, one query per lane and 16 keys of each 32-key block per lane
// half; its bf16 rounding is directly the B operand of O^T += V^T P^T.
//
// Row sums: l, for lse, is the fp32 sum of the weights (per lane, then with
// lane ^ 32).  O is divided by the sum of the bf16-rounded weights the P.V
// products used, so each row is an exact convex combination of V rows
// whatever the rounding of a dominant weight.  That sum comes from the matrix
// core: a product with an all-ones A operand and a P^T chunk adds the chunk's
// rounded weights of each query into every row of a 32 x 32 accumulator.
//
// LDS: a 4-stage ring of K/V tiles, row-major with XOR-swizzled 16-byte
// chunks, filled by direct global->LDS buffer loads (each wave moves a quarter
// of a tile); the four K tiles fill the lower 64 KB and the four V tiles the
// upper.  After the barrier that opens iteration t, the K tile t+1 and the V
// tiles up to t have landed and tile t-2's stage is free; the loads of tile
// t+2 go out early in the body, K before V.  The loop runs four bodies per
// trip, so each body's stages are compile-time constants that ride in the
// immediate offsets of its operand reads.  The workgroup's query rows come in
// the same way, through stages 2 and 3 before the ring first uses them, and
// are read from there into the Q^T AGPRs.
//
// Masking: keys past the sequence end and (causal) keys after the query score
// -inf ("Mini FlashAttention", section 1); a -inf reference is replaced by 0
// before use (the ghost-row guard of section 4).  Query rows past the end
// compute on zeros and are never stored.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_bf16_tile.h"
#include "fa_common.h"
#include "fa_fwd_launch.h"

namespace fa355 {
namespace {

using namespace bf16t;

constexpr int kPWaves = 4;
constexpr int kPThreads = kWave * kPWaves;  // 256
constexpr int kPBlockM = 64 * kPWaves;      // 256 query rows per workgroup
constexpr int kPStages = 4;
constexpr int kPD = 128;
constexpr int kPBN = 64;
using PT = Bf16Tile<kPD, kPBN>;
constexpr int kPLds = kPStages * PT::STAGE;         // 128 KB
// LDS: the K tile of stage s at s TILE, the V tile at kPVBase + s TILE, so
// that any operand of a stage known at compile time sits within the 16-bit
// offset of a ds_read from a fixed per-lane address
constexpr int kPVBase = kPStages * PT::TILE;
constexpr int kPDpw = PT::TILE / (1024 * kPWaves);  // staging loads per wave per tensor: 4
constexpr float kPMargin = 48.f;     // a new reference sits this far above the row max (log2)
constexpr float kPBoundLog2 = 52.f;  // the fast path keeps every weight <= 2^52
static_assert(kPMargin + kPBoundLog2 <= 102.f, "a rebase may drop terms above 2^-24 of the row max");
static_assert(kPDpw == 4, "staging split");

// One 32-row query block of a wave (BLK 0 = a, 1 = b: which AGPRs it owns).
template <int BLK>
struct QBlock {
  static constexpr int kBlk = BLK;
  bf16x8_t q[kPD / 16];  // Q^T operand: Q[row][16c + 8h .. +7] (AGPRs)
  f32x16_t s[2][2];      // S^T of two tiles (set, 32-key block) (VGPRs)
  bf16x8_t p[4];         // P^T, four 16-key chunks (VGPRs)
  f32x16_t o[kPD / 32];  // O^T accumulator (AGPRs)
  f32x4_t lr;            // rounded-weight row sums (AGPRs), see mfma_ones
  float mbl;             // exponent reference, exp2 domain; -inf: none yet
  float g;               // the reference as subtracted (0 while there is none)
  float lim;             // largest raw score the fast path lets through
  float alpha;           // rescale factor of the current body's rebase
  float l;               // this lane's half of the fp32 row sum
  int q0;                // first query row of the block
};

template <int I, class A, class B>
__device__ __forceinline__ auto &pick(A &a, B &b) {
  if constexpr (I == 0)
    return a;
  else
    return b;
}

// The accumulators (O^T and the row sums) are AGPR operands of the inline
// products, placed by the compiler.  The LDS operands of the products go to
// fixed AGPRs, read there directly by the matrix core: V^T ring entry e in
// a224 + 4e .. +3, K ring entry e in a240 + 4e .. +3.
template <int BLK, int DB, int E, int W>
__device__ __forceinline__ void mfma_pv(f32x16_t &acc, const u32x4_t &v, const bf16x8_t p) {
  static_assert(BLK == 0 || BLK == 1, "block");
  static_assert(DB >= 0 && DB < 4 && E >= 0 && E < 4, "accumulator / ring entry");
  // W >= 0: the operand's LDS reads are awaited (lgkmcnt(W)) in the same
  // statement, right before the product.  As two statements the compiler
  // would see an opaque write of the ring registers followed by a read and
  // put a wait state between them.
#define FA_PV_E(E_, VREGS)                                                               \
  if constexpr (E == E_) {                                                               \
    if constexpr (W >= 0)                                                                \
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"    \
                   : "+a"(acc) : "{" VREGS "}"(v), "v"(p), "i"(W));                      \
    else                                                                                 \
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc)                 \
                   : "{" VREGS "}"(v), "v"(p));                                          \
  }
  FA_PV_E(0, "a[224:227]")
  FA_PV_E(1, "a[228:231]")
  FA_PV_E(2, "a[232:235]")
  FA_PV_E(3, "a[236:239]")
#undef FA_PV_E
}
// Row sums of the rounded weights: v_mfma_f32_16x16x32_bf16 with a 0/1
// pattern as A and a P^T chunk as B.  Read as the B operand of that shape,
// lane l's eight weights are column l % 16, k-block l / 16 (0 .. 3); block g
// belongs to query 16 (g % 2) + l % 16 (keys of lane half g / 2).  Row m of A
// is 1 on the k-blocks of parity m / 8, so output row m < 8 of column n is
// query n's sum of the chunk and row m >= 8 query 16 + n's.  Lane l holds
// output rows 4 (l / 16) .. +3 of column l % 16: the sum of query
// 16 (l / 32) + l % 16, which lanes 16..31 and 32..47 exchange at the end.
__device__ __forceinline__ void mfma_ones(f32x4_t &acc, const bf16x8_t sel, const bf16x8_t p) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(sel), "v"(p));
}

// The resident Q^T of block a sits in a128..a159, of block b in a160..a191
// (chunk c in the 4 registers from 128 + 32 BLK + 4c); S^T = K Q^T lands in
// VGPRs.  C0: first product of a chain (zero accumulator).
template <int BLK, int C, bool C0, int E, int W>
__device__ __forceinline__ void mfma_s(f32x16_t &acc, const u32x4_t &k, const bf16x8_t &q) {
  static_assert(BLK == 0 || BLK == 1, "block");
  static_assert(C >= 0 && C < 8 && E >= 0 && E < 4, "chunk / ring entry");
#define FA_S_E(QREGS, E_, KREGS)                                                                  \
  if constexpr (E == E_) {                                                                        \
    if constexpr (C0 && W >= 0)                                                                   \
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"             \
                   : "=v"(acc) : "{" KREGS "}"(k), "{" QREGS "}"(q), "i"(W));                     \
    else if constexpr (C0)                                                                        \
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc)                          \
                   : "{" KREGS "}"(k), "{" QREGS "}"(q));                                         \
    else if constexpr (W >= 0)                                                                    \
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"            \
                   : "+v"(acc) : "{" KREGS "}"(k), "{" QREGS "}"(q), "i"(W));                     \
    else                                                                                          \
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc)                         \
                   : "{" KREGS "}"(k), "{" QREGS "}"(q));                                         \
  }
#define FA_S_CASE(B_, C_, QREGS)                                                                  \
  if constexpr (BLK == B_ && C == C_) {                                                           \
    FA_S_E(QREGS, 0, "a[240:243]")                                                                \
    FA_S_E(QREGS, 1, "a[244:247]")                                                                \
    FA_S_E(QREGS, 2, "a[248:251]")                                                                \
    FA_S_E(QREGS, 3, "a[252:255]")                                                                \
  }
  FA_S_CASE(0, 0, "a[128:131]")
  FA_S_CASE(0, 1, "a[132:135]")
  FA_S_CASE(0, 2, "a[136:139]")
  FA_S_CASE(0, 3, "a[140:143]")
  FA_S_CASE(0, 4, "a[144:147]")
  FA_S_CASE(0, 5, "a[148:151]")
  FA_S_CASE(0, 6, "a[152:155]")
  FA_S_CASE(0, 7, "a[156:159]")
  FA_S_CASE(1, 0, "a[160:163]")
  FA_S_CASE(1, 1, "a[164:167]")
  FA_S_CASE(1, 2, "a[168:171]")
  FA_S_CASE(1, 3, "a[172:175]")
  FA_S_CASE(1, 4, "a[176:179]")
  FA_S_CASE(1, 5, "a[180:183]")
  FA_S_CASE(1, 6, "a[184:187]")
  FA_S_CASE(1, 7, "a[188:191]")
#undef FA_S_CASE
#undef FA_S_E
}

// LDS operand reads into the ring AGPRs (each product that first reads an
// entry awaits it in its own statement, see mfma_pv).  A V^T operand is
// two transposing reads of four key rows each (rows 16c + 4h + e4 and 8
// below), a K operand one 16-byte read.
template <int E, int OFF0, int OFF1>
__device__ __forceinline__ void lds_read_v(u32x4_t &d, uint32_t addr) {
  static_assert(OFF0 >= 0 && OFF1 < 65536, "ds offset");
#define FA_RV(E_, LO, HI, ALL)                                                                   \
  if constexpr (E == E_)                                                                          \
    asm volatile("ds_read_b64_tr_b16 " LO ", %1 offset:%2\n\tds_read_b64_tr_b16 " HI             \
                 ", %1 offset:%3"                                                                 \
                 : "={" ALL "}"(d)                                                                \
                 : "v"(addr), "i"(OFF0), "i"(OFF1));
  FA_RV(0, "a[224:225]", "a[226:227]", "a[224:227]")
  FA_RV(1, "a[228:229]", "a[230:231]", "a[228:231]")
  FA_RV(2, "a[232:233]", "a[234:235]", "a[232:235]")
  FA_RV(3, "a[236:237]", "a[238:239]", "a[236:239]")
#undef FA_RV
}
template <int E, int OFF>
__device__ __forceinline__ void lds_read_k(u32x4_t &d, uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
#define FA_RK(E_, ALL) \
  if constexpr (E == E_) asm volatile("ds_read_b128 %0, %1 offset:%2" : "={" ALL "}"(d) : "v"(addr), "i"(OFF));
  FA_RK(0, "a[240:243]")
  FA_RK(1, "a[244:247]")
  FA_RK(2, "a[248:251]")
  FA_RK(3, "a[252:255]")
#undef FA_RK
}
// Q^T chunks of a block from LDS (laid out as a K tile) into their AGPRs;
// q_settle awaits them.
template <int BLK, class QB>
__device__ __forceinline__ void q_read(QB &x, uint32_t base, const uint32_t *ofs) {
#define FA_RQ(C_, ALL)                                                                  \
  asm volatile("ds_read_b128 %0, %1" : "={" ALL "}"(x.q[C_]) : "v"(base + ofs[C_]));
  if constexpr (BLK == 0) {
    FA_RQ(0, "a[128:131]") FA_RQ(1, "a[132:135]") FA_RQ(2, "a[136:139]") FA_RQ(3, "a[140:143]")
    FA_RQ(4, "a[144:147]") FA_RQ(5, "a[148:151]") FA_RQ(6, "a[152:155]") FA_RQ(7, "a[156:159]")
  } else {
    FA_RQ(0, "a[160:163]") FA_RQ(1, "a[164:167]") FA_RQ(2, "a[168:171]") FA_RQ(3, "a[172:175]")
    FA_RQ(4, "a[176:179]") FA_RQ(5, "a[180:183]") FA_RQ(6, "a[184:187]") FA_RQ(7, "a[188:191]")
  }
#undef FA_RQ
}
template <int BLK, class QB>
__device__ __forceinline__ void q_settle(QB &x) {
  // after the Q^T chunks are written to their AGPRs: wait states before a
  // product reads them
  if constexpr (BLK == 0)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 4"
                 : "+{a[128:131]}"(x.q[0]), "+{a[132:135]}"(x.q[1]), "+{a[136:139]}"(x.q[2]),
                   "+{a[140:143]}"(x.q[3]), "+{a[144:147]}"(x.q[4]), "+{a[148:151]}"(x.q[5]),
                   "+{a[152:155]}"(x.q[6]), "+{a[156:159]}"(x.q[7]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 4"
                 : "+{a[160:163]}"(x.q[0]), "+{a[164:167]}"(x.q[1]), "+{a[168:171]}"(x.q[2]),
                   "+{a[172:175]}"(x.q[3]), "+{a[176:179]}"(x.q[4]), "+{a[180:183]}"(x.q[5]),
                   "+{a[184:187]}"(x.q[6]), "+{a[188:191]}"(x.q[7]));
}

// Wait states between the last inline product that wrote a block's
// accumulators and vector reads or writes of them (the compiler does not see
// inline products as such); tied to the accumulators so no access moves above
// it.
template <class QB>
__device__ __forceinline__ void acc_settle(QB &x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(x.o[0]), "+a"(x.o[1]), "+a"(x.o[2]), "+a"(x.o[3]), "+a"(x.lr));
}
// alpha_lr: the factor of the query whose row sum this lane holds (see
// mfma_ones), which for lanes 16 .. 47 is not the lane's own query.
template <class QB>
__device__ __forceinline__ void acc_scale(QB &x, float alpha, float alpha_lr) {
  acc_settle(x);
#pragma unroll
  for (int db = 0; db < kPD / 32; ++db) x.o[db] *= alpha;
  x.lr *= alpha_lr;
}
// Maximum of eight values, and a running maximum carried on over eight
// more, each chain in one statement: the compiler puts a wait state after
// every inline vector instruction whose result the next one reads, and fmaxf
// on values it cannot prove canonical (these come from inline products) adds
// canonicalising maxima.
__device__ __forceinline__ float max8(float a, float b, float c, float d, float e, float f,
                                      float g, float h) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3\n\tv_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\tv_max_f32 %0, %0, %8"
      : "=&v"(r)
      : "v"(a), "v"(b), "v"(c), "v"(d), "v"(e), "v"(f), "v"(g), "v"(h));
  return r;
}
// The running maximum m carried on over eight more values: four v_max3.
__device__ __forceinline__ float max_on8(float m, float a, float b, float c, float d, float e,
                                         float f, float g, float h) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3\n\tv_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\tv_max3_f32 %0, %0, %8, %9"
      : "=&v"(r)
      : "v"(m), "v"(a), "v"(b), "v"(c), "v"(d), "v"(e), "v"(f), "v"(g), "v"(h));
  return r;
}

// Lane whose query's row sum lane `lane` holds, and vice versa (lanes 16..31
// and 32..47 trade): the partner in the 16x16 output layout of mfma_ones.
__device__ __forceinline__ int lr_partner(int lane) {
  return (((lane >> 4) ^ (lane >> 5)) & 1) ? (lane ^ 48) : lane;
}
__device__ __forceinline__ float lane_fetch(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * src, __builtin_bit_cast(int, v)));
}

// ---- the schedule of one body ------------------------------------------------
// The products in issue order, one per slot.  P.V phase: for each 16-key
// chunk c and 32-wide d block db, block a's then block b's product on the
// same V^T operand; after each chunk the two row-sum products.  Score phase:
// for each 32-key block kb and 16-wide d chunk c, block a's then block b's
// product on the same K operand.  The first product of a pair owns the
// operand's LDS reads.  Accumulator chains: an O block or a row sum recurs
// every 10 slots, a score block every 2 (an independent product between).
struct Slot {
  int kind;   // 0 P.V, 1 row sum, 2 score
  int blk;    // 0 = a, 1 = b
  int c;      // P chunk (P.V, row sum) or d chunk (score)
  int x;      // db (P.V) or kb (score)
  int reads;  // LDS reads the slot's operand needs (0 for the second of a pair)
  int op;     // operand number within its kind: 4c + db (V^T) or 8kb + c (K)
};
constexpr int kPvSlots = 40, kScoreSlots = 32;
template <bool PV, bool S>
struct BodySchedule {
  static constexpr int N = (PV ? kPvSlots : 0) + (S ? kScoreSlots : 0);
  Slot slot[N];
  int reads_before[N + 1];  // operand reads of slots 0 .. s-1
  constexpr BodySchedule() : slot{}, reads_before{} {
    int n = 0;
    if (PV)
      for (int c = 0; c < 4; ++c) {
        for (int db = 0; db < 4; ++db) {
          slot[n++] = Slot{0, 0, c, db, 2, 4 * c + db};
          slot[n++] = Slot{0, 1, c, db, 0, 4 * c + db};
        }
        slot[n++] = Slot{1, 0, c, 0, 0, 0};
        slot[n++] = Slot{1, 1, c, 0, 0, 0};
      }
    if (S)
      for (int kb = 0; kb < 2; ++kb)
        for (int c = 0; c < 8; ++c) {
          slot[n++] = Slot{2, 0, c, kb, 1, 8 * kb + c};
          slot[n++] = Slot{2, 1, c, kb, 0, 8 * kb + c};
        }
    reads_before[0] = 0;
    for (int k = 0; k < N; ++k) reads_before[k + 1] = reads_before[k] + slot[k].reads;
  }
};

// Slots whose operand reads are in flight ahead of the current product.
#ifndef FA_PIPE_READ_AHEAD
#define FA_PIPE_READ_AHEAD 6
#endif
constexpr int kPReadAhead = FA_PIPE_READ_AHEAD;
// Operand waits of a body, per slot (-1: none).  A product that first reads
// an operand waits for its reads; each such wait also covers the operands of
// the next kPWaitGroup - 1 owners whose reads have gone out by then (they
// went out kPReadAhead slots ahead of their own products), so one s_waitcnt
// serves several operands.  The reads issued before slot k's product are
// those of the slots before k + kPReadAhead.
#ifndef FA_PIPE_WAIT_GROUP
#define FA_PIPE_WAIT_GROUP 2
#endif
constexpr int kPWaitGroup = FA_PIPE_WAIT_GROUP;
template <bool PV, bool S>
struct BodyWaits {
  static constexpr int N = BodySchedule<PV, S>::N;
  int w[N];
  constexpr BodyWaits() : w{} {
    constexpr BodySchedule<PV, S> bs{};
    int owners[N] = {};
    int no = 0;
    for (int k = 0; k < N; ++k) {
      w[k] = -1;
      if (bs.slot[k].reads > 0) owners[no++] = k;
    }
    for (int o = 0; o < no;) {
      const int k = owners[o];
      const int hi = k + kPReadAhead < N ? k + kPReadAhead : N;
      int g = 1;
      while (g < kPWaitGroup && o + g < no && owners[o + g] < hi) ++g;
      const int covered = owners[o + g - 1];
      w[k] = bs.reads_before[hi] - bs.reads_before[covered + 1];
      o += g;
    }
  }
};

// Ring entries for the operands of one kind: an operand is live from its
// reads (issued behind the product kPReadAhead slots before its first use)
// until its second use one slot after the first, so at most the owners of
// that kind among kPReadAhead + 2 consecutive slots are live at once.
template <bool PV, bool S>
constexpr int ring_size(int kind) {
  constexpr BodySchedule<PV, S> bs{};
  int best = 1;
  for (int k = 0; k < bs.N; ++k) {
    int c = 0;
    for (int j = k; j < k + kPReadAhead + 2 && j < bs.N; ++j)
      c += (bs.slot[j].kind == kind && bs.slot[j].reads > 0) ? 1 : 0;
    best = c > best ? c : best;
  }
  return best;
}

// The softmax of S(t) in a full body (72 slots).  Element pair u (0 .. 31)
// is pair u % 8 of the 32-key block kb = u / 16 of query block (u / 8) % 2;
// its two weights go to P chunk 2 kb + (u % 8) / 4.
//   slots 0 .. 7: the lane's max of the raw scores, an eighth of the
//                 elements per slot;
//   slot 8:       the rebase test (and the rebase, when taken);
//   then per pair: scale and subtract the reference, exp2 one slot later (in
//                 place), and later still the bf16 rounding into P and the
//                 add into l.
constexpr int sm_blk(int u) { return (u / 8) % 2; }
constexpr int sm_kb(int u) { return u / 16; }
constexpr int sm_chunk(int u) { return 2 * (u / 16) + (u % 8) / 4; }
// Slots behind which this wave's eight staging loads of tile t + 2 go out:
// the four K loads in the first half of the body (the next barrier waits for
// them), the four V loads in the second (they are read two bodies later).
// Spread out, the loads of the four waves do not queue up behind each other.
#ifndef FA_PIPE_DMA_K0
#define FA_PIPE_DMA_K0 1
#define FA_PIPE_DMA_KS 8
#define FA_PIPE_DMA_V0 33
#define FA_PIPE_DMA_VS 10
#endif
constexpr int dma_slot(int part) {
  return part < 4 ? FA_PIPE_DMA_K0 + FA_PIPE_DMA_KS * part
                  : FA_PIPE_DMA_V0 + FA_PIPE_DMA_VS * (part - 4);
}
static_assert(dma_slot(7) < kPvSlots + kScoreSlots, "staging slots");
constexpr int kSmTest = 8;
constexpr int sm_fma(int u) { return kSmTest + 1 + (u * 60) / 32; }
constexpr int sm_exp(int u) { return sm_fma(u) + 1; }
// chunk c of P(t-1) is last read by block b's row-sum product in slot 10c + 9
constexpr int sm_free(int c) { return 10 * c + 10; }
constexpr int sm_pack(int u) {
  int k = 0;
  for (int v = 0; v <= u; ++v) {
    int kv = sm_exp(v) + 1;
    if (kv < sm_free(sm_chunk(v))) kv = sm_free(sm_chunk(v));
    if (v > 0 && kv < k + 1) kv = k + 1;
    k = kv;
  }
  return k;
}
constexpr bool sm_schedule_ok() {
  for (int u = 0; u < 32; ++u) {
    if (sm_pack(u) <= sm_exp(u)) return false;
    if (sm_pack(u) < sm_free(sm_chunk(u))) return false;  // writes P(t) while P(t-1) is read
    if (sm_pack(u) >= kPvSlots + kScoreSlots) return false;
  }
  return sm_fma(0) > kSmTest;
}
static_assert(sm_schedule_ok(), "softmax schedule");

template <bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kPThreads, 1) void fa_fwd_bf16_pipe(const FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kPLds];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const TileCoords tc = tile_coords<VARLEN>(a, kPBlockM);
  const int n = tc.n, m0 = tc.m0;
  if (m0 >= n) return;  // uniform over the workgroup, before any barrier

  const uint16_t *qg = reinterpret_cast<const uint16_t *>(a.q) + tc.base;
  const uint16_t *kg = reinterpret_cast<const uint16_t *>(a.k) + tc.base;
  const uint16_t *vg = reinterpret_cast<const uint16_t *>(a.v) + tc.base;
  const long long rs = a.row_stride;

  const int n_kv = CAUSAL ? (n < m0 + kPBlockM ? n : m0 + kPBlockM) : n;
  const int T = (n_kv + kPBN - 1) / kPBN;  // K/V tiles of the workgroup
  const int q0 = m0 + 64 * w;              // first row of this wave (block a; b starts 32 later)
  // tiles this wave works on: causal, up to the one holding its diagonal
  // (q0 is a multiple of 64, so both blocks share it)
  int Tw = 0;
  if (q0 < n) Tw = CAUSAL ? (q0 / kPBN + 1 < T ? q0 / kPBN + 1 : T) : T;

  QBlock<0> A;
  QBlock<1> B;
  A.q0 = q0;
  B.q0 = q0 + 32;
  A.mbl = B.mbl = neg_inf();
  A.g = B.g = 0.f;
  A.lim = B.lim = neg_inf();  // the first tile always rebases
  A.alpha = B.alpha = 1.f;
  A.l = B.l = 0.f;

  // ---- K/V staging: global -> LDS directly --------------------------------
  // Load i of wave w fills the 1 KB of 16-byte slots p = (4w + i) * 64 + lane
  // (row p / 16, slot p % 16) of the K tile and of the V tile; each lane
  // fetches the logical chunk the swizzle places in its slot.
  uint32_t o_k[kPDpw], o_v[kPDpw];
  const uint32_t rsb = static_cast<uint32_t>(a.row_stride) * 2u;  // bytes per key row
#pragma unroll
  for (int i = 0; i < kPDpw; ++i) {
    const int p = (w * kPDpw + i) * kWave + lane;
    const int row = p / PT::CPR, slot = p % PT::CPR;
    o_k[i] = 16u * (slot ^ PT::swz_k(row)) + row * rsb;
    o_v[i] = 16u * (slot ^ PT::swz_v(row)) + row * rsb;
  }
  // Part i (0 .. 7) of this wave's share of tile t: load i / 2 of the K
  // tile (i even) or of the V tile (i odd), into stage st_t.  The loads are
  // raw buffer loads whose range ends with the tile's last valid key row, so
  // rows past the sequence end read as zeros (their scores are masked) and
  // the ragged last tile needs no separate path.
  auto dma_part = [&](int t, int st_t, int i) {
    const int key0 = t * kPBN;
    // rows of the tile inside the sequence; none for a tile past the last
    // (see dma_tile)
    const int valid = t >= T ? 0 : (n - key0 < kPBN ? n - key0 : kPBN);
    const uint16_t *src = ((i & 1) ? vg : kg) + (long long)key0 * rs;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(src), (short)0,
        valid > 0 ? (int)((valid - 1) * rsb + PT::ROWB) : 0, 0x00020000);
    const int j = i >> 1;
    char *st = smem + (st_t & (kPStages - 1)) * PT::TILE + ((i & 1) ? kPVBase : 0) +
               (w * kPDpw + j) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_LDS void *)st, 16,
                                             (i & 1) ? o_v[j] : o_k[j], 0, 0, 0);
  };
  // Tile t + 2 goes to stage (t + 2) % 4 during iteration t, its K loads
  // before its V loads (kv_part), early in the body: the K tile is read in
  // the next iteration, the V tile two after that, so each barrier waits
  // only for the K loads of the iteration before (and for everything older)
  // while the last four loads, V, may still fly.  Past the last tile the
  // loads still go out, with an empty range: they move no memory and only
  // write zeros into that stage, which holds nothing that is read again.
  // That keeps them unconditional inside the scheduled bodies.  Every load
  // is awaited before the workgroup ends (its LDS then passes to the next
  // workgroup on the compute unit).
  auto kv_part = [](int p) { return p < kPDpw ? 2 * p : 2 * (p - kPDpw) + 1; };
  // The same loads inside the loop, from state carried across the bodies
  // (tile t's source rows and byte range, advanced once per body) instead of
  // addresses recomputed from t for every load.
  const long long tile_elems = (long long)kPBN * rs;
  const int rec_full = (kPBN - 1) * (int)rsb + PT::ROWB;
  const int rec_last = T > 0 ? (n - (T - 1) * kPBN - 1) * (int)rsb + PT::ROWB : 0;
  struct DmaTile {
    const uint16_t *k, *v;  // first row of the tile in K and V
    int t;                  // tile index
    int rec;                // bytes of the tile inside the sequence (0 past the last)
  };
  auto dma_state = [&](int t) {
    DmaTile d;
    d.k = kg + t * tile_elems;
    d.v = vg + t * tile_elems;
    d.t = t;
    d.rec = t < T - 1 ? rec_full : (t == T - 1 ? rec_last : 0);
    return d;
  };
  auto dma_advance = [&](DmaTile &d) {
    d.k += tile_elems;
    d.v += tile_elems;
    d.t += 1;
    d.rec = d.t < T - 1 ? rec_full : (d.t == T - 1 ? rec_last : 0);
  };
  auto dma_part_at = [&](const DmaTile &d, int i) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>((i & 1) ? d.v : d.k), (short)0, d.rec, 0x00020000);
    const int j = i >> 1;
    char *st = smem + (d.t & (kPStages - 1)) * PT::TILE + ((i & 1) ? kPVBase : 0) +
               (w * kPDpw + j) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_LDS void *)st, 16,
                                             (i & 1) ? o_v[j] : o_k[j], 0, 0, 0);
  };
  auto dma_tile = [&](int t) {
#pragma unroll
    for (int p = 0; p < 2 * kPDpw; ++p) dma_part(t, t, kv_part(p));
  };

  // ---- LDS operand addresses (byte offsets within a stage) ----------------
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS char *)smem));
  // LDS addresses of this lane's operands in stage 0 (a stage s adds s TILE)
  uint32_t kofs[kPD / 16];  // K operand (kb, c): row 32 kb + l32, logical chunk 2c + h
  {
    const int sw = PT::swz_k(l32);
#pragma unroll
    for (int c = 0; c < kPD / 16; ++c) kofs[c] = lds_base + l32 * PT::ROWB + 16 * ((2 * c + h) ^ sw);
  }
  uint32_t vofs[kPD / 32];  // V^T operand (db, c): key row 16c (+8) + 4h + e4, d 32db + ...
  {
    const int j = lane & 15, e4 = j >> 2, gq = (lane >> 4) & 1;
    const int sw = PT::swz_v(e4);
#pragma unroll
    for (int db = 0; db < kPD / 32; ++db)
      vofs[db] = lds_base + kPVBase + (4 * h + e4) * PT::ROWB +
                 16 * ((4 * db + 2 * gq + ((j & 3) >> 1)) ^ sw) + 8 * (j & 1);
  }
  auto stage_off = [&](int t) { return static_cast<uint32_t>((t & (kPStages - 1)) * PT::TILE); };

  const float sl2 = a.scale_log2;
  const float inv_sl2 = 1.f / sl2;
  // row-sum selector (mfma_ones): 1.0 where k-block parity (lane / 16) % 2
  // matches output row (lane % 16) / 8, else 0
  const uint32_t sel_w = (((lane >> 4) & 1) == ((lane >> 3) & 1)) ? 0x3f803f80u : 0u;
  const u32x4_t sel4 = {sel_w, sel_w, sel_w, sel_w};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, sel4);

  // Keys past the end, and (causal) keys after the query, score -inf:
  // element (kb, r) of this lane holds key key0 + 4h + 32kb + 8(r / 4) + r % 4
  // (block_key); it is allowed while that offset stays <= lim, the lane's
  // last allowed key (the sequence end, and causal, its query) minus
  // key0 + 4h.  Each element is one compare into vcc and one select, issued
  // together so that no mask outlives its select.
  auto mask = [&](auto &x, auto sb_c, int key0) {
    constexpr int SB = decltype(sb_c)::value;
    int lim = n - 1;
    if constexpr (CAUSAL) lim = lim < x.q0 + l32 ? lim : x.q0 + l32;
    lim -= key0 + 4 * h;
    const float ninf = neg_inf();
    static_for<32>([&x, lim, ninf](auto E) {
      constexpr int kb = decltype(E)::value / 16, r = decltype(E)::value % 16;
      constexpr int off = 32 * kb + 8 * (r >> 2) + (r & 3);
      asm volatile("v_cmp_gt_i32 vcc, %1, %2\n\tv_cndmask_b32 %0, %0, %3, vcc"
                   : "+v"(x.s[SB][kb][r])
                   : "i"(off), "v"(lim), "v"(ninf)
                   : "vcc");
    });
  };
  // The rebase of one block for a lane max m of its raw scores.
  auto rebase = [&](auto &x, float m) {
    const float mrow = pair_max(m);
    const float mx = __builtin_fmaf(mrow, sl2, -x.g);  // the row max against the reference
    const bool bump = (x.mbl == neg_inf()) ? (mrow > neg_inf()) : (mx > 0.f);
    x.alpha = 1.f;
    if (bump) {
      const float mbl_new = x.g + mx + kPMargin;
      x.alpha = exp2_fast(x.mbl - mbl_new);  // 0 when there was no reference
      x.mbl = mbl_new;
      x.g = mbl_new;
      x.lim = (mbl_new + kPBoundLog2) * inv_sl2;
    }
    x.l *= x.alpha;
  };

  // First key tile (by its first key) that needs the mask: the one holding the
  // sequence end, or (causal) the wave's first query, whichever comes first;
  // key0 + 64 > n and key0 + 63 > q0 (both tile starts multiples of 64).
  const int edge_from = CAUSAL ? (n - (kPBN - 1) < A.q0 ? n - (kPBN - 1) : A.q0) : n - (kPBN - 1);

  // ---- one body --------------------------------------------------------------
  // PV: O += P V over the V tile at vbase; S: S = K Q^T over the K tile at
  // kbase; SM: the softmax of the scores of the tile at key0 (a full body
  // has all three and sends this wave's share of tile dma_t + 2).
  auto body = [&](auto pv_c, auto s_c, auto sm_c, auto sb_c, auto vs_c, auto ks_c, int key0,
                  uint32_t vbase, uint32_t kbase, const DmaTile &dn) {
    constexpr bool PV = decltype(pv_c)::value, S = decltype(s_c)::value,
                   SM = decltype(sm_c)::value;
    // the stages of the V and the K tile when known at compile time (their
    // offsets then ride in the ds_read immediates), else -1 and the stage
    // offsets vbase / kbase
    constexpr int VS = decltype(vs_c)::value, KS = decltype(ks_c)::value;
    constexpr int SB = decltype(sb_c)::value;  // S(t) in set SB, S(t+1) goes to set 1 - SB
    constexpr BodySchedule<PV, S> BS{};
    constexpr BodyWaits<PV, S> BW{};
    constexpr int N = BS.N;
    static_assert(!SM || (PV && S), "the softmax runs in full bodies only");
    constexpr int NRV = ring_size<PV, S>(0), NRK = ring_size<PV, S>(2);
    constexpr int RA = kPReadAhead;
    static_assert(NRV <= 4 && NRK <= 4, "ring entries");
    u32x4_t vr[NRV];  // V^T operand 4c + db in entry (4c + db) % NRV
    u32x4_t kr[NRK];  // K operand 8kb + c in entry (8kb + c) % NRK
    float mq[2];         // running maxima of the raw scores (block)
    float ps[2][4];      // partial fp32 sums of the weights
    int rescale = 0;  // the rebase ran (kept opaque below: see the end of the body)

    if constexpr (SM) {
      const bool edge = key0 >= edge_from;
      if (edge) {
        // these read the scores right after the products that wrote them:
        // wait states first, tied to them
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(A.s[SB][0]), "+v"(A.s[SB][1]), "+v"(B.s[SB][0]), "+v"(B.s[SB][1]));
        mask(A, sb_c, key0);
        mask(B, sb_c, key0);
      }
    }

    auto issue = [&](auto K) {
      constexpr int k = decltype(K)::value;
      if constexpr (k < N) {
        constexpr Slot sl = BS.slot[k];
        if constexpr (sl.kind == 0 && sl.reads > 0) {
          if constexpr (VS >= 0)
            lds_read_v<sl.op % NRV, VS * PT::TILE + 16 * sl.c * PT::ROWB,
                       VS * PT::TILE + (16 * sl.c + 8) * PT::ROWB>(vr[sl.op % NRV], vofs[sl.x]);
          else
            lds_read_v<sl.op % NRV, 16 * sl.c * PT::ROWB, (16 * sl.c + 8) * PT::ROWB>(
                vr[sl.op % NRV], vbase + vofs[sl.x]);
        } else if constexpr (sl.kind == 2 && sl.reads > 0) {
          if constexpr (KS >= 0)
            lds_read_k<sl.op % NRK, KS * PT::TILE + sl.x * 32 * PT::ROWB>(kr[sl.op % NRK],
                                                                        kofs[sl.c]);
          else
            lds_read_k<sl.op % NRK, sl.x * 32 * PT::ROWB>(kr[sl.op % NRK], kbase + kofs[sl.c]);
        }
      }
    };
    static_for<RA>([&](auto K) { issue(K); });
    static_for<N>([&](auto K) {
      constexpr int k = decltype(K)::value;
      constexpr Slot sl = BS.slot[k];
      auto &y = pick<sl.blk>(A, B);
      constexpr int W = BW.w[k];  // operand wait (-1: none, see BodyWaits)
      if constexpr (sl.kind == 0) {
        mfma_pv<sl.blk, sl.x, sl.op % NRV, W>(y.o[sl.x], vr[sl.op % NRV], y.p[sl.c]);
      } else if constexpr (sl.kind == 1) {
        mfma_ones(y.lr, ones, y.p[sl.c]);
      } else {
        mfma_s<sl.blk, sl.c, sl.c == 0, sl.op % NRK, W>(y.s[1 - SB][sl.x], kr[sl.op % NRK],
                                                        y.q[sl.c]);
      }
      // LDS reads issue right behind a product: there they cost nothing,
      // while behind the slot's vector work they hold up the next product
      issue(std::integral_constant<int, k + RA>{});
      // the product and its reads open the slot; the vector work follows
      // them, so a result made in one slot is consumed after at least one
      // product's issue (the scheduler would otherwise hoist the consumers
      // next to their producers, where they wait on the exp2 latency)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (SM) {
        // this wave's eight staging loads of tile dma_t + 2, K then V (see
        // dma_slot)
        static_for<2 * kPDpw>([&](auto P) {
          constexpr int part = decltype(P)::value;
          constexpr int i = part < kPDpw ? 2 * part : 2 * (part - kPDpw) + 1;
          if constexpr (dma_slot(part) == k) dma_part_at(dn, i);
        });
        // (each result is pinned to its slot by an empty asm: without it the
        // compiler gathers the vector work where it no longer overlaps the
        // products)
        if constexpr (k < kSmTest) {
          constexpr int kb = k / 4, bi = (k / 2) % 2, j = k % 2;
          auto &x = pick<bi>(A, B);
          constexpr int r0 = 8 * j;
          const f32x16_t &sv = x.s[SB][kb];
          // a block's four eighths run as one chain (its slots are 2 bi, 2 bi + 1,
          // 2 bi + 4 and 2 bi + 5)
          if constexpr (kb == 0 && j == 0)
            mq[bi] = max8(sv[r0], sv[r0 + 1], sv[r0 + 2], sv[r0 + 3], sv[r0 + 4], sv[r0 + 5],
                          sv[r0 + 6], sv[r0 + 7]);
          else
            mq[bi] = max_on8(mq[bi], sv[r0], sv[r0 + 1], sv[r0 + 2], sv[r0 + 3], sv[r0 + 4],
                             sv[r0 + 5], sv[r0 + 6], sv[r0 + 7]);
        }
        if constexpr (k == kSmTest) {
          const float ma = mq[0], mb = mq[1];
          if (__builtin_amdgcn_ballot_w64(ma > A.lim || mb > B.lim) != 0) {
            rebase(A, ma);
            rebase(B, mb);
            rescale = 1;
          }
        }
        static_for<32>([&](auto U) {
          constexpr int u = decltype(U)::value;
          constexpr int bi = sm_blk(u), kb = sm_kb(u), r = 2 * (u % 8);
          constexpr int c = sm_chunk(u), e = 2 * (u % 4);
          auto &x = pick<bi>(A, B);
          if constexpr (sm_fma(u) == k) {
            x.s[SB][kb][r] = __builtin_fmaf(x.s[SB][kb][r], sl2, -x.g);
            x.s[SB][kb][r + 1] = __builtin_fmaf(x.s[SB][kb][r + 1], sl2, -x.g);
            asm volatile("" ::"v"(x.s[SB][kb][r]), "v"(x.s[SB][kb][r + 1]));
          }
          if constexpr (sm_exp(u) == k) {
            x.s[SB][kb][r] = exp2_fast(x.s[SB][kb][r]);
            x.s[SB][kb][r + 1] = exp2_fast(x.s[SB][kb][r + 1]);
            asm volatile("" ::"v"(x.s[SB][kb][r]), "v"(x.s[SB][kb][r + 1]));
          }
          if constexpr (sm_pack(u) == k) {
            x.p[c][e] = (__bf16)x.s[SB][kb][r];
            x.p[c][e + 1] = (__bf16)x.s[SB][kb][r + 1];
            constexpr int i = u % 4;
            if constexpr (u % 8 < 4 && u < 16)
              ps[bi][i] = x.s[SB][kb][r] + x.s[SB][kb][r + 1];
            else
              ps[bi][i] += x.s[SB][kb][r] + x.s[SB][kb][r + 1];
            asm volatile("" ::"v"(x.p[c]), "v"(ps[bi][i]));
          }
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });

    if constexpr (SM) {
      A.l += (ps[0][0] + ps[0][1]) + (ps[0][2] + ps[0][3]);
      B.l += (ps[1][0] + ps[1][1]) + (ps[1][2] + ps[1][3]);
      // (opaque, so the compiler cannot thread the fast and the slow path
      // into two copies of the whole body)
      asm volatile("" : "+s"(rescale));
      // (in the first body the accumulators are still zero: its P.V products
      // ran on P(-1) = 0, so the rebase every row takes there moves nothing)
      if (rescale && key0 != 0) {
        // the body's P.V products added weights of the old reference; the
        // accumulators move to the new one now
        // (a block none of whose rows moved its reference has alpha = 1 in
        // every lane and is left alone)
        const int src = lr_partner(lane);
        if (__builtin_amdgcn_ballot_w64(A.alpha != 1.f) != 0)
          acc_scale(A, A.alpha, lane_fetch(A.alpha, src));
        if (__builtin_amdgcn_ballot_w64(B.alpha != 1.f) != 0)
          acc_scale(B, B.alpha, lane_fetch(B.alpha, src));
      }
    }
  };

  // ---- iterations -----------------------------------------------------------
  // Iteration t opens with the barrier after which K(t+1) and V(t-1) are in
  // LDS (every wave waited for its own loads of them) and tile t-2's stage is
  // free, then runs the body: O += P(t-1) V(t-1), the softmax of S(t),
  // S(t+1), and the loads of tile t+2.  Waves whose rows end before the workgroup's last tile
  // keep taking the barriers and sending their share.
  auto open_iter = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt 4: all but the last tile's V loads
    wg_barrier();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  // where query piece j waits: the K tiles of stages 2 and 3, then their V
  // tiles (none is written before the first body's barrier)
  auto q_piece = [](int j) { return j < 2 ? (2 + j) * PT::TILE : kPVBase + j * PT::TILE; };
  // prologue: the query rows staged through stages 2 and 3 (piece j, rows
  // m0 + 64 j .. + 63, laid out as a K tile; wave w moves a quarter of each
  // piece with the K tile's offsets), then tiles 0 and 1; once the query rows
  // and tile 0's K are in LDS, Q^T goes to its AGPRs and S(0) runs
#pragma unroll
  for (int j = 0; j < kPBlockM / kPBN; ++j) {
    const int r0 = m0 + j * kPBN;
    const int valid = n - r0 < kPBN ? (n - r0 > 0 ? n - r0 : 0) : kPBN;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(qg + (long long)r0 * rs), (short)0,
        __builtin_amdgcn_readfirstlane(valid > 0 ? (int)((valid - 1) * rsb + PT::ROWB) : 0),
        0x00020000);
#pragma unroll
    for (int i = 0; i < kPDpw; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (FA_LDS void *)(smem + q_piece(j) + (w * kPDpw + i) * 1024), 16,
          o_k[i], 0, 0, 0);
  }
  // tiles 0 and 1, both K tiles first: S(0) waits for K(0) and the first
  // body for K(1), while V(0) is first read in the second body
#pragma unroll
  for (int p = 0; p < kPDpw; ++p) dma_part(0, 0, 2 * p);
#pragma unroll
  for (int p = 0; p < kPDpw; ++p) dma_part(1, 1, 2 * p);
#pragma unroll
  for (int p = 0; p < kPDpw; ++p) dma_part(0, 0, 2 * p + 1);
#pragma unroll
  for (int p = 0; p < kPDpw; ++p) dma_part(1, 1, 2 * p + 1);
  // the accumulators and P(-1) are zeroed while the loads fly (before them,
  // the 136 AGPR writes would hold the first load back)
#pragma unroll
  for (int db = 0; db < kPD / 32; ++db) {
    A.o[db] = f32x16_t{};
    B.o[db] = f32x16_t{};
  }
  A.lr = f32x4_t{};
  B.lr = f32x4_t{};
  acc_settle(A);  // places the zeroed accumulators in AGPRs
  acc_settle(B);
  {
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // P(-1) = 0: the first body's P.V adds nothing
      A.p[c] = __builtin_bit_cast(bf16x8_t, z);
      B.p[c] = __builtin_bit_cast(bf16x8_t, z);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F7C);  // vmcnt 12: the query rows and tile 0's K landed
  wg_barrier();
  {
    // wave w's rows are piece w: block a its rows 0 .. 31, block b 32 .. 63
    const uint32_t qa = q_piece(w);
    q_read<0>(A, qa, kofs);
    q_read<1>(B, qa + 32 * PT::ROWB, kofs);
  }
  q_settle<0>(A);  // (awaits the reads)
  q_settle<1>(B);
  if (Tw > 0) {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    DmaTile dn = dma_state(2);  // the loads of body t fetch tile t + 2
    using Vr = std::integral_constant<int, -1>;  // stage known only at run time
    using St0 = std::integral_constant<int, 0>;
    using St1 = std::integral_constant<int, 1>;
    using St2 = std::integral_constant<int, 2>;
    using St3 = std::integral_constant<int, 3>;
    body(F_{}, T_{}, F_{}, S1{}, Vr{}, St0{}, 0, 0u, 0u, dn);  // S(0), into set 0
    // Body t reads V from stage (t - 1) % 4 and K from stage (t + 1) % 4: the
    // loop runs four bodies per trip, so both are compile-time constants.  The
    // first body's P.V runs on P = 0 over stage 3, which holds query rows
    // then (finite data).  On the wave's last tile the score products read a
    // stage whose contents are not used (zeros past the workgroup's last
    // tile), which keeps the loop a straight run of bodies.  Even tiles keep
    // their scores in set 0, odd tiles in set 1, so a body never overwrites
    // the scores it is still turning into weights.
    // the first body's barrier: K(1) has landed, V(0) and V(1) may still fly
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt 8
    wg_barrier();
    for (int t = 0;;) {
      body(T_{}, T_{}, T_{}, S0{}, St3{}, St1{}, t * kPBN, 0u, 0u, dn);
      dma_advance(dn);
      if (++t >= Tw) break;
      open_iter();
      body(T_{}, T_{}, T_{}, S1{}, St0{}, St2{}, t * kPBN, 0u, 0u, dn);
      dma_advance(dn);
      if (++t >= Tw) break;
      open_iter();
      body(T_{}, T_{}, T_{}, S0{}, St1{}, St3{}, t * kPBN, 0u, 0u, dn);
      dma_advance(dn);
      if (++t >= Tw) break;
      open_iter();
      body(T_{}, T_{}, T_{}, S1{}, St2{}, St0{}, t * kPBN, 0u, 0u, dn);
      dma_advance(dn);
      if (++t >= Tw) break;
      open_iter();
    }
    // O += P V of the wave's last tile (its stage is not refilled before this
    // wave's next barrier)
    body(T_{}, F_{}, F_{}, S0{}, Vr{}, Vr{}, 0, stage_off(Tw - 1), 0u, dn);
  }
  for (int t = Tw; t < T; ++t) {  // rows done: barriers and staging only
    open_iter();
    dma_tile(t + 2);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: no staging load outlives the workgroup

  // ---- finalise: O / (rounded-weight sum), lse = ln 2 (m + log2 l) ----------
  // The lane index again, opaque to the compiler, so that the output
  // addresses are computed here rather than kept from the prologue through
  // the loop, where they would take registers the loop needs.
  int lane_f = lane;
  asm volatile("" : "+v"(lane_f));
  auto finalise = [&](auto &x) {
    acc_settle(x);
    const float l_tot = pair_sum(x.l);
    // lane l holds query 16 (l / 32) + l % 16's rounded sum: lanes 16..31
    // and 32..47 trade theirs
    const float lr_tot = lane_fetch(x.lr[0], lr_partner(lane_f));
    const int qrow = x.q0 + (lane_f & 31);
    const int h = lane_f >> 5;
    if (qrow < n) {
      const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
      uint16_t *orow = reinterpret_cast<uint16_t *>(a.o) + tc.base + (long long)qrow * rs;
#pragma unroll
      for (int db = 0; db < kPD / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const bf16x4_t v = {(__bf16)(x.o[db][4 * gq] * inv), (__bf16)(x.o[db][4 * gq + 1] * inv),
                              (__bf16)(x.o[db][4 * gq + 2] * inv),
                              (__bf16)(x.o[db][4 * gq + 3] * inv)};
          *reinterpret_cast<bf16x4_t *>(orow + 32 * db + 8 * gq + 4 * h) = v;
        }
      if (a.lse != nullptr && h == 0) {
        const float m_fin = (x.mbl == neg_inf()) ? 0.f : x.mbl;
        a.lse[tc.lbase + (long long)qrow * a.lse_row_stride] =
            l_tot > 0.f ? (m_fin + __log2f(l_tot)) * 0.693147180559945309f : neg_inf();
      }
    }
  };
  finalise(A);
  finalise(B);
}

template <bool CAUSAL, bool VARLEN>
hipError_t launch_pipe(const FwdArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_bf16_pipe<CAUSAL, VARLEN>), dim3(a.grid), dim3(kPThreads), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_pipe(const FwdArgs &a, bool causal, bool varlen, hipStream_t stream) {
  if (causal)
    return varlen ? launch_pipe<true, true>(a, stream) : launch_pipe<true, false>(a, stream);
  return varlen ? launch_pipe<false, true>(a, stream) : launch_pipe<false, false>(a, stream);
}

}  // namespace fa355
