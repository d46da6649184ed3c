// fa355_api.hip -- the C ABI declared in include/fa355.h: host-side argument
// validation, stride set-up and dispatch to the forward kernels.  Every
// check runs before anything is enqueued; on error nothing is launched.

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "fa355.h"
#include "fa_decode_launch.h"
#include "fa_fwd_launch.h"
#include "fa_naive_launch.h"
#include "fa_small_launch.h"

namespace {

thread_local int g_last_hip = 0;

constexpr long long kMaxRows = 1ll << 40;  // B*H*N bound keeps every offset in int64
constexpr long long kMaxGrid = 0x7fffffffll;
constexpr long long kMaxTokenElems = 1ll << 23;  // H * d of a packed token

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Checks that do not depend on the problem being non-empty.
int value_checks(int d, float scale, int dtype) {
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

// Pointer checks, for non-empty problems (an empty one may pass NULLs).
int pointer_checks(const void *q, const void *k, const void *v, void *o, const float *lse) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
      misaligned(lse, 4))
    return FA_ERR_ALIGN;
  return FA_OK;
}

int launch(const fa355::FwdArgs &a, int dtype, int d, int causal, bool varlen, void *stream) {
  const hipError_t e =
      fa355::launch_fwd(a, dtype, d, causal != 0, varlen, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

// Split plan of fa_decode_fwd: key ranges of `chunk` keys (a multiple of
// 16), `splits` of them per (b, h), and `qchunks` groups of queries.  With
// num_splits = 0 the ranges are sized for about one streaming wave per SIMD
// (1024 waves), or two when a wave carries 4 queries and has more arithmetic
// per byte to hide; fewer, longer streams measured faster than more, shorter
// ones.  No range is shorter than 256 keys.  A request is capped at Nk, and
// rounding the range up to 16 keys can lower it further.
namespace {
constexpr int kDecodeMaxQ = 64;
constexpr int kDecodeMinKeys = 256;

struct DecodePlan {
  bool ok;
  int splits, chunk, qchunks;
  long long tasks;
  size_t ws_bytes;  // 0 when splits == 1
};

DecodePlan decode_plan(int B, int H, int Nq, int Nk, int d, int num_splits) {
  DecodePlan p{};
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || Nq > kDecodeMaxQ || num_splits < 0) return p;
  if (d != 64 && d != 128) return p;
  const long long bh = (long long)B * H;
  if (Nk > (1 << 30) || bh * (Nq > Nk ? Nq : Nk) > kMaxRows) return p;
  if (bh * Nq * d / 256 > kMaxGrid) return p;  // merge grid
  const int nqw = fa355::decode_queries_per_wave(Nq);
  p.qchunks = (Nq + nqw - 1) / nqw;
  const long long items = bh * p.qchunks;
  long long req = num_splits;
  if (req == 0) {
    const long long target = nqw >= 4 ? 2048 : 1024;
    req = (target + items - 1) / items;
    const long long cap = Nk / kDecodeMinKeys > 1 ? Nk / kDecodeMinKeys : 1;
    if (req > cap) req = cap;
  }
  if (req > Nk) req = Nk;
  long long chunk = (Nk + req - 1) / req;
  chunk = (chunk + 15) & ~15ll;
  p.chunk = static_cast<int>(chunk);
  p.splits = static_cast<int>((Nk + chunk - 1) / chunk);
  p.tasks = items * p.splits;
  if (p.tasks > 4 * kMaxGrid) return p;
  const unsigned long long rows = (unsigned long long)bh * Nq;
  p.ws_bytes = p.splits > 1 ? (size_t)(p.splits * rows * (unsigned long long)(d + 1) * 4ull) : 0;
  p.ok = true;
  return p;
}
}  // namespace

// ---- static scratch of fa_decode_fwd_noalloc ------------------------------
// The split partial results of fa_decode_fwd_noalloc live in this array: one
// copy per GPU, created with the code object when the library is loaded on
// that GPU and held until the process ends.  Host code never uses the name
// itself as an address (on the host it is only a stand-in for the symbol):
// each GPU's copy is looked up once, with that GPU current, by
// hipGetSymbolAddress, and that address is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Address of the current GPU's scratch array, looked up on the first call
// made with that GPU current; nullptr (with *status set) on failure.
void *device_scratch(int *status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip = static_cast<int>(e);
    *status = FA_ERR_HIP;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_hip = static_cast<int>(hipErrorInvalidDevice);
    *status = FA_ERR_HIP;
    return nullptr;
  }
  void *ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch[dev].load(std::memory_order_relaxed);
  if (ptr == nullptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      g_last_hip = static_cast<int>(e != hipSuccess ? e : hipErrorInvalidSymbol);
      *status = FA_ERR_HIP;
      return nullptr;
    }
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

// fa_decode_fwd and fa_decode_fwd_noalloc: the same validation, plan and
// kernels; the partial results go to the caller's workspace, or (noalloc) to
// the current GPU's static scratch array.
int decode_common(const void *q, const void *k, const void *v, void *o, float *lse,
                  void *workspace, size_t workspace_bytes, bool noalloc, int B, int H, int Nq,
                  int Nk, int d, float scale, int causal, int dtype, int num_splits,
                  void *stream) {
  int st = value_checks(d, scale, dtype);
  if (st != FA_OK) return st;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || num_splits < 0) return FA_ERR_SHAPE;
  if (B == 0 || H == 0 || Nq == 0) return FA_OK;
  const DecodePlan p = decode_plan(B, H, Nq, Nk, d, num_splits);
  if (!p.ok) return FA_ERR_SHAPE;
  st = pointer_checks(q, k, v, o, lse);
  if (st != FA_OK) return st;
  if (p.ws_bytes > 0 && noalloc) {
    if (p.ws_bytes > FA_DECODE_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  } else if (p.ws_bytes > 0) {
    if (!workspace) return FA_ERR_NULL;
    if (misaligned(workspace, 16)) return FA_ERR_ALIGN;
    if (workspace_bytes < p.ws_bytes) return FA_ERR_WORKSPACE;
  }
  const long long bh = (long long)B * H;
  const size_t esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
  const size_t qbytes = (size_t)(bh * Nq) * d * esz, kbytes = (size_t)(bh * Nk) * d * esz;
  const size_t lbytes = (size_t)(bh * Nq) * sizeof(float);
  if (overlap(o, qbytes, q, qbytes) || overlap(o, qbytes, k, kbytes) ||
      overlap(o, qbytes, v, kbytes))
    return FA_ERR_ALIAS;
  if (lse && (overlap(lse, lbytes, q, qbytes) || overlap(lse, lbytes, k, kbytes) ||
              overlap(lse, lbytes, v, kbytes) || overlap(lse, lbytes, o, qbytes)))
    return FA_ERR_ALIAS;
  if (p.ws_bytes > 0 && !noalloc &&
      (overlap(workspace, p.ws_bytes, q, qbytes) || overlap(workspace, p.ws_bytes, k, kbytes) ||
       overlap(workspace, p.ws_bytes, v, kbytes) || overlap(workspace, p.ws_bytes, o, qbytes) ||
       (lse && overlap(workspace, p.ws_bytes, lse, lbytes))))
    return FA_ERR_ALIAS;
  if (p.ws_bytes > 0 && noalloc) {  // every argument check has passed
    workspace = device_scratch(&st);
    if (!workspace) return st;
  }
  fa355::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  if (p.ws_bytes > 0) {
    a.part_o = static_cast<float *>(workspace);
    a.part_lse = a.part_o + (size_t)p.splits * (size_t)(bh * Nq) * d;
  }
  a.bh = bh;
  a.nq = Nq;
  a.nk = Nk;
  a.splits = p.splits;
  a.chunk = p.chunk;
  a.qchunks = p.qchunks;
  a.tasks = p.tasks;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  const hipError_t e = fa355::launch_decode(a, dtype, d, causal != 0,
                                            reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // namespace

extern "C" {

FA_API int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                  int N, int d, float scale, int causal, int dtype, void *stream) {
  int st = value_checks(d, scale, dtype);
  if (st != FA_OK) return st;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  st = pointer_checks(q, k, v, o, lse);
  if (st != FA_OK) return st;
  const long long bh = (long long)B * H;  // < 2^62, no overflow
  const long long n_qtiles = (N + fa355::kMinBlockM - 1) / fa355::kMinBlockM;
  if (bh > kMaxRows / N || bh > kMaxGrid / n_qtiles) return FA_ERR_SHAPE;
  const long long rows = bh * N;

  const size_t esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
  const size_t tbytes = (size_t)rows * d * esz;
  if (overlap(o, tbytes, q, tbytes) || overlap(o, tbytes, k, tbytes) ||
      overlap(o, tbytes, v, tbytes))
    return FA_ERR_ALIAS;
  if (lse) {
    const size_t lbytes = (size_t)rows * sizeof(float);
    if (overlap(lse, lbytes, q, tbytes) || overlap(lse, lbytes, k, tbytes) ||
        overlap(lse, lbytes, v, tbytes) || overlap(lse, lbytes, o, tbytes))
      return FA_ERR_ALIAS;
  }

  fa355::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_seqlens = nullptr;
  a.row_stride = d;
  a.head_stride = (long long)N * d;
  a.seq_stride = (long long)H * N * d;
  a.lse_row_stride = 1;
  a.lse_head_stride = N;
  a.lse_seq_stride = (long long)H * N;
  a.n = N;
  a.batch = B;
  a.H = H;
  a.max_len = N;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  // The whole sequence is one key tile: the one-tile kernels.  bf16 always
  // (ahead of the streaming kernel at every measured size); fp32 only while
  // the problem is latency-bound -- N <= 32, or at most 2^28 flops in all --
  // since its vector-ALU arithmetic is ~3 x slower per flop than the fp32
  // matrix-core streaming kernel once many heads fill the GPU.
  const double flops = 4.0 * (double)bh * N * (double)N * d;
  const bool one_tile = N <= fa355::kSmallMaxN &&
                        (dtype == FA_DTYPE_BF16 || N <= 32 || flops <= 268435456.0);
  if (one_tile) {
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = dtype == FA_DTYPE_BF16
                             ? fa355::launch_small_bf16(a, d, causal != 0, false, st)
                             : fa355::launch_small_f32(a, d, causal != 0, st);
    if (e != hipSuccess) {
      g_last_hip = static_cast<int>(e);
      return FA_ERR_HIP;
    }
    return FA_OK;
  }
  return launch(a, dtype, d, causal, false, stream);
}

FA_API int fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                         const int *cu_seqlens, int nseq, int max_seqlen, int H, int d,
                         float scale, int causal, int dtype, void *stream) {
  int st = value_checks(d, scale, dtype);
  if (st != FA_OK) return st;
  if (nseq < 0 || H < 0 || max_seqlen < 0) return FA_ERR_SHAPE;
  if (nseq == 0 || H == 0 || max_seqlen == 0) return FA_OK;
  // a K/V tile's rows (up to 128 tokens of H * d elements) are addressed with
  // 32-bit byte offsets
  if ((long long)H * d > kMaxTokenElems) return FA_ERR_SHAPE;
  st = pointer_checks(q, k, v, o, lse);
  if (st != FA_OK) return st;
  if (!cu_seqlens) return FA_ERR_NULL;
  if (misaligned(cu_seqlens, 4)) return FA_ERR_ALIGN;
  const long long n_qtiles = (max_seqlen + fa355::kMinBlockM - 1) / fa355::kMinBlockM;
  if ((long long)nseq * H > kMaxGrid / n_qtiles) return FA_ERR_SHAPE;
  if (o == q || o == k || o == v || (lse && (void *)lse == o)) return FA_ERR_ALIAS;

  fa355::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_seqlens = cu_seqlens;
  a.row_stride = (long long)H * d;
  a.head_stride = d;
  a.seq_stride = 0;
  a.lse_row_stride = H;
  a.lse_head_stride = 1;
  a.lse_seq_stride = 0;
  a.n = 0;
  a.batch = nseq;
  a.H = H;
  a.max_len = max_seqlen;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  // bf16 batches of short sequences (every one a single key tile): the
  // one-tile kernel, as for fa_fwd
  if (dtype == FA_DTYPE_BF16 && max_seqlen <= fa355::kSmallMaxN) {
    const hipError_t e = fa355::launch_small_bf16(a, d, causal != 0, true,
                                                  reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
      g_last_hip = static_cast<int>(e);
      return FA_ERR_HIP;
    }
    return FA_OK;
  }
  return launch(a, dtype, d, causal, true, stream);
}

// Bytes of the scores workspace of fa_naive_fwd: B H N rows of N floats,
// each row padded to a multiple of 4 floats; 0 for sizes out of range.
static size_t naive_bytes(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  const long long ld = ((long long)N + 3) & ~3ll;
  const long long bh = (long long)B * H;
  if (bh > 65535 || N > (1 << 22)) return 0;
  const unsigned long long rows = (unsigned long long)bh * N;
  if (rows > (1ull << 40) / (unsigned long long)ld) return 0;
  return (size_t)(rows * (unsigned long long)ld * 4ull);
}

FA_API size_t fa_naive_workspace_bytes(int B, int H, int N) { return naive_bytes(B, H, N); }

FA_API int fa_naive_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                        void *workspace, size_t workspace_bytes, int B, int H, int N, int d,
                        float scale, int causal, int dtype, void *stream) {
  int st = value_checks(d, scale, dtype);
  if (st != FA_OK) return st;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  const size_t need = naive_bytes(B, H, N);
  if (need == 0) return FA_ERR_SHAPE;
  st = pointer_checks(q, k, v, o, lse);
  if (st != FA_OK) return st;
  if (!workspace) return FA_ERR_NULL;
  if (misaligned(workspace, 16)) return FA_ERR_ALIGN;
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  const long long rows = (long long)B * H * N;
  const size_t esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
  const size_t tbytes = (size_t)rows * d * esz, lbytes = (size_t)rows * sizeof(float);
  if (overlap(o, tbytes, q, tbytes) || overlap(o, tbytes, k, tbytes) ||
      overlap(o, tbytes, v, tbytes))
    return FA_ERR_ALIAS;
  if (lse && (overlap(lse, lbytes, q, tbytes) || overlap(lse, lbytes, k, tbytes) ||
              overlap(lse, lbytes, v, tbytes) || overlap(lse, lbytes, o, tbytes)))
    return FA_ERR_ALIAS;
  if (overlap(workspace, need, q, tbytes) || overlap(workspace, need, k, tbytes) ||
      overlap(workspace, need, v, tbytes) || overlap(workspace, need, o, tbytes) ||
      (lse && overlap(workspace, need, lse, lbytes)))
    return FA_ERR_ALIAS;
  fa355::NaiveArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.s = static_cast<float *>(workspace);
  a.n = N;
  a.ld = (N + 3) & ~3;
  a.bh = B * H;
  a.scale = scale;
  const hipError_t e = fa355::launch_naive(a, dtype, d, causal != 0,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}


FA_API size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  const DecodePlan p = decode_plan(B, H, Nq, Nk, d, num_splits);
  return p.ok ? p.ws_bytes : 0;
}

FA_API int fa_decode_num_splits(int B, int H, int Nq, int Nk, int num_splits) {
  const DecodePlan p = decode_plan(B, H, Nq, Nk, 64, num_splits);
  return p.ok ? p.splits : 0;
}

FA_API int fa_decode_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                         void *workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk,
                         int d, float scale, int causal, int dtype, int num_splits, void *stream) {
  return decode_common(q, k, v, o, lse, workspace, workspace_bytes, false, B, H, Nq, Nk, d, scale,
                       causal, dtype, num_splits, stream);
}

FA_API int fa_decode_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                                 int B, int H, int Nq, int Nk, int d, float scale, int causal,
                                 int dtype, int num_splits, void *stream) {
  return decode_common(q, k, v, o, lse, nullptr, 0, true, B, H, Nq, Nk, d, scale, causal, dtype,
                       num_splits, stream);
}

FA_API const char *fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: negative or oversized problem size";
    case FA_ERR_HEAD_DIM: return "FA_ERR_HEAD_DIM: head dimension must be 64 or 128";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: dtype must be FA_DTYPE_F32 or FA_DTYPE_BF16";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensors need 16-byte alignment, lse 4-byte";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output overlaps an input or the other output";
    case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed (see fa_last_hip_error)";
    case FA_ERR_WORKSPACE:
      return "FA_ERR_WORKSPACE: workspace smaller than the entry point's *_workspace_bytes()";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the split partial results exceed FA_DECODE_SCRATCH_BYTES";
    default: return "unknown status";
  }
}

FA_API int fa_last_hip_error(void) { return g_last_hip; }

FA_API const char *fa_version(void) { return "libfa355 0.1.0 gfx950"; }

}  // extern "C"
