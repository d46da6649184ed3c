// fa_decode_launch.h -- host-side interface of the split-KV decode kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace fa355 {

// Queries each wave carries (1, 2 or 4) for a problem of nq queries.
inline int decode_queries_per_wave(int nq) { return nq >= 3 ? 4 : (nq == 2 ? 2 : 1); }

struct DecodeArgs {
  const void *q;   // [bh, nq, d]
  const void *k;   // [bh, nk, d]
  const void *v;   // [bh, nk, d]
  void *o;         // [bh, nq, d]
  float *lse;      // [bh, nq] or nullptr
  float *part_o;   // [splits, bh * nq, d] fp32 (splits > 1)
  float *part_lse; // [splits, bh * nq] fp32 (splits > 1)
  long long bh;    // batch * heads
  int nq, nk;
  int splits;      // key ranges per (b, h)
  int chunk;       // keys per range, a multiple of 16
  int qchunks;     // groups of queries per (b, h): ceil(nq / queries per wave)
  long long tasks; // bh * splits * qchunks waves
  float scale;     // softmax scale
  float scale_log2;
};

// Enqueues the split kernel (and the merge kernel when splits > 1).
hipError_t launch_decode(const DecodeArgs &a, int dtype, int d, bool causal, hipStream_t stream);

}  // namespace fa355
