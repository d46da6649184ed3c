// fa_naive_launch.h -- internal interface between the C ABI (fa355_api.hip)
// and the unfused three-step kernels (fa_naive.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>

namespace fa355 {

// [B, H, N, d] tensors as B H = bh contiguous (b, h) slices of N x d; the
// scores / probabilities of slice bh occupy rows of ld floats (ld = N rounded
// up to a multiple of 4, so every row starts 16-byte aligned) at
// s + bh N ld.
struct NaiveArgs {
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;  // [bh, N] or null
  float *s;    // workspace, bh * N * ld floats
  int n;
  int ld;
  int bh;
  float scale;
};

hipError_t launch_naive(const NaiveArgs &a, int dtype, int d, bool causal, hipStream_t stream);

}  // namespace fa355
