// fa_small_launch.h -- internal interface of the one-tile kernel for short
// sequences (fa_small.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_fwd_launch.h"

namespace fa355 {

// Longest sequence the one-tile kernel takes: one key tile.
constexpr int kSmallMaxN = 128;

// bf16 batches whose longest sequence has 1 <= a.max_len <= kSmallMaxN
// tokens: fixed-length (a.n = a.max_len) or packed (varlen: lengths from
// a.cu_seqlens); a.batch, a.H, the strides, scale and pointers as for
// launch_fwd.
hipError_t launch_small_bf16(const FwdArgs &a, int d, bool causal, bool varlen,
                             hipStream_t stream);

// The same for fp32 batches (plain fp32 arithmetic, 16 queries per
// workgroup).
hipError_t launch_small_f32(const FwdArgs &a, int d, bool causal, hipStream_t stream);

}  // namespace fa355
