// fa_fwd_launch.h -- internal interface between the C ABI (fa355_api.hip)
// and the forward kernels (fa_fwd_kernel.hip, fa_fwd_f32.hip).  Not
// installed, not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

namespace fa355 {

// Everything a forward launch needs.  Element strides address one
// (sequence, head) slice: token i of sequence s, head h starts at
//   seq_base(s) + h * head_stride + i * row_stride
// where seq_base(s) = s * seq_stride for a fixed-length batch and
// cu_seqlens[s] * row_stride for a packed one.  lse uses the same scheme
// with its own strides.
struct FwdArgs {
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;             // may be null
  const int *cu_seqlens;  // device, packed batches only
  long long seq_stride;
  long long head_stride;
  long long row_stride;
  long long lse_seq_stride;
  long long lse_head_stride;
  long long lse_row_stride;
  int n;         // sequence length (fixed-length batches)
  int batch;     // sequences (B, or nseq for a packed batch)
  int H;         // heads
  int max_len;   // longest sequence (sizes the grid)
  int n_qtiles;  // query tiles per (sequence, head)  -- set by the launcher
  int grid;      // workgroups launched                -- set by the launcher
  int order_group;  // heads of one XCD scheduled as a group (0: all of them) -- set by the launcher
  float scale;       // softmax scale applied to q.k
  float scale_log2;  // scale * log2(e), for exp2
};

// Smallest number of query rows any kernel gives one workgroup (used by the
// host to bound the grid size before dispatch).
constexpr int kMinBlockM = 128;

// Enqueue the forward kernel for (dtype, d, causal, varlen).  Returns the
// HIP status of the launch.
hipError_t launch_fwd(FwdArgs a, int dtype, int d, bool causal, bool varlen,
                      hipStream_t stream);

// The pipelined bf16 kernel at d = 128 (fa_fwd_pipe.hip): 256 query rows per
// workgroup, like the 8-wave kernel, so the same grid and tile order.
hipError_t launch_fwd_pipe(const FwdArgs &a, bool causal, bool varlen, hipStream_t stream);

// The key-split bf16 kernel for small grids (fa_fwd_ksplit.hip): 32 query
// rows per workgroup, grid = (sequence, head) pairs x n_qtiles.
hipError_t launch_fwd_ksplit(const FwdArgs &a, int d, bool causal, bool varlen,
                             hipStream_t stream);
constexpr int kKsplitBlockM = 32;

// The fp32 kernel (fa_fwd_f32.hip).
hipError_t launch_fwd_f32(FwdArgs a, int d, bool causal, bool varlen, hipStream_t stream);

}  // namespace fa355
