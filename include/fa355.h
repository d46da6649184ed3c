/*
 * fa355.h -- C ABI of libfa355, an exact attention forward pass for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (page "Mini FlashAttention", section 1 "What attention
 * is"; the same definition opens "How Did I Write My First FlashAttention
 * Kernel in CUDA?"): for every (batch, head) with rows q_i, k_j, v_j,
 *     S = Q K^T * scale,   P = softmax(S) along each row,   O = P V,
 * with the optional causal mask S[i][j] = -inf for j > i.  The library
 * computes it as the pages' flash algorithm does -- a resident block of
 * query rows, K/V tiles streamed past it, a running row max m, denominator
 * l and output accumulator rescaled by exp(m_old - m_new) per tile, and one
 * division O / l at the end ("Mini FlashAttention", section 4; the grasp.study
 * lesson, "The Complete Kernel: Initialization, Loop, and Finalization") --
 * so the N x N score matrix never reaches memory.  It also returns, per row,
 *     lse_i = ln sum_{j allowed} exp(S[i][j])      (natural log, fp32),
 * the log of the softmax denominator, which lets partial results over
 * disjoint key ranges be merged exactly.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing, frees nothing and never synchronises;
 *     fa_naive_fwd and fa_decode_fwd (when it splits the keys) use a
 *     workspace, which the caller provides.
 *   - A call validates its arguments on the host; on any error it returns a
 *     nonzero FA_ERR_* code and enqueues nothing.  On success it enqueues
 *     its kernel(s) on `stream` (a hipStream_t passed as void*; NULL = the
 *     null stream) and returns FA_OK at once.  Faults inside the kernel surface
 *     at the caller's next synchronisation, as usual for HIP.
 *   - q, k, v and o share one element type, `dtype`: FA_DTYPE_BF16
 *     (bfloat16 storage; products and sums in fp32, the softmax weights
 *     rounded to bf16 for the P.V product, output rounded to nearest even)
 *     or FA_DTYPE_F32 (fp32 throughout).  lse is always fp32.
 *   - Head dimension d is 64 or 128.  q, k, v and o must be 16-byte
 *     aligned, lse 4-byte aligned; o and lse must not overlap q, k, v or
 *     each other.
 *   - `scale` must be finite and > 0 (the pages use 1/sqrt(d)).
 *   - The error state is per host thread (fa_last_hip_error), so calls from
 *     several threads are safe.
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_API __attribute__((visibility("default")))

/* element types */
#define FA_DTYPE_F32 0
#define FA_DTYPE_BF16 1

/* status codes */
#define FA_OK 0
#define FA_ERR_NULL 1     /* a required pointer is NULL */
#define FA_ERR_SHAPE 2    /* negative size, or a size too large to index */
#define FA_ERR_HEAD_DIM 3 /* d is not 64 or 128 */
#define FA_ERR_DTYPE 4    /* dtype is not FA_DTYPE_F32 / FA_DTYPE_BF16 */
#define FA_ERR_SCALE 5    /* scale is not finite and > 0 */
#define FA_ERR_ALIGN 6    /* a tensor pointer is misaligned */
#define FA_ERR_ALIAS 7    /* an output overlaps an input or the other output */
#define FA_ERR_HIP 8      /* the HIP launch failed; see fa_last_hip_error() */
#define FA_ERR_WORKSPACE 9 /* workspace smaller than the *_workspace_bytes() size */
#define FA_ERR_SCRATCH 10  /* fa_decode_fwd_noalloc: partials exceed the static scratch */

/*
 * fa_fwd -- attention forward over a fixed-length batch.
 *
 *   q, k, v  [B, H, N, d] contiguous, dtype elements (read only)
 *   o        [B, H, N, d] contiguous, dtype elements (written)
 *   lse      [B, H, N] fp32 (written), or NULL to skip it
 *   causal   0: every query sees all N keys; nonzero: query i sees keys
 *            0..i (the causal mask of "Mini FlashAttention", section 1)
 *
 * Each (b, h) slice is the pages' row-major [N, d] matrix.  B, H or N equal
 * to 0 is an empty problem: FA_OK, nothing enqueued, pointers not examined
 * (they may be NULL).  Validation order: dtype, d, scale, sizes, then
 * pointers (NULL, alignment, overlap).
 *
 * Short sequences (N <= 128: the whole sequence is one key tile) run a
 * one-tile kernel that computes S, the softmax and P V at once ("Mini
 * FlashAttention", section 3, the one-shot kernel): always for bf16, and for
 * fp32 while the problem is small (N <= 32, or 4 B H N^2 d <= 2^28 flops).
 * bf16 problems with N >= 512 and a small grid (at most 128 query
 * tiles of 256 rows, or 256 when causal) split each tile's key range in two
 * halves streamed side by side and merged exactly through their exponent
 * references.  Results meet the same bounds either way.
 */
FA_API int fa_fwd(const void *q, const void *k, const void *v, void *o,
                  float *lse, int B, int H, int N, int d, float scale,
                  int causal, int dtype, void *stream);

/*
 * fa_fwd_varlen -- attention forward over a packed batch of sequences of
 * different lengths (the pages speak of ragged sequences; the packing is
 * this library's).
 *
 *   q, k, v     [T, H, d] contiguous (token-major), T = cu_seqlens[nseq]
 *   o           [T, H, d] contiguous (written)
 *   lse         [T, H] fp32 (written), or NULL
 *   cu_seqlens  DEVICE int32 [nseq + 1]: sequence s owns tokens
 *               cu_seqlens[s] .. cu_seqlens[s+1]-1 and attends only to
 *               them; the causal mask uses positions local to the sequence.
 *   max_seqlen  host int >= every sequence length (it sizes the grid)
 *
 * Preconditions the host cannot check without reading device memory, so
 * the caller guarantees them: cu_seqlens[0] == 0, non-decreasing, and no
 * length above max_seqlen.  A sequence longer than max_seqlen gets
 * undefined output (rows past max_seqlen are not written, and kernels that
 * size their key staging by max_seqlen may leave out keys of the rows they
 * do write); the other sequences are unaffected.
 * o must not overlap q, k, v or lse (only exact pointer equality is
 * detected here, since T is not known on the host).  nseq, H or max_seqlen
 * equal to 0 is an empty problem, as for fa_fwd.  H d above 2^23 elements
 * per token is FA_ERR_SHAPE (key rows of a tile are addressed with 32-bit
 * byte offsets).
 */
FA_API int fa_fwd_varlen(const void *q, const void *k, const void *v, void *o,
                         float *lse, const int *cu_seqlens, int nseq,
                         int max_seqlen, int H, int d, float scale,
                         int causal, int dtype, void *stream);

/*
 * fa_naive_fwd -- the same attention forward computed the unfused way the
 * pages start from ("How Did I Write My First FlashAttention Kernel in
 * CUDA?", standard attention and its three passes of softmax; "Mini
 * FlashAttention", section 2 on why fusing matters): three kernels,
 *     1. S = Q K^T * scale into the workspace (fp32, N x N per (b, h)),
 *     2. per row: max, sum of exp, P = exp(S - max) / sum written over the
 *        row in dtype, lse = max + ln(sum),
 *     3. O = P V.
 * It exists as the baseline the fused kernel is measured against; its
 * results agree with fa_fwd to the dtype's rounding (not bit for bit).
 *
 *   q, k, v, o, lse, B, H, N, d, scale, causal, dtype  as for fa_fwd
 *   workspace        DEVICE buffer, 16-byte aligned, at least
 *                    fa_naive_workspace_bytes(B, H, N) bytes, owned by the
 *                    caller; its contents are overwritten and must not
 *                    overlap any tensor argument.
 *   workspace_bytes  its size (FA_ERR_WORKSPACE when too small)
 *
 * B H must not exceed 65535 and N not 2^22 (FA_ERR_SHAPE).  Causal score
 * tiles entirely above the diagonal are not computed.
 */
FA_API int fa_naive_fwd(const void *q, const void *k, const void *v, void *o,
                        float *lse, void *workspace, size_t workspace_bytes,
                        int B, int H, int N, int d, float scale, int causal,
                        int dtype, void *stream);

/* Workspace bytes fa_naive_fwd needs: B H N rows of N floats, each row
 * rounded up to a multiple of 4 floats; 0 if a size is <= 0 or out of the
 * range fa_naive_fwd accepts. */
FA_API size_t fa_naive_workspace_bytes(int B, int H, int N);

/*
 * fa_decode_fwd -- attention for decode-shaped problems: per (b, h), a few
 * queries against a long key/value cache.  "Mini FlashAttention", section 1
 * ties the causal mask to autoregressive decoding; the queries are taken to
 * be the newest Nq positions of the Nk-long sequence.  The key range of each
 * (b, h) is split into pieces processed in parallel, and the pieces' results
 * are merged exactly through their log-sum-exp: with lse_s and O_s the
 * softmax results over disjoint key sets, lse = ln sum_s exp(lse_s) and
 * O = sum_s exp(lse_s - lse) O_s.
 *
 *   q, o        [B, H, Nq, d] contiguous, dtype elements
 *   k, v        [B, H, Nk, d] contiguous, dtype elements (read only)
 *   lse         [B, H, Nq] fp32 (written), or NULL
 *   causal      0: every query sees all Nk keys; nonzero: query i
 *               (0-based among the Nq) sees keys 0 .. Nk - Nq + i.  A query
 *               that sees no key (Nq > Nk) gets O = 0 and lse = -inf.
 *   num_splits  0: the library's choice (enough waves to fill the GPU, key
 *               ranges of at least 256 keys); n > 0: at most n ranges per
 *               (b, h) (ranges are whole multiples of 16 keys, so fewer may
 *               result).  fa_decode_num_splits() gives the count used.
 *   workspace   DEVICE buffer, 16-byte aligned, of at least
 *               fa_decode_workspace_bytes(B, H, Nq, Nk, d, num_splits)
 *               bytes, owned by the caller (its contents are overwritten;
 *               it must not overlap any tensor argument).  When that size
 *               is 0 (one range per (b, h)) the workspace may be NULL.
 *   workspace_bytes  its size (FA_ERR_WORKSPACE when too small)
 *
 * 1 <= Nq <= 64 and 1 <= Nk <= 2^30 (FA_ERR_SHAPE otherwise); B, H or Nq
 * equal to 0 is an empty problem (FA_OK, nothing enqueued).  The same
 * validation order and dtype conventions as fa_fwd.  Enqueues one kernel, or
 * two when the keys are split.
 */
FA_API int fa_decode_fwd(const void *q, const void *k, const void *v, void *o,
                         float *lse, void *workspace, size_t workspace_bytes,
                         int B, int H, int Nq, int Nk, int d, float scale,
                         int causal, int dtype, int num_splits, void *stream);

/*
 * fa_decode_fwd_noalloc -- fa_decode_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the
 * same split plan, kernels and results.  The split partial results go to a
 * static device array of FA_DECODE_SCRATCH_BYTES inside the library, one
 * copy per GPU, held until the process ends; the call uses the copy of the
 * current device (hipGetDevice), so `stream` must belong to that device.
 * The call itself allocates nothing (no hipMalloc, no library allocator).
 *
 * Problems whose partial results, fa_decode_workspace_bytes(B, H, Nq, Nk,
 * d, num_splits), exceed FA_DECODE_SCRATCH_BYTES return FA_ERR_SCRATCH and
 * enqueue nothing; pass a smaller num_splits, or use fa_decode_fwd with a
 * workspace.  Every call on one GPU shares that GPU's array and overwrites
 * it (nothing in it needs to start at zero): calls whose kernels may run
 * at the same time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller.  The first call on a device looks up
 * the array's address (FA_ERR_HIP if that fails).
 */
#define FA_DECODE_SCRATCH_BYTES (16u << 20)
FA_API int fa_decode_fwd_noalloc(const void *q, const void *k, const void *v,
                                 void *o, float *lse, int B, int H, int Nq,
                                 int Nk, int d, float scale, int causal,
                                 int dtype, int num_splits, void *stream);

/* Workspace bytes fa_decode_fwd needs for these sizes: splits x B H Nq x
 * (d + 1) floats when the keys are split, else 0; also 0 when the sizes are
 * out of range. */
FA_API size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d,
                                        int num_splits);

/* Number of key ranges per (b, h) fa_decode_fwd uses for these sizes and
 * num_splits request (0 when the sizes are out of range). */
FA_API int fa_decode_num_splits(int B, int H, int Nq, int Nk, int num_splits);

/* Human-readable name of a status code (static storage, never NULL). */
FA_API const char *fa_status_string(int status);

/* The hipError_t of this thread's last FA_ERR_HIP (0 if none). */
FA_API int fa_last_hip_error(void);

/* Library version string, e.g. "libfa355 0.1.0 gfx950". */
FA_API const char *fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
