/*
 * fa.h -- C ABI of the exact, tiled, fused attention library for AMD MI355X (gfx950).
 *
 * What is computed
 *   For every batch element b and head h, with Q, K, V the N x d matrices of that head:
 *     S   = scale * Q K^T + mask                       (mask entries are 0 or -inf)
 *     O   = softmax_rows(S) V
 *     LSE = per-row natural-log log-sum-exp of S      (the statistic the backward reuses)
 *   "NOTE-005: FlashAttention" (anthology-of-the-sota), section "Key results", Theorem 1 states
 *   the product softmax(Q K^T) V; the scaling and masking steps come from the promptingindex page
 *   "FlashAttention: The IO-Aware Algorithm That Rewrote GPU Training Speed Records", section
 *   "Why attention is memory-bound, not compute-bound".  The forward keeps a running maximum and
 *   normaliser per row and stores LSE = m + ln(l); the backward recomputes the attention block
 *   from it instead of reading a stored N x N matrix (NOTE-005, "Method").  The N x N score matrix
 *   never exists in device memory.
 *
 * Masks
 *   causal != 0 : key j is visible to query i only if j <= i (top-left aligned; queries and keys
 *                 have the same length N).
 *   seqlens     : optional device array of B int32 valid key counts.  Key j of batch element b is
 *                 visible only if j < clamp(seqlens[b], 0, N), for every head and every query.
 *                 Query rows at or past that length are still computed (they attend to the valid
 *                 keys).  A row with no visible key gets O = 0, LSE = -inf and no gradient.
 *   Both masks combine by AND.  fa_forward and fa_backward apply no dropout; the fa_*_dropout entry
 *   points below add it.
 *
 * Layout and types (all tensors are caller-owned device memory)
 *   q, k, v, o, dO, dq, dk, dv : contiguous row-major [B][H][N][d], d fastest, element type `dtype`.
 *   lse                        : contiguous [B][H][N] float32 (natural log, units of the scaled
 *                                scores), written by fa_forward and read by fa_backward.
 *   d must be 64 or 128.  Any N >= 1 (ragged tails are masked); offsets are 64-bit.  For bf16 the
 *   bytes of one head, N*d*2, must be below 2^31 (FA_ERR_INVALID_ARGUMENT otherwise).
 *   Base pointers of the [B][H][N][d] tensors must be 16-byte aligned, lse and seqlens 4-byte.
 *   bf16 results are rounded to nearest even; every accumulation is float32.
 *
 * Ownership, threads, streams
 *   The library allocates nothing and keeps no state between calls (apart from a thread-local
 *   error string).  Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and runs
 *   asynchronously; a return of FA_OK means the work was enqueued.  Outputs must not alias
 *   inputs.  Calls from several host threads are safe.
 *
 * Errors
 *   Argument errors are detected on the host before anything is enqueued; outputs are then left
 *   untouched.  A kernel fault surfaces at the caller's next synchronisation, like any HIP error.
 *   No call prints, throws or aborts.  There is no fallback path: an unsupported dtype or head
 *   dimension is an error (FA_ERR_UNSUPPORTED), never a silent switch to another attention.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null pointer, B/H/N <= 0, non-finite scale, grid too large */
  FA_ERR_UNSUPPORTED = 2,      /* dtype not FA_DTYPE_F32/FA_DTYPE_BF16, or d not 64/128 */
  FA_ERR_MISALIGNED = 3,       /* a base pointer breaks the alignment rule above */
  FA_ERR_WORKSPACE = 4,        /* workspace null or smaller than fa_backward_workspace_size() */
  FA_ERR_HIP = 5               /* the HIP runtime reported an error (text in fa_last_error()) */
} fa_status_t;

typedef enum { FA_DTYPE_F32 = 0, FA_DTYPE_BF16 = 1 } fa_dtype_t;

/*
 * Forward: O and LSE (see above).
 *   q, k, v : inputs [B][H][N][d]             o   : output [B][H][N][d]
 *   lse     : output [B][H][N] float32        scale: multiplies Q K^T (usually 1/sqrt(d))
 *   causal  : 0 or 1                          seqlens: device int32[B] or NULL
 * Extra device memory: none.  The tile loop (the pages' tiling of Q, K and V into on-chip blocks
 * with online softmax; NOTE-005 "Method") runs entirely in LDS and registers.
 */
fa_status_t fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, float scale, int causal,
                       const int32_t* seqlens, fa_dtype_t dtype, void* stream);

/*
 * Bytes of device workspace fa_backward needs for these sizes: one float32 per row for
 * -D_i = -sum_c dO_ic O_ic, plus (bf16 only) one float32 per row for LSE_i log2(e).  Returns 0 for
 * invalid or unsupported sizes.  Linear in N (O(N) extra memory; NOTE-005 "Key results",
 * Theorem 1).
 */
size_t fa_backward_workspace_size(int B, int H, int N, int d, fa_dtype_t dtype);

/*
 * Backward of the loss sum(dO * O): writes dq, dk, dv ([B][H][N][d], element type dtype).
 *   o, lse must be exactly what fa_forward returned for the same q, k, v, sizes, scale, causal
 *   and seqlens (not checked; otherwise the result is undefined).
 *   workspace: caller-owned device memory of at least fa_backward_workspace_size() bytes,
 *   16-byte aligned; its contents on entry do not matter and are scratch on exit.
 * The attention block is recomputed from Q, K and LSE (NOTE-005 "Method").  Every output element
 * has a single writer and a fixed summation order, so dq, dk and dv are bitwise reproducible.
 */
fa_status_t fa_backward(const void* q, const void* k, const void* v, const void* o,
                        const void* dO, const float* lse, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, float scale, int causal,
                        const int32_t* seqlens, fa_dtype_t dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward in its stages, for callers that schedule or time them separately.  fa_backward(...)
 * gives the results of these three calls in order on one stream, with the same workspace:
 *   fa_backward_prepare : -D_i = -sum_c dO_ic O_ic into the workspace (negated: the dK/dV pass
 *                         starts its dO V^T products from it); for bf16 also LSE_i log2(e).
 *                         Reads o, dO and lse only.
 *   fa_backward_dkdv    : the recompute pass over query blocks for each block of keys: writes dk
 *                         and dv.  Reads the workspace as fa_backward_prepare left it.
 *   fa_backward_dq      : the recompute pass over key blocks for each block of queries: writes dq.
 *                         Reads the workspace as fa_backward_prepare left it.
 * fa_backward_dkdv and fa_backward_dq do not depend on each other (both only read the workspace),
 * so they may run in either order or on two streams once fa_backward_prepare has completed.
 *   fa_backward_dq_prepare : fa_backward_prepare and fa_backward_dq in one call (it also reads o):
 *                         writes dq and leaves in the workspace exactly what fa_backward_prepare
 *                         writes, so fa_backward_dkdv may follow it.  For bf16 one pass forms D and
 *                         LSE log2(e) of each row from the rows of o and dO it holds anyway, summed in
 *                         the prepare stage's order (bitwise the same values); fa_backward (and the
 *                         block-sparse and dropout backwards) run it, then the dK/dV pass, for bf16.
 * Arguments, layout and errors as in fa_backward.
 */
fa_status_t fa_backward_prepare(const void* o, const void* dO, const float* lse, int B, int H, int N, int d,
                                fa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream);
fa_status_t fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                             void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                             const int32_t* seqlens, fa_dtype_t dtype, const void* workspace,
                             size_t workspace_bytes, void* stream);
fa_status_t fa_backward_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                           void* dq, int B, int H, int N, int d, float scale, int causal,
                           const int32_t* seqlens, fa_dtype_t dtype, const void* workspace,
                           size_t workspace_bytes, void* stream);
fa_status_t fa_backward_dq_prepare(const void* q, const void* k, const void* v, const void* o,
                                   const void* dO, const float* lse, void* dq, int B, int H, int N,
                                   int d, float scale, int causal, const int32_t* seqlens,
                                   fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Block-sparse attention: the computation above restricted to a pattern of 128 x 128 blocks.
 * The pages describe the block-sparse extension as the same tiling applied to a sparse attention
 * pattern ("FlashAttention: The IO-Aware Algorithm That Rewrote GPU Training Speed Records",
 * promptingindex page, section "Benchmark results: speed records without any approximation";
 * NOTE-005: FlashAttention, "Key components" and "Limitations", where it is approximate relative
 * to dense attention).  Relative to its own mask the result is exact.
 *   block_mask : device uint8 array [B][H][nb][nb], nb = ceil(N / FA_MASK_BLOCK), row-major and
 *                contiguous, caller-owned, read only.  Entry (qb, kb) != 0 makes key j visible to
 *                query i when i / FA_MASK_BLOCK == qb and j / FA_MASK_BLOCK == kb; the causal and
 *                seqlens masks still apply (AND).  Blocks that are zero are skipped: their key or
 *                query tiles are neither loaded nor computed.  A row with no visible key gets O = 0,
 *                LSE = -inf and no gradient.
 *   N must be at most FA_MASK_MAX_N (FA_ERR_UNSUPPORTED otherwise); block_mask must not be NULL.
 * All other arguments, layouts, ownership and errors are those of fa_forward and fa_backward
 * (same workspace size); fa_backward_block_sparse must receive the o and lse that
 * fa_forward_block_sparse produced with the same block mask.
 */
#define FA_MASK_BLOCK 128
#define FA_MASK_MAX_N 131072
fa_status_t fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int B, int H, int N, int d, float scale, int causal,
                                    const int32_t* seqlens, const uint8_t* block_mask, fa_dtype_t dtype,
                                    void* stream);
fa_status_t fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o,
                                     const void* dO, const float* lse, void* dq, void* dk, void* dv,
                                     int B, int H, int N, int d, float scale, int causal,
                                     const int32_t* seqlens, const uint8_t* block_mask, fa_dtype_t dtype,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dropout on the attention probabilities, fused: a step of the attention chain the pages list
 * (promptingindex page, "Why attention is memory-bound, not compute-bound": matmul, scaling,
 * masking, softmax, dropout, matmul); the mask is regenerated in every kernel from a counter-based
 * generator and never stored (the recomputation of NOTE-005: FlashAttention, "Method").
 *   O = (P * Z (256 / t)) V with P the softmax of the masked, scaled scores, t = round((1 - p) 256)
 *   (half to even, 1 <= t <= 256) and Z the keep mask: element (b, h, query i, key j) is kept when
 *   byte e of word g of Philox4x32-10 (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2,
 *   3", SC'11) with key (seed & 0xffffffff, seed >> 32) and counter
 *   (i, j / 32, b H + h, 2 offset + (j / 4) % 2) is below t, where j % 32 = 8 g + 4 ((j / 4) % 2) + e.
 *   LSE is that of the undropped P.  The backward is the gradient of sum(dO * O) through the same
 *   Z (same seed and offset).
 *   dropout_p: 0 <= p and t >= 1 (p <= about 0.998), finite; FA_ERR_INVALID_ARGUMENT otherwise.
 *   p = 0 reproduces fa_forward / fa_backward.  Dense attention only (no block mask).
 * fa_dropout_mask writes Z itself as bytes (1 = kept) into keep, device uint8 [B][H][N][N],
 * caller-owned: the decisions the two other calls take, for inspection and tests.
 * Other arguments, layouts and errors as in fa_forward / fa_backward.
 */
fa_status_t fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, int d, float scale, int causal,
                               const int32_t* seqlens, float dropout_p, uint64_t seed, uint32_t offset,
                               fa_dtype_t dtype, void* stream);
fa_status_t fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                                const void* dO, const float* lse, void* dq, void* dk, void* dv,
                                int B, int H, int N, int d, float scale, int causal,
                                const int32_t* seqlens, float dropout_p, uint64_t seed, uint32_t offset,
                                fa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream);
fa_status_t fa_dropout_mask(int B, int H, int N, float dropout_p, uint64_t seed, uint32_t offset,
                            uint8_t* keep, void* stream);

/*
 * The pages' own schedule, for measuring its HBM traffic (NOTE-005: FlashAttention, "Method" and
 * "Key results", Theorem 2: Theta(N^2 d^2 / M) HBM accesses for d <= M <= N d).  Same O and LSE as
 * fa_forward (no masks), computed with K/V blocks in the outer loop and Q blocks in the inner one;
 * O, m and l are kept in HBM (in the workspace, fp32) and read and written back for every block
 * pair.  Tiles follow the pages' rule with an LDS budget of lds_bytes held as fp32:
 * M = lds_bytes / 4 elements, B_c = ceil(M / 4d), B_r = min(B_c, d).  One workgroup per
 * (batch, head); fp32 vector arithmetic.  A measurement instrument, not a fast path.
 *   dtype must be FA_DTYPE_BF16; the tiles (2 B_c d + 2 B_r d + B_r B_c + 2 B_r floats) must fit in
 *   160 KiB of LDS and B_c >= 1, else FA_ERR_UNSUPPORTED.
 *   workspace: at least fa_forward_kv_outer_workspace_size() bytes, 16-byte aligned, scratch.
 */
size_t fa_forward_kv_outer_workspace_size(int B, int H, int N, int d);
fa_status_t fa_forward_kv_outer(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int N, int d, float scale, size_t lds_bytes, fa_dtype_t dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward with FP8 inputs, the step the pages name for FlashAttention-3 (the aicassindra FlashAttention
 * architecture page, "The architecture: every piece explained": FP8 support).  q8, k8, v8 are
 * OCP FP8 E4M3 bytes, [B][H][N][d] (d = 128 only), with per-tensor descales: the attention is that
 * of Q = descale_q q8, K = descale_k k8, V = descale_v v8.  S = scale Q K^T runs on the FP8 matrix
 * cores with fp32 accumulation (every FP8 product is exact in fp32); V is converted exactly to bf16
 * and P V runs as in the bf16 path.  o is bf16, lse fp32, masks as in fa_forward.
 *   Errors as in fa_forward; d != 128 -> FA_ERR_UNSUPPORTED; a descale that is not finite and
 *   positive -> FA_ERR_INVALID_ARGUMENT.
 */
fa_status_t fa_forward_fp8(const void* q8, const void* k8, const void* v8, float descale_q, float descale_k,
                           float descale_v, void* o, float* lse, int B, int H, int N, int d, float scale,
                           int causal, const int32_t* seqlens, void* stream);

/*
 * The backward without a caller workspace, for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid allocation).  Same arguments,
 * results and errors as fa_backward, minus workspace and workspace_bytes: the workspace is a
 * device array of FA_NOALLOC_WORKSPACE_BYTES held by the library, one per GPU, alive until the
 * process ends (its address on each GPU is resolved on the first call there).  Nothing is
 * allocated by the call.  Limit: fa_backward_workspace_size(B, H, N, d, dtype) must not exceed
 * FA_NOALLOC_WORKSPACE_BYTES (for bf16, B*H*N <= 1048576 rows; fp32, 2097152), else
 * FA_ERR_UNSUPPORTED before anything is enqueued.  Calls on one GPU share that array: two calls
 * whose work overlaps in time on the same GPU (different streams, or different host threads) race
 * and give undefined results; calls ordered on one stream do not.  The array needs no clearing:
 * every call writes each workspace value before reading it.
 */
#define FA_NOALLOC_WORKSPACE_BYTES (8 * 1024 * 1024)
fa_status_t fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dO, const float* lse, void* dq, void* dk, void* dv,
                                int B, int H, int N, int d, float scale, int causal,
                                const int32_t* seqlens, fa_dtype_t dtype, void* stream);

/*
 * Error reporting.  The pages warn that an attention integration can fall back to the naive
 * computation without saying so, and that it must be checked that the fused kernel is what runs
 * (aicassindra FlashAttention architecture page, "The architecture: every piece explained" and
 * "End-to-end flow"; stackzen glossary entry "FlashAttention").  This library therefore never
 * falls back: every condition it cannot serve is a status code, and these two calls say which.
 *
 * fa_status_string: a static, never-NULL name of a status code ("FA_ERR_UNKNOWN" for a value
 *   outside fa_status_t).  Thread-safe; the string is owned by the library and never freed.
 */
const char* fa_status_string(fa_status_t status);

/*
 * fa_last_error: detail of the last non-OK status returned on the calling thread: the failed
 *   check with the offending values, or the HIP runtime's error name and text; "" after a call
 *   that returned FA_OK.  The buffer is thread-local, owned by the library, valid until the next
 *   call on the same thread; never NULL.
 */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
