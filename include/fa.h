/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (forward and
 * backward passes).
 *
 * The operation is exact attention O = softmax(scale * Q K^T) V evaluated tile
 * by tile with the online softmax: a running row offset m (the running
 * maximum's role), a running denominator l, rescaling of an unnormalised
 * output accumulator by exp(m_old - m_new) when m moves, and a single division
 * by l at the end, so that no score or probability matrix is ever written to
 * device memory.  (The bf16/fp16 forward kernels move m only when a tile's
 * weights would grow past a fixed bound, which gives the same result up to
 * rounding.)  The method is the one described in "FlashAttention: Why Tiling
 * Attention Makes Transformers Fast Without Changing the Result" (Dev.to),
 * sections "Online softmax: correct as you go" and "The tiled forward pass",
 * and in the aicomputerinstitute.com grade-12 chapter on flash attention,
 * section "Tiling and the running (online) softmax".  Its interface (Q, K, V
 * in device memory as [batch, heads, S, head_dim], a causal or sliding-window
 * mask, output O plus a per-row logsumexp) follows the foundry.adhana.ai page
 * "FlashAttention: IO-aware attention kernels", section "In and out".
 *
 * Every entry point is plain C: no C++ exception crosses it, no torch or HIP
 * type appears in it, and it is safe to call from several host threads (error
 * detail is kept per thread).
 */
#ifndef IO_AWARE_TILED_FLASH_FA_H
#define IO_AWARE_TILED_FLASH_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 1

/* Element type of q, k, v and o.  lse is always fp32. */
typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/*
 * Which keys j a query i may attend to (0-based positions, same sequence):
 *   FA_MASK_NONE   every j in [0, S);
 *   FA_MASK_CAUSAL j <= i;
 *   FA_MASK_WINDOW i - window < j <= i  (window >= 1 counts the diagonal;
 *                  window >= S is the causal mask).
 * Causal and sliding-window masks are the kinds the foundry.adhana.ai page
 * lists as natively supported ("The knobs", mask type); arbitrary boolean
 * masks are deliberately not offered.
 */
typedef enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1, FA_MASK_WINDOW = 2 } fa_mask;

/*
 * Status of every call.  A valid request that no kernel serves is an error
 * (FA_EUNSUPPORTED), never a quiet switch to a slower path: the
 * foundry.adhana.ai page, section "Failure modes", names the silent fallback
 * to unfused attention as the usual way the method's benefit is lost without
 * notice, and the Dev.to article's section "Using it in practice" warns that
 * the fast path is taken only when its conditions (dtype, head size, mask)
 * hold.
 */
typedef enum {
  FA_OK = 0,
  FA_EINVAL = 1,        /* an argument is invalid (see fa_fwd)                     */
  FA_EUNSUPPORTED = 2,  /* valid request with no kernel; there is never a fallback */
  FA_EHIP = 3           /* the HIP runtime reported an error on launch             */
} fa_status;

/*
 * fa_fwd -- launch the attention forward pass on `stream`.
 *
 * q, k, v : device pointers, [B, H, S, d] contiguous (d fastest), element type
 *           `dtype`.  Read only.
 * o       : device pointer, [B, H, S, d] contiguous, `dtype`.  Written:
 *           O[b,h,i,:] = sum_j P[i,j] V[b,h,j,:] with P the softmax over the
 *           visible keys of scale * (Q[b,h,i,:] . K[b,h,j,:]), rounded to
 *           nearest-even into `dtype`.
 * lse     : device pointer, [B, H, S] fp32.  Written: natural-log logsumexp
 *           of the visible scaled scores of each row (m + ln l).
 * B, H, S, d : sizes, all >= 1.  Supported head sizes: d in {64, 128, 256}
 *           for FA_F16 / FA_BF16; d in {64, 128} for FA_F32.
 * mask, window : see fa_mask; `window` is read only for FA_MASK_WINDOW and
 *           must then be >= 1.
 * scale   : finite multiplier applied in fp32 to Q.K (callers usually pass
 *           1/sqrt(d); there is no default inside the library).
 * stream  : a hipStream_t (NULL = the null stream).
 *
 * Ownership: the caller owns every buffer; the library allocates, frees and
 * copies nothing and keeps no pointer after returning.  The launch is
 * asynchronous in stream order; completion is observed by synchronising the
 * stream.  Results are deterministic: the same inputs give bit-identical
 * outputs on every call (no atomics).
 *
 * Errors (all checked on the host before any HIP call, so they can be tested
 * without a GPU; nothing is launched when one is returned):
 *   FA_EINVAL      null pointer; a pointer not 16-byte aligned; B, H, S or d
 *                  < 1; unknown dtype or mask; window < 1 with
 *                  FA_MASK_WINDOW; a scale that is not finite or whose
 *                  product with log2(e) overflows fp32 (|scale| above about
 *                  2.4e38: the kernels work in base 2); o overlapping q, k, v or
 *                  lse, or lse overlapping q, k or v; a size whose byte count
 *                  overflows, or a single head larger than 2 GiB.
 *   FA_EUNSUPPORTED (dtype, d) without a kernel.
 *   FA_EHIP        the launch failed; fa_last_error() holds the HIP message.
 * With the environment variable FA_LOG=1 each call prints the chosen kernel
 * and grid to stderr: the foundry.adhana.ai page, section "Evals", asks that
 * the backend actually selected be logged on every run, so that a measurement
 * can be tied to the kernel that produced it.
 */
fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                 int64_t B, int64_t H, int64_t S, int64_t d, int dtype, int mask,
                 int64_t window, float scale, void *stream);

/*
 * fa_fwd_gqa -- fa_fwd with grouped key/value heads (grouped-query attention;
 * multi-query attention when Hkv == 1).  The Dev.to article on FlashAttention,
 * section "Using it in practice", names grouped-query attention among the
 * patterns later variants of the method support; the computation per query
 * head is exactly fa_fwd's, against one shared key/value head.
 *
 * q, o    : [B, H, S, d] as in fa_fwd.
 * k, v    : [B, Hkv, S, d] contiguous, `dtype`.  Query head h of batch b
 *           attends with key/value head h / (H / Hkv) of batch b (contiguous
 *           groups of H / Hkv query heads share one key/value head).
 * lse     : [B, H, S] fp32, as in fa_fwd.
 * Hkv     : >= 1 and dividing H.  Hkv == H gives exactly fa_fwd.
 * Every other argument, the ownership rules and the error list are those of
 * fa_fwd; in addition FA_EINVAL is returned when Hkv < 1 or Hkv does not
 * divide H, and the overlap checks use the [B, Hkv, S, d] extent of k and v.
 */
fa_status fa_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse,
                     int64_t B, int64_t H, int64_t Hkv, int64_t S, int64_t d, int dtype,
                     int mask, int64_t window, float scale, void *stream);

/*
 * fa_bwd -- gradients of the attention forward pass (fa_fwd / fa_fwd_gqa with
 * the same q, k, v, B, H, Hkv, S, d, dtype, mask, window and scale) with
 * respect to q, k and v, given the gradient dout of its output.  The method is
 * the one in the Dev.to article "FlashAttention: Why Tiling Attention Makes
 * Transformers Fast Without Changing the Result", section "The backward pass:
 * recompute instead of storing": the probabilities are recomputed tile by tile
 * from q, k and the stored logsumexp, never stored, and
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = dO_i . O_i,
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * with P and dS restricted to the visible keys of the mask.  With grouped
 * key/value heads, dK and dV of key/value head g sum the contributions of its
 * H / Hkv query heads.
 *
 * q, dout : device, [B, H, S, d] contiguous, `dtype`.  Read only.
 * k, v    : device, [B, Hkv, S, d] contiguous, `dtype`.  Read only.
 * o, lse  : device; the forward pass's outputs for these arguments (o
 *           [B, H, S, d] `dtype`, lse [B, H, S] fp32).  Read only.  The
 *           gradients are those of the forward whose logsumexp is `lse`:
 *           pass the pair fa_fwd wrote.
 * dq      : device, [B, H, S, d] `dtype`.  Written.
 * dk, dv  : device, [B, Hkv, S, d] `dtype`.  Written (each element once, no
 *           accumulation into existing contents).
 * delta   : device, [B, H, S] fp32 workspace owned by the caller.  Written
 *           with D_i (fp32) and read back by the later kernels of this call;
 *           its contents on return are those row terms.
 * Hkv     : >= 1 and dividing H (Hkv == H: multi-head attention).
 * Every other argument is read as by fa_fwd.  Supported: FA_F16 / FA_BF16
 * with d in {64, 128, 256}.  fp32 products are accumulated in fp32 and each
 * gradient is rounded to nearest-even into `dtype` once, at the end.
 *
 * Ownership, stream order and determinism are as for fa_fwd (three kernel
 * launches on `stream`, no atomics: bit-identical results on every call).
 * Errors, all checked on the host before any launch:
 *   FA_EINVAL       a null or not 16-byte-aligned pointer; B, H, Hkv, S or d
 *                   < 1; Hkv not dividing H; unknown dtype or mask; window <
 *                   1 with FA_MASK_WINDOW; a scale rejected as by fa_fwd; any of dq, dk,
 *                   dv, delta overlapping an input or another of them; byte
 *                   counts that overflow, or one head larger than 2 GiB.
 *   FA_EUNSUPPORTED FA_F32, or d outside {64, 128, 256}.
 *   FA_EHIP         a launch failed; fa_last_error() holds the HIP message.
 */
fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 const void *dout, void *dq, void *dk, void *dv, float *delta, int64_t B,
                 int64_t H, int64_t Hkv, int64_t S, int64_t d, int dtype, int mask,
                 int64_t window, float scale, void *stream);

/*
 * fa_decode_paged -- attention of a few new tokens per request over a paged
 * key/value cache (decoding).  The aicomputerinstitute.com grade-12 chapter on
 * flash attention, sections "A different bottleneck: the KV cache during
 * inference" and "PagedAttention: memory management borrowed from an
 * operating system", describes the layout: the cache is cut into fixed-size
 * physical blocks stored anywhere, and each request's block table maps its
 * logical token positions to blocks, which the kernel walks and gathers.
 *
 * For request b with n_b = min(max(ctx_lens[b], 0), max_ctx, max_blocks *
 * block_size) cached tokens:
 *   token t < n_b lives in physical block P = block_table[b * max_blocks +
 *   t / block_size], slot t % block_size; a table entry outside
 *   [0, num_blocks) holds no token (its positions are skipped, never read);
 *   query row i (0 <= i < n_q) is the token at position n_b - n_q + i, whose
 *   key and value are already cached, and attends to positions t <= n_b -
 *   n_q + i (with n_q = 1: every cached token);
 *   query head h uses key/value head h / (H / Hkv).
 * O and lse are the exact attention of each row over its visible tokens
 * (softmax of scale * q.k, as fa_fwd); a row with no visible token gets O = 0
 * and lse = -inf.
 *
 * q, o       : device, [B, H, n_q, d] contiguous, `dtype` (o written).
 * k_cache, v_cache : device, [num_blocks, Hkv, block_size, d] contiguous,
 *              `dtype`.  Read only; only the slots of valid tokens are read.
 * block_table: device int32 [B, max_blocks].   ctx_lens: device int32 [B].
 * lse        : device fp32 [B, H, n_q] (written, natural log).
 * workspace, workspace_bytes : device scratch for the partial results of
 *              long contexts, split over several work-groups and merged; the
 *              size is given by fa_decode_workspace_size for the same sizes
 *              (0 when no split is needed: workspace may then be NULL).  Its
 *              contents are undefined before and after the call.
 * max_ctx    : an upper bound the caller guarantees for the context lengths
 *              (host value; it sizes the split and the workspace).  Longer
 *              contexts are cut to max_ctx tokens.
 * block_size : a power of two, 1 .. 1024.
 * Supported: FA_F16 / FA_BF16 with d in {64, 128, 256} (at 256 every row
 *            count runs on the vector kernel).
 *
 * Ownership, stream order and determinism as for fa_fwd (one or two launches).
 * Errors, checked on the host before any launch:
 *   FA_EINVAL       a null pointer (workspace only when needed); q, caches,
 *                   o or workspace not 16-byte aligned, block_table, ctx_lens
 *                   or lse not 4-byte aligned; B, H, Hkv, n_q, d, num_blocks,
 *                   block_size or max_blocks < 1; max_ctx < 0; Hkv not
 *                   dividing H; unknown dtype; a scale rejected as by fa_fwd; workspace
 *                   smaller than required; o, lse or workspace overlapping an
 *                   input or each other; sizes beyond the kernels' index range.
 *   FA_EUNSUPPORTED FA_F32, d outside {64, 128, 256}, or a block_size that is not a
 *                   power of two up to 1024.
 *   FA_EHIP         a launch failed.
 * Values inside block_table and ctx_lens are device data and are never
 * checked on the host; out-of-range entries are handled as described above.
 */
fa_status fa_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *block_table, const int32_t *ctx_lens, void *o,
                          float *lse, void *workspace, size_t workspace_bytes, int64_t B,
                          int64_t H, int64_t Hkv, int64_t n_q, int64_t d, int64_t num_blocks,
                          int64_t block_size, int64_t max_blocks, int64_t max_ctx, int dtype,
                          float scale, void *stream);

/*
 * fa_decode_paged_noalloc -- fa_decode_paged for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It takes no workspace argument and allocates
 * nothing (no hipMalloc, no hipFree, no allocating library call): the split
 * workspace is a static device array of FA_NOALLOC_SCRATCH_BYTES that the
 * library owns, one copy per GPU, held until the process ends.  Its device
 * address is looked up once per device, on the first call made with that
 * device current.
 *
 * Arguments, results, ownership of the caller's buffers and every error of
 * fa_decode_paged apply (without the workspace rules), and the kernels and
 * results are the same, bit for bit.  In addition:
 *   FA_EINVAL  the sizes need a split workspace larger than
 *              FA_NOALLOC_SCRATCH_BYTES (fa_decode_workspace_size reports
 *              the need; such sizes must use fa_decode_paged);
 *   FA_EHIP    the scratch's device address could not be looked up.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's partial results: calls whose executions overlap on one GPU (on
 * different streams, or from different threads without ordering) race and
 * may return wrong results.  Calls ordered on one stream are safe.  No part
 * of the scratch needs to start cleared: the kernels write every slot they
 * read within the same call.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
fa_status fa_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_table, const int32_t *ctx_lens, void *o,
                                  float *lse, int64_t B, int64_t H, int64_t Hkv, int64_t n_q,
                                  int64_t d, int64_t num_blocks, int64_t block_size,
                                  int64_t max_blocks, int64_t max_ctx, int dtype, float scale,
                                  void *stream);

/*
 * fa_decode_workspace_size -- bytes of workspace fa_decode_paged needs for
 * these sizes (written to *bytes; 0 when none).  Same size checks and error
 * codes as fa_decode_paged; touches no device memory.
 */
fa_status fa_decode_workspace_size(int64_t B, int64_t H, int64_t Hkv, int64_t n_q, int64_t d,
                                   int64_t num_blocks, int64_t block_size, int64_t max_blocks,
                                   int64_t max_ctx, int dtype, size_t *bytes);

/*
 * fa_query -- name the kernel instance fa_fwd would launch for (d, dtype,
 * mask), without launching anything or touching the GPU.  Writes a
 * NUL-terminated name into kernel_name[0..len) (truncated if needed; may be
 * NULL when len == 0).  Returns FA_OK, FA_EINVAL (bad enum or d < 1) or
 * FA_EUNSUPPORTED (no kernel for that combination).
 * Purpose: the Dev.to article's section "Using it in practice" tells the
 * user to verify which attention implementation is dispatched rather than
 * assume the fast one runs; the foundry.adhana.ai page's "Evals" section
 * makes the same check part of every evaluation.  This call answers that
 * question before any launch.
 */
fa_status fa_query(int64_t d, int dtype, int mask, char *kernel_name, size_t len);

/*
 * fa_query_fwd -- like fa_query, for the sizes of one fa_fwd / fa_fwd_gqa
 * call: names the kernel instance that call would launch (the instance can
 * depend on the sizes: grids too small to fill the chip split the keys of
 * each query tile over several waves) and, when grid is not NULL, stores its
 * number of work-groups.  Launches nothing and touches no device.  Returns
 * FA_OK, FA_EINVAL (the size, enum and window checks of fa_fwd) or
 * FA_EUNSUPPORTED.  Same purpose as fa_query (Dev.to, "Using it in
 * practice", "Verify the dispatch").
 */
fa_status fa_query_fwd(int64_t B, int64_t H, int64_t Hkv, int64_t S, int64_t d, int dtype,
                       int mask, int64_t window, char *kernel_name, size_t len,
                       int64_t *grid);

/*
 * fa_status_str -- static English text for a status code (never NULL).
 * fa_last_error -- detail of the last non-OK status returned on the calling
 * thread ("" if none), e.g. which (dtype, head size) has no kernel; the
 * string stays valid until the next fa_* call on that thread.
 * Both exist so that an unsupported or invalid request fails loudly and says
 * why, which is what the foundry.adhana.ai page ("Failure modes") asks of a
 * fused-attention path instead of a silent fallback.
 */
const char *fa_status_str(int status);
const char *fa_last_error(void);

/*
 * fa_abi_version -- FA_ABI_VERSION of the loaded library.  A binding checks
 * it before its first call, so that a stale library is an error rather than
 * a different kernel running unnoticed (the same "verify the dispatch" check
 * as fa_query, Dev.to "Using it in practice").
 */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_TILED_FLASH_FA_H */
