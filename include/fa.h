/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (forward and
 * backward passes).
 *
 * The operation is exact attention O = softmax(scale * Q K^T) V evaluated tile
 * by tile with the online softmax: a running row maximum m, a running
 * denominator l, rescaling of an unnormalised output accumulator by
 * exp(m_old - m_new) whenever the maximum grows, and a single division by l at
 * the end, so that no score or probability matrix is ever written to device
 * memory.  The method is the one described in "FlashAttention: Why Tiling
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
 *                  FA_MASK_WINDOW; non-finite scale; o overlapping q, k, v or
 *                  lse, or lse overlapping q, k or v; a size whose byte count
 *                  overflows, or a single head larger than 2 GiB.
 *   FA_EUNSUPPORTED (dtype, d) without a kernel.
 *   FA_EHIP        the launch failed; fa_last_error() holds the HIP message.
 * With the environment variable FA_LOG=1 each call prints the chosen kernel
 * and grid to stderr.
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
 * with d in {64, 128}.  fp32 products are accumulated in fp32 and each
 * gradient is rounded to nearest-even into `dtype` once, at the end.
 *
 * Ownership, stream order and determinism are as for fa_fwd (three kernel
 * launches on `stream`, no atomics: bit-identical results on every call).
 * Errors, all checked on the host before any launch:
 *   FA_EINVAL       a null or not 16-byte-aligned pointer; B, H, Hkv, S or d
 *                   < 1; Hkv not dividing H; unknown dtype or mask; window <
 *                   1 with FA_MASK_WINDOW; non-finite scale; any of dq, dk,
 *                   dv, delta overlapping an input or another of them; byte
 *                   counts that overflow, or one head larger than 2 GiB.
 *   FA_EUNSUPPORTED FA_F32, or d outside {64, 128}.
 *   FA_EHIP         a launch failed; fa_last_error() holds the HIP message.
 */
fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 const void *dout, void *dq, void *dk, void *dv, float *delta, int64_t B,
                 int64_t H, int64_t Hkv, int64_t S, int64_t d, int dtype, int mask,
                 int64_t window, float scale, void *stream);

/*
 * fa_query -- name the kernel instance fa_fwd would launch for (d, dtype,
 * mask), without launching anything or touching the GPU.  Writes a
 * NUL-terminated name into kernel_name[0..len) (truncated if needed; may be
 * NULL when len == 0).  Returns FA_OK, FA_EINVAL (bad enum or d < 1) or
 * FA_EUNSUPPORTED (no kernel for that combination).
 */
fa_status fa_query(int64_t d, int dtype, int mask, char *kernel_name, size_t len);

/* Static English text for a status code (never NULL). */
const char *fa_status_str(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none).  The string stays valid until the next fa_* call on that thread. */
const char *fa_last_error(void);

/* FA_ABI_VERSION of the loaded library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_TILED_FLASH_FA_H */
