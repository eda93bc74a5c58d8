// C ABI of the attention library (forward and backward): argument validation, choice of the
// kernel instance, launch, and per-thread error text.
//
// Unsupported requests are errors, never a silent switch to a slower path:
// the foundry.adhana.ai page "FlashAttention: IO-aware attention kernels"
// (sections "Evals" and "Failure modes") describes such silent fallbacks as
// the failure that corrupts measurements, and recommends logging which kernel
// ran; FA_LOG=1 does that here.
#include "../../include/fa.h"
#include "fa_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

// Split workspace of fa_decode_paged_noalloc: device memory the library owns,
// so that callers which cannot allocate (code under graph capture, tight
// serving loops) need not pass any.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code this name is only a
// stand-in for the symbol: its device address on the current device comes
// from hipGetSymbolAddress (decode_scratch below), and only that address is
// ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512];

fa_status fail(fa_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool log_enabled() {
  static int cached = -1;
  if (cached < 0) {
    const char *e = getenv("FA_LOG");
    cached = (e && e[0] && strcmp(e, "0") != 0) ? 1 : 0;
  }
  return cached == 1;
}

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  const uint64_t x = (uint64_t)(uintptr_t)a, y = (uint64_t)(uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }

// The kernels work in base 2 on scale * log2(e), rounded to fp32: a finite
// scale above about 2.4e38 would turn that factor into inf, and inf times a
// zero score into NaN.
constexpr double kLog2e = 1.4426950408889634;
bool scale_ok(float scale) {
  return isfinite(scale) && isfinite((float)((double)scale * kLog2e));
}

// Resolve (dtype, d, mask) to a kernel; `launch` false only fills `info`.
bool dispatch(int dtype, int d, int mask, const fa::FwdArgs *a, hipStream_t stream, bool launch,
              fa::LaunchInfo *info, hipError_t *err) {
  if (dtype == FA_F32) return fa::f32_forward(d, mask, a, stream, launch, info, err);
  return fa::mfma_forward(dtype == FA_BF16 ? fa::kBF16 : fa::kF16, d, mask, a, stream, launch,
                          info, err);
}

const char *dtype_name(int dt) {
  return dt == FA_F32 ? "f32" : dt == FA_F16 ? "f16" : dt == FA_BF16 ? "bf16" : "?";
}

// The forward pass for H query heads over Hkv key/value heads (Hkv == H is
// plain multi-head attention).  `name` labels log lines.
fa_status fwd_impl(const char *name, const void *q, const void *k, const void *v, void *o,
                   float *lse, int64_t B, int64_t H, int64_t Hkv, int64_t S, int64_t d,
                   int dtype, int mask, int64_t window, float scale, void *stream) {
  g_err[0] = '\0';
  if (!q || !k || !v || !o || !lse) return fail(FA_EINVAL, "null pointer argument");
  const void *ptrs[5] = {q, k, v, o, lse};
  for (int i = 0; i < 5; ++i)
    if ((uintptr_t)ptrs[i] % 16 != 0)
      return fail(FA_EINVAL, "pointer argument %d is not 16-byte aligned", i);
  if (B < 1 || H < 1 || Hkv < 1 || S < 1 || d < 1)
    return fail(FA_EINVAL, "sizes must be >= 1 (B=%lld H=%lld Hkv=%lld S=%lld d=%lld)",
                (long long)B, (long long)H, (long long)Hkv, (long long)S, (long long)d);
  if (H % Hkv != 0)
    return fail(FA_EINVAL, "key/value heads (%lld) must divide query heads (%lld)",
                (long long)Hkv, (long long)H);
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_EINVAL, "unknown dtype %d", dtype);
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_WINDOW)
    return fail(FA_EINVAL, "unknown mask %d", mask);
  if (mask == FA_MASK_WINDOW && window < 1)
    return fail(FA_EINVAL, "window must be >= 1 for the sliding-window mask (got %lld)",
                (long long)window);
  if (!scale_ok(scale))
    return fail(FA_EINVAL, "scale must be finite, with scale*log2(e) finite in fp32 (got %g)",
                (double)scale);

  const int64_t esz = dtype == FA_F32 ? 4 : 2;
  int64_t bh, rows, elems, bytes, row_bytes, head_bytes, lse_bytes, bhkv, kv_bytes;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, S, &rows) || !mul_ok(rows, d, &elems) ||
      !mul_ok(elems, esz, &bytes) || !mul_ok(rows, 4, &lse_bytes) ||
      !mul_ok(d, esz, &row_bytes) || !mul_ok(S, row_bytes, &head_bytes) ||
      !mul_ok(B, Hkv, &bhkv) || !mul_ok(bhkv, head_bytes, &kv_bytes))
    return fail(FA_EINVAL, "tensor size overflows 64-bit byte counts");
  if (head_bytes > (int64_t)INT32_MAX)
    return fail(FA_EINVAL, "one head's [S, d] slab (%lld bytes) exceeds 2 GiB",
                (long long)head_bytes);
  if (bh > (int64_t)INT32_MAX || rows > (int64_t)INT64_MAX / 2)
    return fail(FA_EINVAL, "batch*heads too large");
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, kv_bytes) ||
      overlaps(o, bytes, v, kv_bytes) || overlaps(o, bytes, lse, lse_bytes))
    return fail(FA_EINVAL, "output o overlaps an input or lse");
  if (overlaps(lse, lse_bytes, q, bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
      overlaps(lse, lse_bytes, v, kv_bytes))
    return fail(FA_EINVAL, "lse overlaps an input");

  // A window that covers the whole sequence is the causal mask.
  int eff_mask = mask;
  if (mask == FA_MASK_WINDOW && window >= S) eff_mask = FA_MASK_CAUSAL;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = (int)B;
  a.H = (int)H;
  a.Hkv = (int)Hkv;
  a.S = (int)S;
  a.window = eff_mask == FA_MASK_WINDOW ? (int)window : 0;
  a.scale_log2 = (float)((double)scale * kLog2e);

  fa::LaunchInfo info = {nullptr, 0, 0};
  hipError_t err = hipSuccess;
  if (!dispatch(dtype, (int)d, eff_mask, &a, nullptr, false, &info, &err))
    return fail(FA_EUNSUPPORTED, "no kernel for dtype=%s d=%lld (supported: bf16/f16 with d in "
                "{64,128,256}; f32 with d in {64,128})", dtype_name(dtype), (long long)d);
  const int64_t nq = (S + info.block_rows - 1) / info.block_rows;
  if (nq * bh > (int64_t)INT32_MAX) return fail(FA_EINVAL, "grid too large");

  if (log_enabled())
    fprintf(stderr, "%s: kernel=%s grid=%lld block=%d B=%lld H=%lld Hkv=%lld S=%lld d=%lld\n",
            name, info.name, (long long)(nq * bh), info.threads, (long long)B, (long long)H,
            (long long)Hkv, (long long)S, (long long)d);

  dispatch(dtype, (int)d, eff_mask, &a, (hipStream_t)stream, true, &info, &err);
  if (err != hipSuccess)
    return fail(FA_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

// The backward pass (gradients of the forward pass with the same
// arguments); Hkv == H is plain multi-head attention.
fa_status bwd_impl(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv, float *delta, int64_t B,
                   int64_t H, int64_t Hkv, int64_t S, int64_t d, int dtype, int mask,
                   int64_t window, float scale, void *stream) {
  g_err[0] = '\0';
  const void *ptrs[10] = {q, k, v, o, lse, dout, dq, dk, dv, delta};
  for (int i = 0; i < 10; ++i) {
    if (!ptrs[i]) return fail(FA_EINVAL, "null pointer argument %d", i);
    if ((uintptr_t)ptrs[i] % 16 != 0)
      return fail(FA_EINVAL, "pointer argument %d is not 16-byte aligned", i);
  }
  if (B < 1 || H < 1 || Hkv < 1 || S < 1 || d < 1)
    return fail(FA_EINVAL, "sizes must be >= 1 (B=%lld H=%lld Hkv=%lld S=%lld d=%lld)",
                (long long)B, (long long)H, (long long)Hkv, (long long)S, (long long)d);
  if (H % Hkv != 0)
    return fail(FA_EINVAL, "key/value heads (%lld) must divide query heads (%lld)",
                (long long)Hkv, (long long)H);
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_EINVAL, "unknown dtype %d", dtype);
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_WINDOW)
    return fail(FA_EINVAL, "unknown mask %d", mask);
  if (mask == FA_MASK_WINDOW && window < 1)
    return fail(FA_EINVAL, "window must be >= 1 for the sliding-window mask (got %lld)",
                (long long)window);
  if (!scale_ok(scale))
    return fail(FA_EINVAL, "scale must be finite, with scale*log2(e) finite in fp32 (got %g)",
                (double)scale);

  const int64_t esz = dtype == FA_F32 ? 4 : 2;
  int64_t bh, rows, elems, bytes, row_bytes, head_bytes, stat_bytes, bhkv, kv_bytes;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, S, &rows) || !mul_ok(rows, d, &elems) ||
      !mul_ok(elems, esz, &bytes) || !mul_ok(rows, 4, &stat_bytes) ||
      !mul_ok(d, esz, &row_bytes) || !mul_ok(S, row_bytes, &head_bytes) ||
      !mul_ok(B, Hkv, &bhkv) || !mul_ok(bhkv, head_bytes, &kv_bytes))
    return fail(FA_EINVAL, "tensor size overflows 64-bit byte counts");
  if (head_bytes > (int64_t)INT32_MAX)
    return fail(FA_EINVAL, "one head's [S, d] slab (%lld bytes) exceeds 2 GiB",
                (long long)head_bytes);
  if (bh > (int64_t)INT32_MAX) return fail(FA_EINVAL, "batch*heads too large");
  // Written buffers may overlap neither each other nor any input.
  const void *outs[4] = {dq, dk, dv, delta};
  const int64_t out_n[4] = {bytes, kv_bytes, kv_bytes, stat_bytes};
  const void *ins[6] = {q, k, v, o, lse, dout};
  const int64_t in_n[6] = {bytes, kv_bytes, kv_bytes, bytes, stat_bytes, bytes};
  static const char *out_names[4] = {"dq", "dk", "dv", "delta"};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j]))
        return fail(FA_EINVAL, "output %s overlaps an input", out_names[i]);
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j]))
        return fail(FA_EINVAL, "outputs %s and %s overlap", out_names[i], out_names[j]);
  }

  int eff_mask = mask;
  if (mask == FA_MASK_WINDOW && window >= S) eff_mask = FA_MASK_CAUSAL;

  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.B = (int)B;
  a.H = (int)H;
  a.Hkv = (int)Hkv;
  a.S = (int)S;
  a.window = eff_mask == FA_MASK_WINDOW ? (int)window : 0;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * kLog2e);

  fa::LaunchInfo info = {nullptr, 0, 0};
  hipError_t err = hipSuccess;
  const fa::DType dt = dtype == FA_BF16 ? fa::kBF16 : fa::kF16;
  if (dtype == FA_F32 || !fa::mfma_backward(dt, (int)d, eff_mask, &a, nullptr, false, &info, &err))
    return fail(FA_EUNSUPPORTED, "no backward kernel for dtype=%s d=%lld (supported: bf16/f16 "
                "with d in {64,128,256})", dtype_name(dtype), (long long)d);
  const int64_t nt = (S + info.block_rows - 1) / info.block_rows;
  // at d = 256 two dK/dV work-groups share each key tile; the row-term
  // kernel takes 2048 / d rows per work-group
  if (nt * bh * (d == 256 ? 2 : 1) > (int64_t)INT32_MAX ||
      rows / (2048 / d) + 1 > (int64_t)INT32_MAX)
    return fail(FA_EINVAL, "grid too large");

  if (log_enabled())
    fprintf(stderr, "fa_bwd: kernel=%s tiles=%lld block=%d B=%lld H=%lld Hkv=%lld S=%lld d=%lld\n",
            info.name, (long long)nt, info.threads, (long long)B, (long long)H, (long long)Hkv,
            (long long)S, (long long)d);

  fa::mfma_backward(dt, (int)d, eff_mask, &a, (hipStream_t)stream, true, &info, &err);
  if (err != hipSuccess)
    return fail(FA_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

// Shared size checks of the decode entry points; fills the plan.
fa_status decode_sizes(int64_t B, int64_t H, int64_t Hkv, int64_t n_q, int64_t d,
                       int64_t num_blocks, int64_t block_size, int64_t max_blocks,
                       int64_t max_ctx, int dtype, int *bs_shift, int64_t *ctx_cap,
                       fa::DecodePlan *plan) {
  if (B < 1 || H < 1 || Hkv < 1 || n_q < 1 || d < 1 || num_blocks < 1 || block_size < 1 ||
      max_blocks < 1)
    return fail(FA_EINVAL, "sizes must be >= 1 (B=%lld H=%lld Hkv=%lld n_q=%lld d=%lld "
                "num_blocks=%lld block_size=%lld max_blocks=%lld)", (long long)B, (long long)H,
                (long long)Hkv, (long long)n_q, (long long)d, (long long)num_blocks,
                (long long)block_size, (long long)max_blocks);
  if (max_ctx < 0) return fail(FA_EINVAL, "max_ctx must be >= 0 (got %lld)", (long long)max_ctx);
  if (H % Hkv != 0)
    return fail(FA_EINVAL, "key/value heads (%lld) must divide query heads (%lld)",
                (long long)Hkv, (long long)H);
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_EINVAL, "unknown dtype %d", dtype);
  int sh = 0;
  while (sh < 10 && (int64_t(1) << sh) < block_size) ++sh;
  if ((int64_t(1) << sh) != block_size)
    return fail(FA_EUNSUPPORTED, "no decode kernel for block_size=%lld (supported: powers of "
                "two up to 1024)", (long long)block_size);
  int64_t cap, bhq, bhqd, tab, t;
  if (!mul_ok(max_blocks, block_size, &cap) || !mul_ok(B, H, &bhq) || !mul_ok(bhq, n_q, &bhq) ||
      !mul_ok(bhq, d, &bhqd) || !mul_ok(B, max_blocks, &tab) || !mul_ok(num_blocks, Hkv, &t) ||
      !mul_ok(t, block_size, &t) || !mul_ok(t, d, &t) || !mul_ok(t, 2, &t))
    return fail(FA_EINVAL, "tensor size overflows 64-bit byte counts");
  if (cap > INT32_MAX || tab > INT32_MAX || bhqd > INT32_MAX || num_blocks > INT32_MAX ||
      n_q > 65536)
    return fail(FA_EINVAL, "sizes exceed the 32-bit index range of the decode kernels");
  if (max_ctx < cap) cap = max_ctx;
  if (dtype == FA_F32 || !fa::decode_plan((int)d, B, H, Hkv, n_q, cap, plan))
    return fail(FA_EUNSUPPORTED, "no decode kernel for dtype=%s d=%lld (supported: bf16/f16 "
                "with d in {64,128,256})", dtype_name(dtype), (long long)d);
  if (plan->grid > INT32_MAX) return fail(FA_EINVAL, "grid too large");
  *bs_shift = sh;
  *ctx_cap = cap;
  return FA_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

fa_status decode_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_EUNSUPPORTED, "device %d is beyond the %d devices the scratch table holds",
                dev, kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return fail(FA_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(g_scratch_err[dev]));
  *ptr = g_scratch_ptr[dev];
  return FA_OK;
}

// The decode launch.  With use_scratch the split workspace is the library's
// own `scratch` (workspace and workspace_bytes are ignored), else the
// caller's.
fa_status decode_impl(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_table, const int32_t *ctx_lens, void *o, float *lse,
                      void *workspace, size_t workspace_bytes, int64_t B, int64_t H,
                      int64_t Hkv, int64_t n_q, int64_t d, int64_t num_blocks,
                      int64_t block_size, int64_t max_blocks, int64_t max_ctx, int dtype,
                      float scale, void *stream, bool use_scratch) {
  g_err[0] = '\0';
  const void *need16[4] = {q, k_cache, v_cache, o};
  for (int i = 0; i < 4; ++i) {
    if (!need16[i]) return fail(FA_EINVAL, "null pointer argument (q, k_cache, v_cache or o)");
    if ((uintptr_t)need16[i] % 16 != 0)
      return fail(FA_EINVAL, "pointer argument %d is not 16-byte aligned", i);
  }
  const void *need4[3] = {block_table, ctx_lens, lse};
  for (int i = 0; i < 3; ++i) {
    if (!need4[i]) return fail(FA_EINVAL, "null pointer argument (block_table, ctx_lens or lse)");
    if ((uintptr_t)need4[i] % 4 != 0)
      return fail(FA_EINVAL, "block_table, ctx_lens and lse must be 4-byte aligned");
  }
  if (!scale_ok(scale))
    return fail(FA_EINVAL, "scale must be finite, with scale*log2(e) finite in fp32 (got %g)",
                (double)scale);
  int sh = 0;
  int64_t cap = 0;
  fa::DecodePlan plan;
  fa_status st = decode_sizes(B, H, Hkv, n_q, d, num_blocks, block_size, max_blocks, max_ctx,
                              dtype, &sh, &cap, &plan);
  if (st != FA_OK) return st;
  if (use_scratch) {
    workspace = nullptr;
    workspace_bytes = 0;
    if (plan.ws_bytes > (int64_t)FA_NOALLOC_SCRATCH_BYTES)
      return fail(FA_EINVAL, "these sizes need %lld bytes of split workspace, more than the "
                  "%lld-byte scratch of fa_decode_paged_noalloc (use fa_decode_paged with a "
                  "workspace)", (long long)plan.ws_bytes, (long long)FA_NOALLOC_SCRATCH_BYTES);
  } else if (plan.ws_bytes > 0) {
    if (!workspace || (uintptr_t)workspace % 16 != 0)
      return fail(FA_EINVAL, "this launch needs a 16-byte-aligned workspace of %lld bytes",
                  (long long)plan.ws_bytes);
    if ((int64_t)workspace_bytes < plan.ws_bytes)
      return fail(FA_EINVAL, "workspace too small: %zu bytes given, %lld needed", workspace_bytes,
                  (long long)plan.ws_bytes);
  }
  const int64_t esz = 2;
  const int64_t q_bytes = B * H * n_q * d * esz, lse_bytes = B * H * n_q * 4;
  const int64_t cache_bytes = num_blocks * Hkv * block_size * d * esz;
  const int64_t table_bytes = B * max_blocks * 4, ctx_bytes = B * 4;
  const void *ins[5] = {q, k_cache, v_cache, block_table, ctx_lens};
  const int64_t in_n[5] = {q_bytes, cache_bytes, cache_bytes, table_bytes, ctx_bytes};
  const void *outs[3] = {o, lse, workspace};
  // (the library's own scratch cannot overlap the caller's buffers)
  const int64_t out_n[3] = {q_bytes, lse_bytes, use_scratch ? 0 : plan.ws_bytes};
  static const char *out_names[3] = {"o", "lse", "workspace"};
  for (int i = 0; i < 3; ++i) {
    if (out_n[i] == 0) continue;
    for (int j = 0; j < 5; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j]))
        return fail(FA_EINVAL, "%s overlaps an input", out_names[i]);
    for (int j = i + 1; j < 3; ++j)
      if (out_n[j] > 0 && overlaps(outs[i], out_n[i], outs[j], out_n[j]))
        return fail(FA_EINVAL, "%s and %s overlap", out_names[i], out_names[j]);
  }

  if (use_scratch && plan.ws_bytes > 0) {
    st = decode_scratch(&workspace);
    if (st != FA_OK) return st;
  }

  fa::DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.o = o;
  a.lse = lse;
  a.ws_o = plan.ws_bytes > 0 ? (float *)workspace : nullptr;
  a.ws_lse = plan.ws_bytes > 0 ? (float *)workspace + B * H * n_q * plan.n_splits * d : nullptr;
  a.B = (int)B;
  a.H = (int)H;
  a.Hkv = (int)Hkv;
  a.n_q = (int)n_q;
  a.num_blocks = (int)num_blocks;
  a.bs_shift = sh;
  a.max_blocks = (int)max_blocks;
  a.ctx_cap = (int)cap;
  a.split_len = plan.split_len;
  a.n_splits = plan.n_splits;
  a.rows = plan.rows;
  a.row_slices = plan.row_slices;
  a.scale_log2 = (float)((double)scale * kLog2e);

  fa::LaunchInfo info = {nullptr, 0, 0};
  hipError_t err = hipSuccess;
  const fa::DType dt = dtype == FA_BF16 ? fa::kBF16 : fa::kF16;
  fa::decode_paged(dt, (int)d, &a, &plan, nullptr, false, &info, &err);
  if (log_enabled())
    fprintf(stderr, "fa_decode_paged: kernel=%s grid=%lld splits=%d split_len=%d row_slices=%d "
            "B=%lld H=%lld Hkv=%lld n_q=%lld d=%lld block_size=%lld\n", info.name,
            (long long)plan.grid, plan.n_splits, plan.split_len, plan.row_slices, (long long)B,
            (long long)H, (long long)Hkv, (long long)n_q, (long long)d, (long long)block_size);
  fa::decode_paged(dt, (int)d, &a, &plan, (hipStream_t)stream, true, &info, &err);
  if (err != hipSuccess)
    return fail(FA_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                 int64_t H, int64_t S, int64_t d, int dtype, int mask, int64_t window,
                 float scale, void *stream) {
  return fwd_impl("fa_fwd", q, k, v, o, lse, B, H, H, S, d, dtype, mask, window, scale,
                  stream);
}

fa_status fa_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse,
                     int64_t B, int64_t H, int64_t Hkv, int64_t S, int64_t d, int dtype,
                     int mask, int64_t window, float scale, void *stream) {
  return fwd_impl("fa_fwd_gqa", q, k, v, o, lse, B, H, Hkv, S, d, dtype, mask, window, scale,
                  stream);
}

fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 const void *dout, void *dq, void *dk, void *dv, float *delta, int64_t B,
                 int64_t H, int64_t Hkv, int64_t S, int64_t d, int dtype, int mask,
                 int64_t window, float scale, void *stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, S, d, dtype, mask, window,
                  scale, stream);
}

fa_status fa_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *block_table, const int32_t *ctx_lens, void *o,
                          float *lse, void *workspace, size_t workspace_bytes, int64_t B,
                          int64_t H, int64_t Hkv, int64_t n_q, int64_t d, int64_t num_blocks,
                          int64_t block_size, int64_t max_blocks, int64_t max_ctx, int dtype,
                          float scale, void *stream) {
  return decode_impl(q, k_cache, v_cache, block_table, ctx_lens, o, lse, workspace,
                     workspace_bytes, B, H, Hkv, n_q, d, num_blocks, block_size, max_blocks,
                     max_ctx, dtype, scale, stream, false);
}

fa_status fa_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_table, const int32_t *ctx_lens, void *o,
                                  float *lse, int64_t B, int64_t H, int64_t Hkv, int64_t n_q,
                                  int64_t d, int64_t num_blocks, int64_t block_size,
                                  int64_t max_blocks, int64_t max_ctx, int dtype, float scale,
                                  void *stream) {
  return decode_impl(q, k_cache, v_cache, block_table, ctx_lens, o, lse, nullptr, 0, B, H, Hkv,
                     n_q, d, num_blocks, block_size, max_blocks, max_ctx, dtype, scale, stream,
                     true);
}

fa_status fa_decode_workspace_size(int64_t B, int64_t H, int64_t Hkv, int64_t n_q, int64_t d,
                                   int64_t num_blocks, int64_t block_size, int64_t max_blocks,
                                   int64_t max_ctx, int dtype, size_t *bytes) {
  g_err[0] = '\0';
  if (!bytes) return fail(FA_EINVAL, "null pointer argument");
  int sh = 0;
  int64_t cap = 0;
  fa::DecodePlan plan;
  fa_status st = decode_sizes(B, H, Hkv, n_q, d, num_blocks, block_size, max_blocks, max_ctx,
                              dtype, &sh, &cap, &plan);
  if (st != FA_OK) return st;
  *bytes = (size_t)plan.ws_bytes;
  return FA_OK;
}

fa_status fa_query(int64_t d, int dtype, int mask, char *kernel_name, size_t len) {
  g_err[0] = '\0';
  if (d < 1) return fail(FA_EINVAL, "d must be >= 1");
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_EINVAL, "unknown dtype %d", dtype);
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_WINDOW)
    return fail(FA_EINVAL, "unknown mask %d", mask);
  if (len > 0 && !kernel_name) return fail(FA_EINVAL, "null name buffer");
  fa::LaunchInfo info = {nullptr, 0, 0};
  hipError_t err = hipSuccess;
  if (d > INT32_MAX || !dispatch(dtype, (int)d, mask, nullptr, nullptr, false, &info, &err))
    return fail(FA_EUNSUPPORTED, "no kernel for dtype=%s d=%lld", dtype_name(dtype),
                (long long)d);
  if (len > 0) {
    strncpy(kernel_name, info.name, len - 1);
    kernel_name[len - 1] = '\0';
  }
  return FA_OK;
}

fa_status fa_query_fwd(int64_t B, int64_t H, int64_t Hkv, int64_t S, int64_t d, int dtype,
                       int mask, int64_t window, char *kernel_name, size_t len,
                       int64_t *grid) {
  g_err[0] = '\0';
  if (B < 1 || H < 1 || Hkv < 1 || S < 1 || d < 1)
    return fail(FA_EINVAL, "sizes must be >= 1");
  if (H % Hkv != 0) return fail(FA_EINVAL, "key/value heads must divide query heads");
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_EINVAL, "unknown dtype %d", dtype);
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_WINDOW)
    return fail(FA_EINVAL, "unknown mask %d", mask);
  if (mask == FA_MASK_WINDOW && window < 1) return fail(FA_EINVAL, "window must be >= 1");
  if (len > 0 && !kernel_name) return fail(FA_EINVAL, "null name buffer");
  int64_t bh;
  if (!mul_ok(B, H, &bh) || bh > (int64_t)INT32_MAX || S > (int64_t)INT32_MAX ||
      d > (int64_t)INT32_MAX)
    return fail(FA_EINVAL, "sizes too large");
  const int eff_mask = (mask == FA_MASK_WINDOW && window >= S) ? FA_MASK_CAUSAL : mask;
  fa::FwdArgs a = {};
  a.B = (int)B;
  a.H = (int)H;
  a.Hkv = (int)Hkv;
  a.S = (int)S;
  a.window = eff_mask == FA_MASK_WINDOW ? (int)window : 0;
  fa::LaunchInfo info = {nullptr, 0, 0};
  hipError_t err = hipSuccess;
  if (!dispatch(dtype, (int)d, eff_mask, &a, nullptr, false, &info, &err))
    return fail(FA_EUNSUPPORTED, "no kernel for dtype=%s d=%lld", dtype_name(dtype),
                (long long)d);
  if (len > 0) {
    strncpy(kernel_name, info.name, len - 1);
    kernel_name[len - 1] = '\0';
  }
  if (grid) *grid = (S + info.block_rows - 1) / info.block_rows * bh;
  return FA_OK;
}

const char *fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_EINVAL: return "FA_EINVAL: invalid argument";
    case FA_EUNSUPPORTED: return "FA_EUNSUPPORTED: no kernel for this configuration";
    case FA_EHIP: return "FA_EHIP: HIP runtime error";
  }
  return "unknown fa_status";
}

const char *fa_last_error(void) { return g_err; }

int fa_abi_version(void) { return FA_ABI_VERSION; }

}  // extern "C"
