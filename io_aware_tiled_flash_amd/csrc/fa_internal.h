// Internal interface between the C-ABI host layer (fa_api.hip) and the kernel
// translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum MaskKind : int { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2 };
enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Arguments of one forward launch, already validated on the host.
struct FwdArgs {
  const void *q;           // [B, H, S, d] contiguous
  const void *k, *v;       // [B, Hkv, S, d] contiguous; Hkv divides H
  void *o;                 // [B, H, S, d] contiguous
  float *lse;              // [B, H, S]
  int B, H, Hkv, S;
  int window;              // used by the sliding-window instances only
  float scale_log2;        // scale * log2(e): scores are kept in base-2 units
};

// Arguments of one backward launch, already validated on the host.
struct BwdArgs {
  const void *q;           // [B, H, S, d]
  const void *k, *v;       // [B, Hkv, S, d]
  const void *o, *dout;    // [B, H, S, d] forward output and its gradient
  const float *lse;        // [B, H, S] natural-log logsumexp from the forward pass
  void *dq;                // [B, H, S, d]
  void *dk, *dv;           // [B, Hkv, S, d]
  float *delta;            // [B, H, S] workspace: rowsum(dO * O)
  int B, H, Hkv, S;
  int window;              // used by the sliding-window instances only
  float scale;             // the forward's scale (natural units)
  float scale_log2;        // scale * log2(e)
};

// Arguments of one paged-cache decode launch, already validated on the host.
struct DecodeArgs {
  const void *q;                    // [B, H, n_q, d]
  const void *k_cache, *v_cache;    // [num_blocks, Hkv, block_size, d]
  const int32_t *block_table;       // [B, max_blocks]
  const int32_t *ctx_lens;          // [B]
  void *o;                          // [B, H, n_q, d]
  float *lse;                       // [B, H, n_q]
  float *ws_o;                      // [B*H*n_q, n_splits, d] partial outputs (n_splits > 1)
  float *ws_lse;                    // [B*H*n_q, n_splits]    partial logsumexps
  int B, H, Hkv, n_q;
  int num_blocks, bs_shift, max_blocks;
  int ctx_cap;                      // min(max_ctx, max_blocks * block_size)
  int split_len, n_splits;          // tokens per work-group, work-groups per request
  int rows, row_slices;             // query rows per work-group, work-groups per split
  float scale_log2;
};

// How a decode launch is cut up; a pure function of the sizes, shared by the
// workspace query and the launch.
struct DecodePlan {
  int rows, row_slices, split_len, n_splits;
  int64_t grid;                     // work-groups of the split kernel
  int64_t ws_bytes;                 // workspace the launch needs (0: none)
};

// Query head (index into the B*H heads of q, o, lse) and key/value head
// (index into the B*Hkv heads of k, v) served by work-group slot s in
// [0, B*H).  Query head h of batch b reads key/value head h / (H / Hkv).
// Slots run over every key/value head first and then over the members of
// each group, so when B*Hkv is a multiple of 8 the query heads of one group
// land on the same XCD (work-groups are dealt round-robin over the 8 XCDs)
// and share its L2 for their K/V tiles.  With Hkv == H the mapping is the
// identity.
struct HeadPair {
  int q, kv;
};
__device__ inline HeadPair head_of_slot(int s, int B, int H, int Hkv) {
  const int group = H / Hkv, n_kv = B * Hkv;
  const int j = s / n_kv, kvi = s - j * n_kv;
  const int b = kvi / Hkv, hk = kvi - b * Hkv;
  return HeadPair{b * H + hk * group + j, kvi};
}

// What a launch would look like, for logging and fa_query.
struct LaunchInfo {
  const char *name;        // human-readable instance name
  int block_rows;          // query rows per work-group
  int threads;             // threads per work-group
};

// Each returns false when no instance exists for (d, mask); otherwise fills
// `info` and, when `launch` is true, launches on `stream` and stores the HIP
// status in `*err`.
bool mfma_forward(DType dt, int d, int mask, const FwdArgs *a, hipStream_t stream,
                  bool launch, LaunchInfo *info, hipError_t *err);
bool f32_forward(int d, int mask, const FwdArgs *a, hipStream_t stream, bool launch,
                 LaunchInfo *info, hipError_t *err);
// Backward pass: three launches on `stream` (row terms, dK/dV, dQ).  Returns
// false when no instance exists for (dtype, d, mask); `info` names the dK/dV
// kernel.
bool mfma_backward(DType dt, int d, int mask, const BwdArgs *a, hipStream_t stream,
                   bool launch, LaunchInfo *info, hipError_t *err);
// Paged-cache decode: the plan of a launch (false when d has no kernel), and
// the launch itself (split kernel, then the merge kernel when n_splits > 1).
bool decode_plan(int d, int64_t B, int64_t H, int64_t Hkv, int64_t n_q, int64_t ctx_cap,
                 DecodePlan *plan);
// Split kernel (and, when n_splits > 1, the merge kernel) on `stream`.
// Returns false when no instance exists for (dtype, d).
bool decode_paged(DType dt, int d, const DecodeArgs *a, const DecodePlan *plan,
                  hipStream_t stream, bool launch, LaunchInfo *info, hipError_t *err);

}  // namespace fa
