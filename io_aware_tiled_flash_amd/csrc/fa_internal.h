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
  const void *q, *k, *v;   // [B, H, S, d] contiguous
  void *o;                 // [B, H, S, d] contiguous
  float *lse;              // [B, H, S]
  int B, H, S;
  int window;              // used by the sliding-window instances only
  float scale_log2;        // scale * log2(e): scores are kept in base-2 units
};

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

}  // namespace fa
