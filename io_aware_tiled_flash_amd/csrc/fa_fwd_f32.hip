// Exact attention forward for fp32 inputs (no down-conversion anywhere).
//
// Same online-softmax tiling as the bf16/fp16 kernel ("FlashAttention: Why
// Tiling Attention Makes Transformers Fast Without Changing the Result",
// section "The tiled forward pass"), written for fp32 on the vector ALUs:
// one lane owns one query row (its Q row and fp32 output accumulator sit in
// VGPRs), K and V tiles of 32 keys are staged in LDS and read back as
// wave-wide broadcasts.  fp32 exists for exactness checks rather than speed:
// the matrix-core path is bf16/fp16.
#include "fa_internal.h"

#include <math.h>
#include <stdio.h>

namespace fa {
namespace {

template <int MASK>
__device__ inline bool key_visible(int key, int row, int S, int window) {
  if (MASK == kMaskNone) return key < S;
  if (MASK == kMaskCausal) return key <= row;
  return key <= row && key > row - window;
}

template <int D, int MASK>
__global__ __launch_bounds__(64, 1) void fa_fwd_f32_kernel(FwdArgs a) {
  constexpr int BR = 64, BC = 32, D4 = D / 4;
  __shared__ float4 k_lds[BC * D4];
  __shared__ float4 v_lds[BC * D4];

  const int tid = threadIdx.x;
  const int S = a.S;
  const int BH = a.B * a.H;
  const int nq = (S + BR - 1) / BR;
  const HeadPair hp = head_of_slot(blockIdx.x % BH, a.B, a.H, a.Hkv);
  const int bh = hp.q;
  int qt = blockIdx.x / BH;
  if (MASK != kMaskNone) qt = nq - 1 - qt;
  const int q0 = qt * BR;
  const int row = q0 + tid;
  const size_t head_off = (size_t)bh * (size_t)S * D;   // q, o
  const size_t kv_off = (size_t)hp.kv * (size_t)S * D;  // k, v
  const float4 *qh = (const float4 *)((const float *)a.q + head_off);
  const float4 *kh = (const float4 *)((const float *)a.k + kv_off);
  const float4 *vh = (const float4 *)((const float *)a.v + kv_off);

  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D4; ++c) {
    const float4 x = row < S ? qh[(size_t)row * D4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    q[4 * c] = x.x; q[4 * c + 1] = x.y; q[4 * c + 2] = x.z; q[4 * c + 3] = x.w;
  }
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int ntk = (S + BC - 1) / BC;
  int kt_begin = 0, kt_end = ntk;
  if (MASK != kMaskNone) {
    kt_end = (min(q0 + BR, S) - 1) / BC + 1;
    if (MASK == kMaskWindow) kt_begin = max(0, q0 - a.window + 1) / BC;
  }

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int k0 = kt * BC;
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < BC * D4 / 64; ++i) {
      const int idx = tid + 64 * i;
      const int r = idx / D4;
      const bool in = k0 + r < S;
      k_lds[idx] = in ? kh[(size_t)(k0 + r) * D4 + idx % D4] : make_float4(0.f, 0.f, 0.f, 0.f);
      v_lds[idx] = in ? vh[(size_t)(k0 + r) * D4 + idx % D4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    float s[BC];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D4; ++c) {
        const float4 kv = k_lds[j * D4 + c];
        acc = fmaf(q[4 * c], kv.x, acc);
        acc = fmaf(q[4 * c + 1], kv.y, acc);
        acc = fmaf(q[4 * c + 2], kv.z, acc);
        acc = fmaf(q[4 * c + 3], kv.w, acc);
      }
      float x = acc * a.scale_log2;
      x = key_visible<MASK>(k0 + j, row, S, a.window) ? x : -INFINITY;
      s[j] = x;
      tmax = fmaxf(tmax, x);
    }
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = __builtin_amdgcn_exp2f(s[j] - m_use);
      l += p;
#pragma unroll
      for (int c = 0; c < D4; ++c) {
        const float4 vv = v_lds[j * D4 + c];
        o[4 * c] = fmaf(p, vv.x, o[4 * c]);
        o[4 * c + 1] = fmaf(p, vv.y, o[4 * c + 1]);
        o[4 * c + 2] = fmaf(p, vv.z, o[4 * c + 2]);
        o[4 * c + 3] = fmaf(p, vv.w, o[4 * c + 3]);
      }
    }
  }

  if (row < S) {
    const float inv = 1.f / l;
    float4 *oh = (float4 *)((float *)a.o + head_off) + (size_t)row * D4;
#pragma unroll
    for (int c = 0; c < D4; ++c)
      oh[c] = make_float4(o[4 * c] * inv, o[4 * c + 1] * inv, o[4 * c + 2] * inv,
                          o[4 * c + 3] * inv);
    a.lse[(size_t)bh * S + row] = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
  }
}

template <int D, int MASK>
bool run(const FwdArgs *a, hipStream_t stream, bool launch, LaunchInfo *info, hipError_t *err) {
  static char name[80];
  static const char *mk[3] = {"none", "causal", "window"};
  snprintf(name, sizeof(name), "fa_fwd_f32<d%d,%s,br64,bc32>", D, mk[MASK]);
  info->name = name;
  info->block_rows = 64;
  info->threads = 64;
  if (!launch) return true;
  const int nq = (a->S + 63) / 64;
  FwdArgs args = *a;
  void *kargs[] = {&args};
  *err = hipLaunchKernel((const void *)&fa_fwd_f32_kernel<D, MASK>,
                         dim3((unsigned)(nq * a->B * a->H)), dim3(64), kargs, 0, stream);
  return true;
}

template <int D>
bool by_mask(int mask, const FwdArgs *a, hipStream_t s, bool launch, LaunchInfo *info,
             hipError_t *err) {
  switch (mask) {
    case kMaskNone: return run<D, kMaskNone>(a, s, launch, info, err);
    case kMaskCausal: return run<D, kMaskCausal>(a, s, launch, info, err);
    case kMaskWindow: return run<D, kMaskWindow>(a, s, launch, info, err);
  }
  return false;
}

}  // namespace

bool f32_forward(int d, int mask, const FwdArgs *a, hipStream_t stream, bool launch,
                 LaunchInfo *info, hipError_t *err) {
  switch (d) {
    case 64: return by_mask<64>(mask, a, stream, launch, info, err);
    case 128: return by_mask<128>(mask, a, stream, launch, info, err);
  }
  return false;
}

}  // namespace fa
