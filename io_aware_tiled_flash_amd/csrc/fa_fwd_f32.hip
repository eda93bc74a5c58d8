// Exact attention forward for fp32 inputs (no down-conversion anywhere).
//
// Same online-softmax tiling as the bf16/fp16 kernel ("FlashAttention: Why
// Tiling Attention Makes Transformers Fast Without Changing the Result",
// section "The tiled forward pass"), written for fp32 on the vector ALUs.
// A work-group owns 64 query rows; each of its four waves holds all 64 rows
// (one lane per row: its Q row and fp32 output accumulator in registers) and
// runs the online softmax over every fourth key tile of the visible range,
// staging its 32-key K and V tiles in its own LDS buffers and reading them
// back as wave-wide broadcasts.  The four partial states (m, l, O) of a row
// are then merged with the same rescaling algebra the online softmax uses
// between tiles (the split over the key sequence of the grade-12 chapter's
// section "What FlashAttention-2 changed"): m = max m_w,
// l = sum l_w exp(m_w - m), O = sum O_w exp(m_w - m), then O / l once.
// fp32 exists for exactness checks rather than speed: the matrix-core path
// is bf16/fp16.
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

// Make this wave's LDS writes visible to its own later reads (and keep the
// compiler from moving LDS accesses across).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

constexpr int kF32Waves = 4, kF32Rows = 64, kF32Keys = 32;

template <int D, int MASK>
__global__ __launch_bounds__(kF32Waves * 64, 1) void fa_fwd_f32_kernel(FwdArgs a) {
  constexpr int NW = kF32Waves, BR = kF32Rows, BC = kF32Keys, D4 = D / 4;
  constexpr int TILE4 = BC * D4;  // float4 per K or V tile
  static_assert(TILE4 % 64 == 0, "tile must split evenly over a wave");
  static_assert(NW * 2 * TILE4 * 4 >= NW * D * BR, "merge area must fit in the stages");
  // Per wave: a K and a V stage.  After the key loop the same memory holds
  // the waves' partial accumulators for the merge, [wave][column][row].
  __shared__ float4 stage[NW][2][TILE4];
  __shared__ float part_ml[NW][2][BR];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S;
  const int BH = a.B * a.H;
  const int nq = (S + BR - 1) / BR;
  const HeadPair hp = head_of_slot(blockIdx.x % BH, a.B, a.H, a.Hkv);
  const int bh = hp.q;
  int qt = blockIdx.x / BH;
  if (MASK != kMaskNone) qt = nq - 1 - qt;
  const int q0 = qt * BR;
  const int row = q0 + lane;
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

  float4 *kl = &stage[wave][0][0], *vl = &stage[wave][1][0];
  for (int kt = kt_begin + wave; kt < kt_end; kt += NW) {
    const int k0 = kt * BC;
    wave_lds_sync();  // this wave's previous tile fully read
#pragma unroll
    for (int i = 0; i < TILE4 / 64; ++i) {
      const int idx = lane + 64 * i;
      const int r = idx / D4;
      const bool in = k0 + r < S;
      kl[idx] = in ? kh[(size_t)(k0 + r) * D4 + idx % D4] : make_float4(0.f, 0.f, 0.f, 0.f);
      vl[idx] = in ? vh[(size_t)(k0 + r) * D4 + idx % D4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    wave_lds_sync();

    // Scores of the 32 keys, accumulated key-interleaved (independent chains).
    float s[BC];
#pragma unroll
    for (int j = 0; j < BC; ++j) s[j] = 0.f;
#pragma unroll
    for (int c = 0; c < D4; ++c)
#pragma unroll
      for (int j = 0; j < BC; ++j) {
        const float4 kv = kl[j * D4 + c];
        s[j] = fmaf(q[4 * c], kv.x, s[j]);
        s[j] = fmaf(q[4 * c + 1], kv.y, s[j]);
        s[j] = fmaf(q[4 * c + 2], kv.z, s[j]);
        s[j] = fmaf(q[4 * c + 3], kv.w, s[j]);
      }
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float x = s[j] * a.scale_log2;
      s[j] = key_visible<MASK>(k0 + j, row, S, a.window) ? x : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
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
        const float4 vv = vl[j * D4 + c];
        o[4 * c] = fmaf(p, vv.x, o[4 * c]);
        o[4 * c + 1] = fmaf(p, vv.y, o[4 * c + 1]);
        o[4 * c + 2] = fmaf(p, vv.z, o[4 * c + 2]);
        o[4 * c + 3] = fmaf(p, vv.w, o[4 * c + 3]);
      }
    }
  }

  // Merge the waves' partial states.  A wave that saw no visible key of a
  // row has m = -inf, l = 0, O = 0 and gets factor 0.
  __syncthreads();  // every wave is done with its stages
  float *po = (float *)&stage[0][0][0];
#pragma unroll
  for (int c = 0; c < D; ++c) po[(wave * D + c) * BR + lane] = o[c];
  part_ml[wave][0][lane] = m;
  part_ml[wave][1][lane] = l;
  __syncthreads();
  float mw[NW], m_tot = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mw[w] = part_ml[w][0][lane];
    m_tot = fmaxf(m_tot, mw[w]);
  }
  float f[NW], l_tot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    f[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - m_tot);
    l_tot = fmaf(f[w], part_ml[w][1][lane], l_tot);
  }
  if (row < S) {
    const float inv = 1.f / l_tot;
    float *orow = (float *)a.o + head_off + (size_t)row * D;
    constexpr int CPW = D / NW;  // output columns this wave merges
#pragma unroll
    for (int c4 = 0; c4 < CPW / 4; ++c4) {
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = wave * CPW + 4 * c4 + e;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc = fmaf(f[w], po[(w * D + c) * BR + lane], acc);
        r[e] = acc * inv;
      }
      *(float4 *)(orow + wave * CPW + 4 * c4) = make_float4(r[0], r[1], r[2], r[3]);
    }
    if (wave == 0)
      a.lse[(size_t)bh * S + row] = (m_tot + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, int MASK>
bool run(const FwdArgs *a, hipStream_t stream, bool launch, LaunchInfo *info, hipError_t *err) {
  static char name[80];
  static const char *mk[3] = {"none", "causal", "window"};
  snprintf(name, sizeof(name), "fa_fwd_f32<d%d,%s,br64,bc32,w4>", D, mk[MASK]);
  info->name = name;
  info->block_rows = kF32Rows;
  info->threads = kF32Waves * 64;
  if (!launch) return true;
  const int nq = (a->S + kF32Rows - 1) / kF32Rows;
  FwdArgs args = *a;
  void *kargs[] = {&args};
  *err = hipLaunchKernel((const void *)&fa_fwd_f32_kernel<D, MASK>,
                         dim3((unsigned)(nq * a->B * a->H)), dim3(kF32Waves * 64), kargs, 0,
                         stream);
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
