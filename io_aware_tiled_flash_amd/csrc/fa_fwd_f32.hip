// Exact attention forward for fp32 inputs (no down-conversion anywhere).
//
// Same online-softmax tiling as the bf16/fp16 kernel ("FlashAttention: Why
// Tiling Attention Makes Transformers Fast Without Changing the Result",
// section "The tiled forward pass"), written for fp32 on the vector ALUs.
// Four lanes of a quad serve one query row, each with a quarter of d (its
// Q values and fp32 output accumulator in registers), so a wave covers 16
// rows and a work-group 16 rows: small problems still spread over many
// compute units.  The work-group's waves (16 at d = 64, 8 at d = 128) take
// every NW-th 16-key tile of the visible range, each staging its K and V
// tiles in its own LDS buffers (the next tile loaded into registers while
// the current one is used) and reading them back as quad-wide broadcasts; a
// score's quarter sums are added across the quad.  The waves' partial states
// (m, l, O) of a row are then merged with the same rescaling algebra the
// online softmax uses between tiles (the split over the key sequence of the
// grade-12 chapter's section "What FlashAttention-2 changed"): m = max m_w,
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

// x plus the value of the lane whose index differs in the bits of CTRL's
// permutation within each group of four (a quad_perm DPP move).
template <int CTRL>
__device__ inline float quad_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Four lanes (a quad) serve one query row, each holding a quarter of d; a
// wave covers 16 rows, and the four waves of a work-group take every fourth
// 16-key tile of those rows' visible range.  So a small problem still spreads
// over many compute units (one work-group per 16 rows), and each lane's work
// per key is d/4 multiply-adds for the score and d/4 for the output.
constexpr int kF32LanesPerRow = 4, kF32Rows = 64 / kF32LanesPerRow, kF32Keys = 16;
template <int D> constexpr int f32_waves() { return D == 64 ? 16 : 8; }

template <int D, int MASK>
__global__ __launch_bounds__(f32_waves<D>() * 64) void fa_fwd_f32_kernel(FwdArgs a) {
  constexpr int NW = f32_waves<D>(), LPR = kF32LanesPerRow, BR = kF32Rows, BC = kF32Keys;
  constexpr int D4 = D / 4;        // float4 per row
  constexpr int DL = D / LPR;      // d values per lane
  constexpr int DL4 = DL / 4;
  constexpr int TILE4 = BC * D4;   // float4 per K or V tile
  static_assert(TILE4 % 64 == 0, "tile must split evenly over a wave");
  static_assert(NW * 2 * TILE4 * 4 >= NW * D * BR, "merge area must fit in the stages");
  static_assert((D / NW) % LPR == 0, "merge columns must split evenly over the quad");
  // Per wave: a K and a V stage.  After the key loop the same memory holds
  // the waves' partial accumulators for the merge, [wave][column][row].
  __shared__ float4 stage[NW][2][TILE4];
  __shared__ float part_ml[NW][2][BR];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rl = lane / LPR, part = lane % LPR;  // row within the tile, quarter of d
  const int S = a.S;
  const int BH = a.B * a.H;
  const int nq = (S + BR - 1) / BR;
  const HeadPair hp = head_of_slot(blockIdx.x % BH, a.B, a.H, a.Hkv);
  const int bh = hp.q;
  int qt = blockIdx.x / BH;
  if (MASK != kMaskNone) qt = nq - 1 - qt;
  const int q0 = qt * BR;
  const int row = q0 + rl;
  const size_t head_off = (size_t)bh * (size_t)S * D;   // q, o
  const size_t kv_off = (size_t)hp.kv * (size_t)S * D;  // k, v
  const float4 *qh = (const float4 *)((const float *)a.q + head_off);
  const float4 *kh = (const float4 *)((const float *)a.k + kv_off);
  const float4 *vh = (const float4 *)((const float *)a.v + kv_off);

  // This lane's quarter of the row: d values part*DL .. part*DL + DL - 1.
  float q[DL], o[DL];
#pragma unroll
  for (int c = 0; c < DL4; ++c) {
    const float4 x =
        row < S ? qh[(size_t)row * D4 + part * DL4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    q[4 * c] = x.x; q[4 * c + 1] = x.y; q[4 * c + 2] = x.z; q[4 * c + 3] = x.w;
  }
#pragma unroll
  for (int c = 0; c < DL; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int ntk = (S + BC - 1) / BC;
  int kt_begin = 0, kt_end = ntk;
  if (MASK != kMaskNone) {
    kt_end = (min(q0 + BR, S) - 1) / BC + 1;
    if (MASK == kMaskWindow) kt_begin = max(0, q0 - a.window + 1) / BC;
  }

  // Each wave's next tile is loaded into registers while it computes on the
  // current one, then staged in its LDS buffers (coalesced float4 loads:
  // consecutive lanes, consecutive 16-byte pieces of the tile's rows).
  float4 *kl = &stage[wave][0][0], *vl = &stage[wave][1][0];
  constexpr int PER_LANE = TILE4 / 64;
  float4 nk[PER_LANE], nv[PER_LANE];
  auto fetch = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BC;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int idx = lane + 64 * i;
      const int r = idx / D4;
      const bool in = k0 + r < S;
      nk[i] = in ? kh[(size_t)(k0 + r) * D4 + idx % D4] : make_float4(0.f, 0.f, 0.f, 0.f);
      nv[i] = in ? vh[(size_t)(k0 + r) * D4 + idx % D4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if (kt_begin + wave < kt_end) fetch(kt_begin + wave);
  for (int kt = kt_begin + wave; kt < kt_end; kt += NW) {
    const int k0 = kt * BC;
    wave_lds_sync();  // this wave's previous tile fully read
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      kl[lane + 64 * i] = nk[i];
      vl[lane + 64 * i] = nv[i];
    }
    wave_lds_sync();
    if (kt + NW < kt_end) fetch(kt + NW);

    // Partial scores over this lane's quarter of d, accumulated
    // key-interleaved (independent chains), then summed over the quad: the
    // two exchanges add the same partial sums in the same pairs on every
    // lane of the quad, so all four hold the same bits.
    float s[BC];
#pragma unroll
    for (int j = 0; j < BC; ++j) s[j] = 0.f;
#pragma unroll
    for (int c = 0; c < DL4; ++c)
#pragma unroll
      for (int j = 0; j < BC; ++j) {
        const float4 kv = kl[j * D4 + part * DL4 + c];
        s[j] = fmaf(q[4 * c], kv.x, s[j]);
        s[j] = fmaf(q[4 * c + 1], kv.y, s[j]);
        s[j] = fmaf(q[4 * c + 2], kv.z, s[j]);
        s[j] = fmaf(q[4 * c + 3], kv.w, s[j]);
      }
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float sum = quad_add<0x4e>(quad_add<0xb1>(s[j]));  // [1,0,3,2] then [2,3,0,1]
      const float x = sum * a.scale_log2;
      s[j] = key_visible<MASK>(k0 + j, row, S, a.window) ? x : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < DL; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = __builtin_amdgcn_exp2f(s[j] - m_use);
      l += p;
#pragma unroll
      for (int c = 0; c < DL4; ++c) {
        const float4 vv = vl[j * D4 + part * DL4 + c];
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
  for (int c = 0; c < DL; ++c) po[(wave * D + part * DL + c) * BR + rl] = o[c];
  if (part == 0) {
    part_ml[wave][0][rl] = m;
    part_ml[wave][1][rl] = l;
  }
  __syncthreads();
  float mw[NW], m_tot = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mw[w] = part_ml[w][0][rl];
    m_tot = fmaxf(m_tot, mw[w]);
  }
  float f[NW], l_tot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    f[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - m_tot);
    l_tot = fmaf(f[w], part_ml[w][1][rl], l_tot);
  }
  if (row < S) {
    const float inv = 1.f / l_tot;
    float *orow = (float *)a.o + head_off + (size_t)row * D;
    // wave w stores columns w*D/NW ..; the quad splits them in runs of CPL
    constexpr int CPL = D / NW / LPR;
    const int cb = wave * (D / NW) + part * CPL;
    float r[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) acc = fmaf(f[w], po[(w * D + cb + e) * BR + rl], acc);
      r[e] = acc * inv;
    }
    if constexpr (CPL % 4 == 0) {
#pragma unroll
      for (int c4 = 0; c4 < CPL / 4; ++c4)
        *(float4 *)(orow + cb + 4 * c4) =
            make_float4(r[4 * c4], r[4 * c4 + 1], r[4 * c4 + 2], r[4 * c4 + 3]);
    } else {
#pragma unroll
      for (int e = 0; e < CPL; ++e) orow[cb + e] = r[e];
    }
    if (wave == 0 && part == 0)
      a.lse[(size_t)bh * S + row] = (m_tot + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, int MASK>
bool run(const FwdArgs *a, hipStream_t stream, bool launch, LaunchInfo *info, hipError_t *err) {
  static char name[80];
  static const char *mk[3] = {"none", "causal", "window"};
  constexpr int NW = f32_waves<D>();
  snprintf(name, sizeof(name), "fa_fwd_f32<d%d,%s,br%d,bc%d,w%d,lanes_per_row%d>", D, mk[MASK],
           kF32Rows, kF32Keys, NW, kF32LanesPerRow);
  info->name = name;
  info->block_rows = kF32Rows;
  info->threads = NW * 64;
  if (!launch) return true;
  const int nq = (a->S + kF32Rows - 1) / kF32Rows;
  FwdArgs args = *a;
  void *kargs[] = {&args};
  *err = hipLaunchKernel((const void *)&fa_fwd_f32_kernel<D, MASK>,
                         dim3((unsigned)(nq * a->B * a->H)), dim3(NW * 64), kargs, 0,
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
