// Attention decoding over a paged key/value cache on gfx950.
//
// Each request's cached keys and values live in fixed-size physical blocks
// scattered over a pool; a per-request block table maps logical token
// positions to blocks, and the kernel walks that table to gather what it
// reads (aicomputerinstitute.com grade-12 chapter on flash attention, section
// "PagedAttention: memory management borrowed from an operating system").
// The attention itself is exact, with the same running-maximum softmax as the
// forward kernel, evaluated as the cache streams past.
//
// Decoding is bound by reading the cache: a new token's few query rows meet
// every cached key and value row once, about one multiply-add per byte, so
// the work goes on the vector ALUs (packed 2-element dot products) and the
// design serves the memory system:
//   * one work-group per (request, key/value head, split of the context), so
//     that a few long requests still fill the chip; each group of query heads
//     sharing a key/value head is served by one work-group, which reads the
//     shared rows once;
//   * d/8 lanes share a token, 16 bytes each, so every load instruction of a
//     wave covers whole contiguous cache rows of one block;
//   * the split's slice of the block table is staged in LDS once, and entries
//     outside the pool are treated as holding no tokens (never dereferenced);
//   * each lane group keeps its own running maximum, sum and output for its
//     tokens (rescaled only when a score exceeds the maximum by more than 2^8),
//     and the groups, waves and finally the splits are merged with the
//     logsumexp algebra: O = sum_s exp(LSE_s - LSE) O_s, LSE = log sum_s
//     exp(LSE_s).
#include "fa_gfx950.h"

#include <math.h>
#include <stdio.h>

namespace fa {
namespace {

using namespace tile;

constexpr int kThreads = 256;
constexpr int kMaxSplitLen = 4096;               // tokens per work-group at most
constexpr int kMaxTable = kMaxSplitLen + 2;      // table entries one split can touch
constexpr float kTau = 8.f;                      // lazy-rescale threshold (base 2)

template <class Ty> struct Dot;
template <> struct Dot<TBF16> {
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
};
template <> struct Dot<TF16> {
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b),
                                  c, false);
  }
};

// Sum over the LPT lanes of a token group (a DPP row of 16 lanes or half of
// one); every lane of the group ends with the same bits (each step adds the
// same two partial sums, in either order).
template <int LPT>
__device__ inline float group_sum(float x) {
  auto add = [](float v, auto ctrl) __attribute__((always_inline)) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                             0xf, 0xf, false));
  };
  x = add(x, std::integral_constant<int, 0xb1>{});   // quad_perm [1,0,3,2]
  x = add(x, std::integral_constant<int, 0x4e>{});   // quad_perm [2,3,0,1]
  x = add(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if (LPT == 16) x = add(x, std::integral_constant<int, 0x140>{});  // row_mirror
  return x;
}

template <class Ty, int D, int R>
__global__ __launch_bounds__(kThreads) void fa_decode_split_kernel(DecodeArgs a) {
  constexpr int LPT = D / 8;         // lanes per token
  constexpr int TPW = 64 / LPT;      // tokens per wave per step
  constexpr int TPS = 4 * TPW;       // tokens per work-group per step
  static_assert(LPT == 8 || LPT == 16, "d must be 64 or 128");
  __shared__ int tab[kMaxTable];
  __shared__ float red_m[4][R], red_l[4][R];
  __shared__ float red_o[4][R][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane % LPT, gi = lane / LPT;

  // Work-group -> (row slice, request and key/value head, split).  Row slices
  // of one split sit 8 work-groups apart, so they share an XCD and its L2.
  const int pairs = a.B * a.Hkv;
  int rs = 0, base = blockIdx.x;
  if (a.row_slices > 1) {
    const int per = 8 * a.row_slices;
    const int grp = base / per, rem = base - grp * per;
    rs = rem >> 3;
    base = grp * 8 + (rem & 7);
  }
  if (base >= pairs * a.n_splits) return;
  const int pair = base % pairs, split = base / pairs;
  const int b = pair / a.Hkv, g = pair - b * a.Hkv;
  const int n = min(max(a.ctx_lens[b], 0), a.ctx_cap);
  const int ns_b = max(1, (n + a.split_len - 1) / a.split_len);
  if (split >= ns_b) return;
  const int t0 = split * a.split_len, t1 = min(n, t0 + a.split_len);
  const int group = a.H / a.Hkv, rows_total = group * a.n_q;
  const int sh = a.bs_shift, bs_mask = (1 << sh) - 1;

  // The split's slice of the block table, validated.
  const int first = t0 >> sh;
  const int cnt = t1 > t0 ? ((t1 - 1) >> sh) - first + 1 : 0;
  for (int e = tid; e < cnt; e += kThreads) {
    const int v = a.block_table[(size_t)b * a.max_blocks + first + e];
    tab[e] = (v >= 0 && v < a.num_blocks) ? v : -1;
  }

  // This work-group's query rows: row rho = rs * R + r is query i of head
  // g * group + j with rho = j * n_q + i; it sits at position n - n_q + i.
  u32x4 qr[R];
  int pos[R];
  int out_row[R];  // index into the B*H*n_q rows of o and lse (-1: padding)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rho = rs * R + r;
    out_row[r] = -1;
    qr[r] = u32x4{0, 0, 0, 0};
    pos[r] = -1;
    if (rho < rows_total) {
      const int j = rho / a.n_q, i = rho - j * a.n_q;
      const int h = g * group + j;
      out_row[r] = (b * a.H + h) * a.n_q + i;
      pos[r] = n - a.n_q + i;
      qr[r] = *(const u32x4 *)((const uint16_t *)a.q + (size_t)out_row[r] * D + 8 * c);
    }
  }
  __syncthreads();

  float m[R], l[R], o[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
  }

  const size_t blk_stride = (size_t)a.Hkv << sh;  // rows per physical block (all heads)
  const uint16_t *kc = (const uint16_t *)a.k_cache + ((size_t)g << sh) * D + 8 * c;
  const uint16_t *vc = (const uint16_t *)a.v_cache + ((size_t)g << sh) * D + 8 * c;
  auto fetch = [&](int t, u32x4 &kk, u32x4 &vv) __attribute__((always_inline)) {
    int blk = -1;
    if (t < t1) blk = tab[(t >> sh) - first];
    if (blk >= 0) {
      const size_t row = (size_t)blk * blk_stride + (size_t)(t & bs_mask);
      kk = __builtin_nontemporal_load((const u32x4 *)(kc + row * D));
      vv = __builtin_nontemporal_load((const u32x4 *)(vc + row * D));
    } else {
      kk = u32x4{0, 0, 0, 0};
      vv = u32x4{0, 0, 0, 0};
    }
    return blk >= 0;
  };

  const float cl2 = a.scale_log2;
  const int steps = (t1 - t0 + TPS - 1) / TPS;
  const int tw = t0 + wave * TPW + gi;  // this lane's token in step 0
  u32x4 kk, vv;
  bool ok = fetch(tw, kk, vv);
  for (int st = 0; st < steps; ++st) {
    const int t = tw + st * TPS;
    u32x4 kn, vn;
    const bool okn = fetch(t + TPS, kn, vn);
    float vf[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2 x = Ty::unpack2(vv[j]);
      vf[2 * j] = x[0];
      vf[2 * j + 1] = x[1];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) s = Dot<Ty>::dot2(qr[r][j], kk[j], s);
      s = group_sum<LPT>(s) * cl2;
      const bool vis = ok && t <= pos[r];
      if (vis && s > m[r] + kTau) {  // rare: move the offset, rescale the state
        const float al = __builtin_amdgcn_exp2f(m[r] - s);
        l[r] *= al;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] *= al;
        m[r] = s;
      }
      const float p = vis ? __builtin_amdgcn_exp2f(s - m[r]) : 0.f;
      l[r] += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
    }
    kk = kn;
    vv = vn;
    ok = okn;
  }

  // Merge the wave's token groups (lanes c, c + LPT, ...), then the waves.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float mm = m[r];
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
    const float al = m[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[r] - mm);
    float ls = l[r] * al;
    float os[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) os[e] = o[r][e] * al;
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
      ls += __shfl_xor(ls, off, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) os[e] += __shfl_xor(os[e], off, 64);
    }
    if (gi == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wave][r][8 * c + e] = os[e];
      if (c == 0) {
        red_m[wave][r] = mm;
        red_l[wave][r] = ls;
      }
    }
  }
  __syncthreads();

  const bool direct = ns_b == 1;
  for (int idx = tid; idx < R * D; idx += kThreads) {
    const int r = idx / D, e = idx - r * D;
    int orow = -1;
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
      if (rr == r) orow = out_row[rr];
    if (orow < 0) continue;
    float mm = red_m[0][r];
#pragma unroll
    for (int w = 1; w < 4; ++w) mm = fmaxf(mm, red_m[w][r]);
    float ls = 0.f, os = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float al = red_m[w][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red_m[w][r] - mm);
      ls = fmaf(al, red_l[w][r], ls);
      os = fmaf(al, red_o[w][r][e], os);
    }
    const bool empty = !(ls > 0.f);
    const float ov = empty ? 0.f : os / ls;
    const float lv = empty ? -INFINITY : (mm + __builtin_amdgcn_logf(ls)) * 0.69314718055994531f;
    if (direct) {
      const uint32_t w2 = Ty::pack2(ov, 0.f);
      ((uint16_t *)a.o)[(size_t)orow * D + e] = (uint16_t)(w2 & 0xffffu);
      if (e == 0) a.lse[orow] = lv;
    } else {
      const size_t slot = (size_t)orow * a.n_splits + split;
      a.ws_o[slot * D + e] = ov;
      if (e == 0) a.ws_lse[slot] = lv;
    }
  }
}

// Combine the splits of every output row whose request needed more than one.
template <class Ty, int D>
__global__ __launch_bounds__(kThreads) void fa_decode_merge_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= a.B * a.H * a.n_q) return;
  const int b = row / (a.H * a.n_q);
  const int n = min(max(a.ctx_lens[b], 0), a.ctx_cap);
  const int ns_b = max(1, (n + a.split_len - 1) / a.split_len);
  if (ns_b == 1) return;  // written directly by the split kernel
  const float *ls = a.ws_lse + (size_t)row * a.n_splits;
  const float *os = a.ws_o + (size_t)row * a.n_splits * D;
  float mx = -INFINITY;
  for (int s = 0; s < ns_b; ++s) mx = fmaxf(mx, ls[s]);
  uint16_t *orow = (uint16_t *)a.o + (size_t)row * D;
  if (mx == -INFINITY) {
    for (int e = lane; e < D; e += 64) orow[e] = 0;
    if (lane == 0) a.lse[row] = -INFINITY;
    return;
  }
  constexpr float kLog2e = 1.4426950408889634f;
  float sum = 0.f;
  for (int s = 0; s < ns_b; ++s) sum += __builtin_amdgcn_exp2f((ls[s] - mx) * kLog2e);
  const float lse = mx + __builtin_amdgcn_logf(sum) * 0.69314718055994531f;
  for (int e = lane; e < D; e += 64) {
    float acc = 0.f;
    for (int s = 0; s < ns_b; ++s)
      acc = fmaf(__builtin_amdgcn_exp2f((ls[s] - lse) * kLog2e), os[(size_t)s * D + e], acc);
    orow[e] = (uint16_t)(Ty::pack2(acc, 0.f) & 0xffffu);
  }
  if (lane == 0) a.lse[row] = lse;
}

template <class Ty, int D, int R>
bool run_decode(const DecodeArgs *a, const DecodePlan *p, hipStream_t stream, bool launch,
                LaunchInfo *info, hipError_t *err) {
  static char name[96];
  snprintf(name, sizeof(name), "fa_decode_paged<%s,d%d,rows%d>", Ty::kName, D, R);
  info->name = name;
  info->block_rows = R;
  info->threads = kThreads;
  if (!launch) return true;
  DecodeArgs args = *a;
  void *kargs[] = {&args};
  *err = hipLaunchKernel((const void *)&fa_decode_split_kernel<Ty, D, R>,
                         dim3((unsigned)p->grid), dim3(kThreads), kargs, 0, stream);
  if (*err != hipSuccess || p->n_splits == 1) return true;
  const int64_t rows = (int64_t)a->B * a->H * a->n_q;
  *err = hipLaunchKernel((const void *)&fa_decode_merge_kernel<Ty, D>,
                         dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), kargs, 0, stream);
  return true;
}

template <class Ty, int D>
bool decode_by_rows(const DecodeArgs *a, const DecodePlan *p, hipStream_t s, bool launch,
                    LaunchInfo *info, hipError_t *err) {
  switch (p->rows) {
    case 1: return run_decode<Ty, D, 1>(a, p, s, launch, info, err);
    case 2: return run_decode<Ty, D, 2>(a, p, s, launch, info, err);
    case 4: return run_decode<Ty, D, 4>(a, p, s, launch, info, err);
    case 8: return run_decode<Ty, D, 8>(a, p, s, launch, info, err);
  }
  return false;
}

template <class Ty>
bool decode_by_dim(int d, const DecodeArgs *a, const DecodePlan *p, hipStream_t s, bool launch,
                   LaunchInfo *info, hipError_t *err) {
  switch (d) {
    case 64: return decode_by_rows<Ty, 64>(a, p, s, launch, info, err);
    case 128: return decode_by_rows<Ty, 128>(a, p, s, launch, info, err);
  }
  return false;
}

}  // namespace

bool decode_plan(int d, int64_t B, int64_t H, int64_t Hkv, int64_t n_q, int64_t ctx_cap,
                 DecodePlan *p) {
  if (d != 64 && d != 128) return false;
  const int64_t rows_total = (H / Hkv) * n_q;
  p->rows = rows_total <= 1 ? 1 : rows_total <= 2 ? 2 : rows_total <= 4 ? 4 : 8;
  p->row_slices = (int)((rows_total + p->rows - 1) / p->rows);
  // Enough work-groups to fill the chip several times over: split each
  // context when requests x key/value heads x row slices alone are too few.
  const int64_t units = B * Hkv * p->row_slices;
  const int64_t want = units >= 2048 ? 1 : (2048 + units - 1) / units;
  int64_t len = (ctx_cap + want - 1) / want;
  len = (len + 63) / 64 * 64;
  if (want > 1 && len < 256) len = 256;
  if (len < 64) len = 64;
  if (len > kMaxSplitLen) len = kMaxSplitLen;
  p->split_len = (int)len;
  p->n_splits = (int)(ctx_cap > 0 ? (ctx_cap + len - 1) / len : 1);
  const int64_t base = B * Hkv * p->n_splits;
  p->grid = p->row_slices > 1 ? (base + 7) / 8 * 8 * p->row_slices : base;
  p->ws_bytes = p->n_splits > 1 ? B * H * n_q * p->n_splits * (int64_t)(d + 1) * 4 : 0;
  return true;
}

bool decode_paged(DType dt, int d, const DecodeArgs *a, const DecodePlan *p, hipStream_t stream,
                  bool launch, LaunchInfo *info, hipError_t *err) {
  if (dt == kBF16) return decode_by_dim<TBF16>(d, a, p, stream, launch, info, err);
  if (dt == kF16) return decode_by_dim<TF16>(d, a, p, stream, launch, info, err);
  return false;
}

}  // namespace fa
