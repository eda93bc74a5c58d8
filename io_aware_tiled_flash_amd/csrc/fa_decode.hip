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
#include "fa_tile_ops.h"

#include <math.h>
#include <stdio.h>

namespace fa {
namespace {

using namespace tile;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxSplitLen = 4096;               // tokens per work-group at most
constexpr int kMaxTable = kMaxSplitLen + 2;      // table entries one split can touch
constexpr float kTau = 8.f;                      // lazy-rescale threshold (base 2)
constexpr int kMfmaRows = 5;                     // query rows per key/value head for MFMA
constexpr int kMfmaGroups = 1024;                // work-groups the MFMA path aims for
constexpr int kValuGroups = 4096;                // work-groups the vector path aims for
constexpr int kMinSplit = 1024;                  // shortest split worth its merge


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

// Sum over the LPT lanes of a token group (half a DPP row of 16 lanes, a
// row, or two rows); every lane of the group ends with the same bits (each
// step adds the same two partial sums, in either order).
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
  if (LPT >= 16) x = add(x, std::integral_constant<int, 0x140>{});  // row_mirror
  if (LPT == 32) x += __shfl_xor(x, 16, 64);                        // the other row
  return x;
}

template <class Ty, int D, int R>
__global__ __launch_bounds__(kThreads) void fa_decode_split_kernel(DecodeArgs a) {
  constexpr int LPT = D / 8;         // lanes per token
  constexpr int TPW = 64 / LPT;      // tokens per wave per step
  constexpr int TPS = 4 * TPW;       // tokens per work-group per step
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "d must be 64, 128 or 256");
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
  // Every lane loads (a token that does not exist reads block 0's first row,
  // always valid memory; loads under a branch would make the compiler wait
  // for all of them at the next use); such tokens get weight 0 and a zero V.
  auto fetch = [&](int t, u32x4 &kk, u32x4 &vv) __attribute__((always_inline)) {
    int blk = -1;
    if (t < t1) blk = tab[(t >> sh) - first];
    const size_t row = blk >= 0 ? (size_t)blk * blk_stride + (size_t)(t & bs_mask) : 0;
    kk = __builtin_nontemporal_load((const u32x4 *)(kc + row * D));
    vv = __builtin_nontemporal_load((const u32x4 *)(vc + row * D));
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
      const f32x2 x = Ty::unpack2(ok ? vv[j] : 0u);
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

// Combine the splits of every output row whose request needed more than one:
// LSE = log sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s.  One wave per
// row; the partials are hot in L2, so the kernel is latency-bound: the
// splits' logsumexps are read by all lanes at once (lane s: split s, then
// s + 64, ...) and reduced across the wave, and the partial rows are read
// eight splits at a time (each lane D/64 columns) before they are combined,
// in split order.
template <class Ty, int D>
__global__ __launch_bounds__(kThreads) void fa_decode_merge_kernel(DecodeArgs a) {
  constexpr int CPL = D / 64;  // output columns per lane
  constexpr int U = 8;         // splits whose partial rows are in flight together
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= a.B * a.H * a.n_q) return;
  const int b = row / (a.H * a.n_q);
  const int n = min(max(a.ctx_lens[b], 0), a.ctx_cap);
  const int ns_b = max(1, (n + a.split_len - 1) / a.split_len);
  if (ns_b == 1) return;  // written directly by the split kernel
  const float *ls = a.ws_lse + (size_t)row * a.n_splits;
  const float *os = a.ws_o + (size_t)row * a.n_splits * D;
  // The first U splits' partial rows are loaded together with the
  // logsumexps (past the last split: the last one again, a valid address,
  // later given weight 0), so the common case costs one round trip.
  float v0[U][CPL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int s = min(u, ns_b - 1);
#pragma unroll
    for (int c = 0; c < CPL; ++c) v0[u][c] = os[(size_t)s * D + lane + 64 * c];
  }
  const float ls_lane = lane < ns_b ? ls[lane] : -INFINITY;  // split `lane`'s logsumexp
  float mx = ls_lane;
  for (int s = lane + 64; s < ns_b; s += 64) mx = fmaxf(mx, ls[s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  uint16_t *orow = (uint16_t *)a.o + (size_t)row * D;
  if (mx == -INFINITY) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) orow[lane + 64 * c] = 0;
    if (lane == 0) a.lse[row] = -INFINITY;
    return;
  }
  constexpr float kLog2e = 1.4426950408889634f;
  float sum = lane < ns_b ? __builtin_amdgcn_exp2f((ls_lane - mx) * kLog2e) : 0.f;
  for (int s = lane + 64; s < ns_b; s += 64) sum += __builtin_amdgcn_exp2f((ls[s] - mx) * kLog2e);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  const float lse = mx + __builtin_amdgcn_logf(sum) * 0.69314718055994531f;
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int s0 = 0; s0 < ns_b; s0 += U) {
    float w[U], v[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + u, ns_b - 1);
      // split s's logsumexp: from lane s for the first 64, else from memory
      const float lss = s < 64 ? __shfl(ls_lane, s, 64) : ls[s];
      w[u] = s0 + u < ns_b ? __builtin_amdgcn_exp2f((lss - lse) * kLog2e) : 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        v[u][c] = s0 == 0 ? v0[u][c] : os[(size_t)s * D + lane + 64 * c];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = fmaf(w[u], v[u][c], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) orow[lane + 64 * c] = (uint16_t)(Ty::pack2(acc[c], 0.f) & 0xffffu);
  if (lane == 0) a.lse[row] = lse;
}

// Matrix-core variant, for a key/value head serving many query rows (grouped
// heads times new tokens): 16 keys and 16 query rows per wave step, on
// v_mfma_f32_16x16x32 (scores S^T = K Q^T) and v_mfma_f32_16x16x16 (output
// O^T += V^T P^T).  The score accumulator's layout (lane: one row, four
// consecutive keys) is exactly the B operand of the output product, and one
// transposing LDS read (ds_read_b64_tr_b16) gives each lane the four keys of
// its V^T operand, so nothing is permuted.  K rows are gathered through the
// block table straight into operand registers (lane: one key's 16-byte
// chunks); V rows pass through a wave-private LDS tile.  Waves take every
// fourth step of the split, with two register sets alternating so one step's
// rows are in flight while the other computes, and merge through LDS at the
// end; splits merge as in the vector kernel.  A step's operands take 32
// registers, so three waves share a SIMD.
template <class Ty> struct M16;
template <> struct M16<TBF16> {
  __device__ static inline f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                     __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
  }
};
template <> struct M16<TF16> {
  __device__ static inline f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
};

// Plain (cached) loads for the matrix-core kernel: each of its load
// instructions covers 64 bytes of 16 rows, and the rows' other bytes follow
// in the next instructions (measured 2.86 against 2.67 TB/s with
// non-temporal loads at 16 rows per key/value head).
__device__ inline u32x4 m16_load(const u32x4 *p) { return *p; }

template <class Ty, int D>
__global__ __launch_bounds__(kThreads, 3) void fa_decode_m16_kernel(DecodeArgs a) {
  constexpr int NK = D / 32;                       // score MFMAs (32 d values each)
  constexpr int NDB = D / 16;                      // output blocks of 16 d values
  constexpr int KCH = D / 8;                       // 16-byte chunks per row
  constexpr int NV = KCH / 4;                      // V chunks per lane per step
  constexpr int TK = 16;                           // keys (and rows) per wave step
  constexpr int VT_BYTES = TK * D * 2;
  static_assert(2 * TK * D * 4 <= 4 * VT_BYTES, "merge buffer must fit in the V tiles");
  __shared__ int tab[kMaxTable];
  __shared__ __attribute__((aligned(16))) char vt_raw[4 * VT_BYTES];
  __shared__ float mrg_m[2][TK], mrg_l[2][TK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g4 = lane >> 4;

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

  const int first = t0 >> sh;
  const int cnt = t1 > t0 ? ((t1 - 1) >> sh) - first + 1 : 0;
  for (int e = tid; e < cnt; e += kThreads) {
    const int v = a.block_table[(size_t)b * a.max_blocks + first + e];
    tab[e] = (v >= 0 && v < a.num_blocks) ? v : -1;
  }

  // This lane's row (shared by lanes i16, i16 + 16, i16 + 32, i16 + 48).
  const int rho = rs * TK + i16;
  const bool row_ok = rho < rows_total;
  int out_row = 0, pos = -1;
  if (row_ok) {
    const int j = rho / a.n_q, i = rho - j * a.n_q;
    out_row = (b * a.H + g * group + j) * a.n_q + i;
    pos = n - a.n_q + i;
  }
  // Q^T as the B operand of S^T = K Q^T: row i16, d values 32*ks + 8*g4 ..
  u32x4 qreg[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
    qreg[ks] = row_ok ? *(const u32x4 *)((const uint16_t *)a.q + (size_t)out_row * D + 32 * ks +
                                         8 * g4)
                      : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) asm volatile("" : "+a"(qreg[ks]));
  const int min_pos = n - a.n_q;
  __syncthreads();

  const size_t blk_stride = (size_t)a.Hkv << sh;
  const uint16_t *kc = (const uint16_t *)a.k_cache + ((size_t)g << sh) * D;
  const uint16_t *vc = (const uint16_t *)a.v_cache + ((size_t)g << sh) * D;
  char *vt = vt_raw + wave * VT_BYTES;
  // Transposing read of output block db: rows (keys) 4*g4 + (lane%16)/4,
  // 4 values from column 16*db + 4*(lane%4); lane receives column
  // 16*db + i16 of keys 4*g4 .. 4*g4 + 3.
  // (The swizzle XORs every chunk-index bit of a row, so each block needs
  // its own lane offset.)
  const int tr_r = 4 * g4 + (i16 >> 2);
  int tr_off[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    tr_off[db] = tr_r * (D * 2) + 16 * swz<D>(tr_r, 2 * db + ((lane & 3) >> 1)) + 8 * (lane & 1);

  // Step j's key i16: K chunks (A operand, d = 32*ks + 8*g4) and V chunks
  // 4*s + g4.  Every lane loads (a missing key reads block 0's first row,
  // always valid memory); missing keys are masked and their V rows zeroed.
  struct Rows {
    u32x4 k[NK], v[NV];
  };
  auto fetch = [&](int j) __attribute__((always_inline)) {
    const int key = t0 + TK * j + i16;
    int blk = -1;
    if (key < t1) blk = tab[(key >> sh) - first];
    const size_t row = blk >= 0 ? ((size_t)blk * blk_stride + (size_t)(key & bs_mask)) * D : 0;
    Rows out;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      out.k[ks] = m16_load((const u32x4 *)(kc + row + 32 * ks + 8 * g4));
#pragma unroll
    for (int s2 = 0; s2 < NV; ++s2)
      out.v[s2] = m16_load((const u32x4 *)(vc + row + 8 * (4 * s2 + g4)));
    return out;
  };

  float m = -INFINITY, l = 0.f;
  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float cl2 = a.scale_log2;
  const int n_steps = (t1 - t0 + TK - 1) / TK;

  auto body = [&](int j, const Rows &cur) __attribute__((always_inline)) {
    const int tk = t0 + TK * j;
    bool key_ok;
    {
      const int key = tk + i16;
      key_ok = key < t1;
      if (key_ok) key_ok = tab[(key >> sh) - first] >= 0;
    }
    const int kvalid = (int)((uint32_t)__builtin_amdgcn_ballot_w64(key_ok) & 0xffffu);
#pragma unroll
    for (int s2 = 0; s2 < NV; ++s2) {
      u32x4 v = cur.v[s2];
      if (kvalid != 0xffff) v = key_ok ? v : u32x4{0, 0, 0, 0};
      *(u32x4 *)(vt + i16 * (D * 2) + 16 * swz<D>(i16, 4 * s2 + g4)) = v;
    }
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) sacc = M16<Ty>::mfma32(cur.k[ks], qreg[ks], sacc);
    // lane: keys 4*g4 + r (r = 0..3) of row i16
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = sacc[r] * cl2;
    if (kvalid != 0xffff || tk + TK - 1 > min_pos) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = 4 * g4 + r;
        const bool vis = ((kvalid >> kr) & 1) && tk + kr <= pos;
        if (!vis) sv[r] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = mx > m + kTau ? mx : m;
    if (__builtin_amdgcn_ballot_w64(m_new != m) != 0) {
      const float al = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      l *= al;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][r] *= al;
      m = m_new;
    }
    const float mu = m == -INFINITY ? 0.f : m;
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pw[r] = __builtin_amdgcn_exp2f(sv[r] - mu);
    l += (pw[0] + pw[1]) + (pw[2] + pw[3]);
    u32x2 ppk;
    ppk[0] = Ty::pack2(pw[0], pw[1]);
    ppk[1] = Ty::pack2(pw[2], pw[3]);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2 va = lds_read_tr16((const FA_LDS void *)(vt + tr_off[db]));
      oacc[db] = M16<Ty>::mfma16(va, ppk, oacc[db]);
    }
  };

  Rows ra = fetch(wave);
  for (int j = wave; j < n_steps; j += 8) {
    const Rows rb = fetch(j + 4);
    body(j, ra);
    ra = fetch(j + 8);
    if (j + 4 < n_steps) body(j + 4, rb);
  }

  // Row sums over the row's four lanes, then the four waves (2, 3 into 0, 1;
  // then 1 into 0) through LDS.
  float lr = l + __shfl_xor(l, 16, 64);
  lr += __shfl_xor(lr, 32, 64);
  float *mo = (float *)vt_raw;  // [2][TK rows][D] fp32, over the V tiles
  __syncthreads();
  auto put = [&](int slot) __attribute__((always_inline)) {
    if (g4 == 0) {
      mrg_m[slot][i16] = m;
      mrg_l[slot][i16] = lr;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *(float4 *)&mo[(slot * TK + i16) * D + 16 * db + 4 * g4] =
          float4{oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]};
  };
  auto take = [&](int slot) __attribute__((always_inline)) {
    const float m2 = mrg_m[slot][i16], l2 = mrg_l[slot][i16];
    const float mm = fmaxf(m, m2);
    const float a1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mm);
    const float a2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mm);
    lr = a1 * lr + a2 * l2;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const float4 v = *(const float4 *)&mo[(slot * TK + i16) * D + 16 * db + 4 * g4];
      oacc[db][0] = a1 * oacc[db][0] + a2 * v.x;
      oacc[db][1] = a1 * oacc[db][1] + a2 * v.y;
      oacc[db][2] = a1 * oacc[db][2] + a2 * v.z;
      oacc[db][3] = a1 * oacc[db][3] + a2 * v.w;
    }
    m = mm;
  };
  if (wave >= 2) put(wave - 2);
  __syncthreads();
  if (wave < 2) take(wave);
  __syncthreads();
  if (wave == 1) put(0);
  __syncthreads();
  if (wave != 0 || !row_ok) return;
  take(0);

  const bool empty = !(lr > 0.f);
  const float inv = empty ? 0.f : 1.f / lr;
  const float lv = empty ? -INFINITY : (m + __builtin_amdgcn_logf(lr)) * 0.69314718055994531f;
  if (ns_b == 1) {
    uint16_t *orow = (uint16_t *)a.o + (size_t)out_row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      u32x2 w;
      w[0] = Ty::pack2(oacc[db][0] * inv, oacc[db][1] * inv);
      w[1] = Ty::pack2(oacc[db][2] * inv, oacc[db][3] * inv);
      *(u32x2 *)(orow + 16 * db + 4 * g4) = w;
    }
    if (g4 == 0) a.lse[out_row] = lv;
  } else {
    const size_t slot = (size_t)out_row * a.n_splits + split;
    float *wo = a.ws_o + slot * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *(float4 *)&wo[16 * db + 4 * g4] =
          float4{oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv};
    if (g4 == 0) a.ws_lse[slot] = lv;
  }
}

template <class Ty, int D>
bool run_decode_m16(const DecodeArgs *a, const DecodePlan *p, hipStream_t stream, bool launch,
                    LaunchInfo *info, hipError_t *err) {
  static char name[96];
  snprintf(name, sizeof(name), "fa_decode_paged_m16<%s,d%d,rows16>", Ty::kName, D);
  info->name = name;
  info->block_rows = 16;
  info->threads = kThreads;
  if (!launch) return true;
  DecodeArgs args = *a;
  void *kargs[] = {&args};
  *err = hipLaunchKernel((const void *)&fa_decode_m16_kernel<Ty, D>, dim3((unsigned)p->grid),
                         dim3(kThreads), kargs, 0, stream);
  if (*err != hipSuccess || p->n_splits == 1) return true;
  const int64_t rows = (int64_t)a->B * a->H * a->n_q;
  *err = hipLaunchKernel((const void *)&fa_decode_merge_kernel<Ty, D>,
                         dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), kargs, 0, stream);
  return true;
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
    case 16:
      if constexpr (D <= 128) return run_decode_m16<Ty, D>(a, p, s, launch, info, err);
      return false;
  }
  return false;
}

template <class Ty>
bool decode_by_dim(int d, const DecodeArgs *a, const DecodePlan *p, hipStream_t s, bool launch,
                   LaunchInfo *info, hipError_t *err) {
  switch (d) {
    case 64: return decode_by_rows<Ty, 64>(a, p, s, launch, info, err);
    case 128: return decode_by_rows<Ty, 128>(a, p, s, launch, info, err);
    case 256: return decode_by_rows<Ty, 256>(a, p, s, launch, info, err);
  }
  return false;
}

}  // namespace

bool decode_plan(int d, int64_t B, int64_t H, int64_t Hkv, int64_t n_q, int64_t ctx_cap,
                 DecodePlan *p) {
  if (d != 64 && d != 128 && d != 256) return false;
  const int64_t rows_total = (H / Hkv) * n_q;
  // A key/value head serving many query rows goes to the matrix-core kernel
  // (16 rows per work-group); up to kMfmaRows - 1 rows stay on the vector
  // ALUs.  Measured: at 4 rows the vector kernel is faster (5.8 against
  // 5.3 TB/s); at 5, 6 and 8 rows the matrix-core kernel (5.3 against 3.3,
  // 5.3 against 3.4, 4.4 against 2.8 TB/s).  The vector kernel takes at most 4
  // rows per work-group: more rows slices (whose repeated cache reads hit
  // the shared L2) measured faster than 8-row work-groups, whose registers
  // cut the waves per SIMD from 5 to 3.
  // At d = 256 every row count takes the vector kernel (in 4-row slices):
  // the matrix-core kernel's two register sets of 16 K and V rows would not
  // fit beside its accumulators.
  p->rows = rows_total <= 1 ? 1 : rows_total <= 2 ? 2
          : (rows_total < kMfmaRows || d == 256) ? 4 : 16;
  p->row_slices = (int)((rows_total + p->rows - 1) / p->rows);
  // Enough work-groups to fill the chip several times over: split each
  // context when requests x key/value heads x row slices alone are too few,
  // but never into pieces shorter than kMinSplit tokens (the merge grows with
  // the number of pieces).  The vector kernel runs up to five work-groups per
  // CU and aims for 4096; the matrix-core kernel, three, and aims for 1024.
  // Both measured best over the decode workloads.
  const int64_t units = B * Hkv * p->row_slices;
  const int64_t target = p->rows >= 16 ? kMfmaGroups : kValuGroups;
  const int64_t want = units >= target ? 1 : (target + units - 1) / units;
  int64_t len = (ctx_cap + want - 1) / want;
  len = (len + 63) / 64 * 64;
  if (want > 1 && len < kMinSplit) len = kMinSplit;
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
