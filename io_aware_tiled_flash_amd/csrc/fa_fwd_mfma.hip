// Exact attention forward for bf16 / fp16 inputs on CDNA4 (gfx950) matrix cores.
//
// Method: the tiled forward pass with the online softmax ("FlashAttention: Why
// Tiling Attention Makes Transformers Fast Without Changing the Result",
// sections "Online softmax: correct as you go" and "The tiled forward pass";
// aicomputerinstitute.com grade-12 flash-attention chapter, section "Tiling
// and the running (online) softmax").  Per query row the kernel keeps a
// running maximum m, a running denominator l and an unnormalised fp32 output
// accumulator; for every visible key tile it rescales l and the accumulator by
// exp(m_old - m_new) when the maximum moves, adds the tile's exponentiated
// scores, and divides by l once after the last tile.  Score and probability
// tiles live only in registers.  The work split over the query sequence (one
// work-group per query tile, per batch and head) follows the same chapter's
// section "What FlashAttention-2 changed"; each wavefront owns distinct query
// rows, so waves never combine partial results.
//
// gfx950 mapping (one work-group = NW wave64s; each wave owns NH blocks of 32
// query rows, "halves"):
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{bf16,f16}: lane (q = lane%32, g = lane/32) then
//     holds 16 of each 32 keys of one query column, so a row maximum or sum is
//     a register reduction plus one exchange with lane^32;
//   * Q^T (the B operand) is loaded once into VGPRs;
//   * K and V tiles go from HBM straight into LDS with 16-byte-per-lane
//     direct buffer loads (no VGPR staging); both are stored row-major
//     [key][d] with a 16-byte-chunk XOR swizzle (chunk ^ (key & 7)), chosen
//     through each lane's global offset, so that the operand reads below are
//     free of bank conflicts;
//   * the K operand of S^T is one ds_read_b128 per lane; the V^T operand of
//     O^T = V^T P^T is two ds_read_b64_tr_b16 transposing reads, which hand
//     each lane four keys of one d column.  The keys each lane receives follow
//     the P^T accumulator layout of S^T, so the scores' registers are used
//     directly as the B operand (a contraction's summation order is free as
//     long as both operands agree on it);
//   * with NH = 2 each K or V operand read from LDS feeds two MFMAs (one per
//     half), halving LDS traffic per flop, and the loop body is ordered
//     S_0, {S_1 | softmax_0}, {O_0 | softmax_1}, O_1 so that one half's
//     vector-ALU softmax can issue while the other half's MFMAs run;
//   * the loads of tile t+1 are issued before the math of tile t into a free
//     LDS stage (K double-buffered, V triple-buffered because the lagging
//     half reads the previous tile's V), with one barrier per tile;
//   * causal and sliding-window masks skip whole tiles: the work-group visits
//     only key tiles that intersect its rows' visible band, a wave skips the
//     math of tiles that are invisible to all of its rows, and the elementwise
//     mask is evaluated only in a separate loop body used for tiles that
//     straddle a band edge;
//   * scores are scaled into base 2 (scale * log2 e) so that every exponential
//     is one v_exp_f32, with the scale folded into the exponent's FMA;
//   * lazy rescaling: the running offset m is only moved when a row's maximum
//     exceeds it by more than TAU (base-2 units); until then exponentials are
//     taken against the stale m, so unnormalised weights stay below 2^TAU.
//     The final O = acc / l and LSE = m + log l use the same m, so the result
//     is unchanged up to rounding (the deferred-rescaling idea of the
//     "What FlashAttention-2 changed" section);
//   * l accumulates the fp32 weights (before they are rounded to the input
//     dtype for the PV product), so the logsumexp is not limited by bf16
//     precision;
//   * heavy query tiles (the last ones, under a causal or window mask) are
//     dispatched first; consecutive work-groups take different heads, so with
//     the round-robin placement over the 8 XCDs all query tiles of one head
//     land on the same XCD and share its L2.
#include "fa_internal.h"

#include <math.h>
#include <stdio.h>

#include <type_traits>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float TAU = 8.0f;  // max growth (base 2) tolerated before rescaling

struct TBF16 {
  static constexpr const char *kName = "bf16";
  __device__ static inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // round-to-nearest-even pack of two floats (v_cvt_pk_bf16_f32)
  __device__ static inline uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
};

struct TF16 {
  static constexpr const char *kName = "f16";
  __device__ static inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // round-to-nearest-even pack of two floats (v_cvt_pk_f16_f32)
  __device__ static inline uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
};

// Raw buffer resource over one head's [S, d] slab: loads past `bytes` return 0,
// which zero-fills ragged tails without branches.  Word 3 = 0x00020000 selects
// the 32-bit data format that raw (untyped) buffer loads need on gfx9 parts.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define FA_LDS __attribute__((address_space(3)))

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds_base + 16 * i (lds_base must be the same in every lane of the wave).
__device__ inline void load16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                     FA_LDS void *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, byte_off, 0, 0, 0);
}

// ds_read_b64_tr_b16: in every group of 16 lanes, lanes 4k..4k+3 name row k
// (4 elements each, 16 in total); lane n of the group receives column n, i.e.
// element n of rows 0..3.
__device__ inline u32x2 lds_read_tr16(const FA_LDS void *p) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4 *)const_cast<FA_LDS void *>(p)));
}

__device__ inline float wave_partner(float x) {  // value held by lane ^ 32
  return __shfl_xor(x, 32, 64);
}

template <int MASK>
__device__ inline bool key_visible(int key, int row, int S, int window) {
  if (MASK == kMaskNone) return key < S;
  if (MASK == kMaskCausal) return key <= row;
  return key <= row && key > row - window;
}

template <class Ty, int D, int MASK, int NW, int BC, int NH>
__global__ __launch_bounds__(NW * 64, 1) void fa_fwd_mfma_kernel(FwdArgs a) {
  constexpr int NT = NW * 64;          // threads per work-group
  constexpr int QW = 32 * NH;          // query rows per wave
  constexpr int BR = QW * NW;          // query rows per work-group
  constexpr int NKB = BC / 32;         // 32-key blocks per key tile
  constexpr int NKS = D / 16;          // contraction steps of S^T = K Q^T
  constexpr int NDB = D / 32;          // 32-wide d blocks of O^T
  constexpr int NPS = BC / 16;         // contraction steps of O^T = V^T P^T
  constexpr int KCH = D / 8;           // 16-byte chunks per K row
  constexpr int TILE_CHUNKS = BC * KCH;  // 16-byte chunks per K or V tile
  constexpr int LOADS_PER_WAVE = TILE_CHUNKS / 64 / NW;  // direct loads per tensor
  static_assert(D % 32 == 0 && BC % 32 == 0, "tile shape");
  static_assert(KCH >= 8, "swizzle needs >= 8 chunks per LDS row");
  static_assert(TILE_CHUNKS % (64 * NW) == 0, "tile must split evenly over the waves");

  // K is double-buffered; V is triple-buffered because the last half's PV
  // product for tile t is issued during tile t+1 (see the loop below).
  __shared__ u32x4 k_lds[2][BC * KCH];
  __shared__ u32x4 v_lds[3][BC * KCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, lg = lane >> 5;
  const int S = a.S;
  const int BH = a.B * a.H;
  const int nq = (S + BR - 1) / BR;

  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if (MASK != kMaskNone) qt = nq - 1 - qt;  // heaviest query tiles first
  const int q0 = qt * BR;

  const size_t head_off = (size_t)bh * (size_t)S * D;  // elements
  const uint32_t head_bytes = (uint32_t)S * D * 2u;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t *)a.q + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t *)a.k + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t *)a.v + head_off, head_bytes);

  // The softmax runs on c * s with c >= 0: a negative scale is applied by
  // flipping the sign bits of Q (exact in bf16 and fp16).
  const float c = fabsf(a.scale_log2);
  const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  // Q^T as the B operand: lane holds Q[row][16*ks + 8*lg .. +7] for every ks.
  const int wr0 = q0 + wave * QW;  // first query row of this wave
  const int wr1 = wr0 + QW - 1;    // last query row of this wave
  u32x4 qreg[NH][NKS];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qreg[h][ks] = load16(rq, (uint32_t)((wr0 + 32 * h + lq) * D + 16 * ks + 8 * lg) * 2u) ^ qflip;

  // Key tiles this work-group visits.
  const int ntk = (S + BC - 1) / BC;
  int kt_begin = 0, kt_end = ntk;
  if (MASK != kMaskNone) {
    const int last_row = min(q0 + BR, S) - 1;
    kt_end = last_row / BC + 1;
    if (MASK == kMaskWindow) kt_begin = max(0, q0 - a.window + 1) / BC;
  }

  // Direct loads of tile kt into K stage kst and V stage vst.  Chunk position
  // p of a stage holds row p / KCH, global chunk (p % KCH) ^ (row & 7).
  auto load_tile = [&](int kt, int kst, int vst) {
    const int k0 = kt * BC;
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int blk = wave * LOADS_PER_WAVE + i;  // 64-chunk block of the tile
      const int pos = 64 * blk + lane;
      const int r = pos / KCH, cc = (pos % KCH) ^ (r & 7);
      const uint32_t off = (uint32_t)((k0 + r) * D + 8 * cc) * 2u;
      load16_to_lds(rk, off, (FA_LDS void *)&k_lds[kst][64 * blk]);
      load16_to_lds(rv, off, (FA_LDS void *)&v_lds[vst][64 * blk]);
    }
  };

  f32x16 oacc[NH][NDB];
  f32x16 sacc[NH][NKB];
  u32x4 pk[NH][NPS];  // packed weights of each half's latest tile
  float m[NH], l[NH], alpha[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[h][i] = f32x16{};
#pragma unroll
    for (int i = 0; i < NPS; ++i) pk[h][i] = u32x4{};
    m[h] = -INFINITY;  // running offset, base 2 (equal in lanes q and q^32)
    l[h] = 0.f;        // this lane's share of the running denominator
    alpha[h] = 1.f;
  }
  // The PV product of the last half (NH-1) lags one tile behind: `pending`
  // says pk[NH-1] / alpha[NH-1] still have to be folded into oacc[NH-1].
  bool pending = false;

  auto s_phase = [&](int kst) __attribute__((always_inline)) {
    const u32x4 *kl = k_lds[kst];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[h][kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int r = 32 * kb + lq;
        const u32x4 op = kl[r * KCH + ((2 * ks + lg) ^ (r & 7))];
#pragma unroll
        for (int h = 0; h < NH; ++h) sacc[h][kb] = Ty::mfma(op, qreg[h][ks], sacc[h][kb]);
      }
  };

  // V^T operand of step kk, d block db: lane (group G = lane/16, n = lane%16)
  // reads rows key = 16*kk + 8*i2 + 4*lg + n/4 at d = 32*db + 16*(G&1) + 4*(n&3)
  // and receives keys 16*kk + 8*i2 + 4*lg + 0..3 of column d = 32*db + lane%32.
  const int tr_key = 4 * lg + ((lane & 15) >> 2);
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto o_mfma = [&](int h, int vst) __attribute__((always_inline)) {
    const char *vl = (const char *)&v_lds[vst][0];
#pragma unroll
    for (int kk = 0; kk < NPS; ++kk)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x4 op;
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const int key = 16 * kk + 8 * i2 + tr_key;
          const int d = 32 * db + tr_d;
          const int off = key * (D * 2) + ((((d >> 3) ^ (key & 7))) << 4) + ((d & 7) << 1);
          const u32x2 v2 = lds_read_tr16((const FA_LDS void *)(vl + off));
          op[2 * i2] = v2[0];
          op[2 * i2 + 1] = v2[1];
        }
        oacc[h][db] = Ty::mfma(op, pk[h][kk], oacc[h][db]);
      }
  };

  auto rescale = [&](int h) __attribute__((always_inline)) {
    if (__any(alpha[h] != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[h][db] *= alpha[h];
    }
  };

  // Online-softmax update of half h from its raw scores in sacc[h]; leaves the
  // packed weights in pk[h] and the accumulator factor in alpha[h].
  auto softmax = [&](int h, auto masked_c, int k0) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int row = wr0 + 32 * h + lq;
    float tmax = -INFINITY;
    if (MASKED) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * lg + (r & 3);
          const float x = key_visible<MASK>(key, row, S, a.window) ? sacc[h][kb][r] * c
                                                                    : -INFINITY;
          sacc[h][kb][r] = x;
          tmax = fmaxf(tmax, x);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[h][kb][r]);
      tmax *= c;  // c >= 0 and every score is finite here
    }
    tmax = fmaxf(tmax, wave_partner(tmax));
    const float m_old = m[h];
    const float m_new = tmax > m_old + TAU ? tmax : m_old;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // row fully masked so far
    alpha[h] = __builtin_amdgcn_exp2f(m_old - m_use);      // 1 if unchanged, 0 from -inf
    m[h] = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < NPS; ++kk) {
      const int kb = kk >> 1, base = 8 * (kk & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p0, p1;
        if (MASKED) {
          p0 = __builtin_amdgcn_exp2f(sacc[h][kb][base + 2 * j] - m_use);
          p1 = __builtin_amdgcn_exp2f(sacc[h][kb][base + 2 * j + 1] - m_use);
        } else {
          p0 = __builtin_amdgcn_exp2f(fmaf(sacc[h][kb][base + 2 * j], c, -m_use));
          p1 = __builtin_amdgcn_exp2f(fmaf(sacc[h][kb][base + 2 * j + 1], c, -m_use));
        }
        pk[h][kk][j] = Ty::pack2(p0, p1);
        lsum += p0 + p1;
      }
    }
    l[h] = l[h] * alpha[h] + lsum;
  };

  // Fold the lagging half's pending tile (whose V sits in stage vst) into O.
  auto flush = [&](int vst) __attribute__((always_inline)) {
    rescale(NH - 1);
    o_mfma(NH - 1, vst);
#pragma unroll
    for (int i = 0; i < NPS; ++i) pk[NH - 1][i] = u32x4{};
    alpha[NH - 1] = 1.f;
  };

  // One key tile.  Phase 1: S for every half (each K operand read once).
  // Phase 2: the lagging half's previous PV product, independent of the
  // softmax of half 0 that issues next to it.  Phase 3 (NH == 2): PV of half
  // 0 next to the softmax of half 1.
  auto tile = [&](auto masked_c, int kst, int vst, int vprev, int k0) __attribute__((always_inline)) {
    s_phase(kst);
    rescale(NH - 1);
    o_mfma(NH - 1, vprev);  // zero weights when nothing is pending
    softmax(0, masked_c, k0);
    if (NH == 2) {
      rescale(0);
      o_mfma(0, vst);
      softmax(NH - 1, masked_c, k0);
    }
  };

  // Zero the V stage that the first tile's lagging product reads, so that its
  // zero weights never meet uninitialised LDS.
  for (int i = tid; i < TILE_CHUNKS; i += NT) v_lds[2][i] = u32x4{};
  if (kt_begin < kt_end) load_tile(kt_begin, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int it = kt - kt_begin;
    const int kst = it & 1, vst = it % 3, vprev = (it + 2) % 3;
    const bool has_next = kt + 1 < kt_end;
    if (has_next) load_tile(kt + 1, (it + 1) & 1, (it + 1) % 3);

    const int k0 = kt * BC;
    bool active = true, need_mask;
    if (MASK == kMaskCausal) {
      active = k0 <= wr1;
      need_mask = k0 + BC - 1 > wr0;
    } else if (MASK == kMaskWindow) {
      active = k0 <= wr1 && k0 + BC - 1 > wr0 - a.window;
      need_mask = k0 + BC - 1 > wr0 || k0 <= wr1 - a.window;
    } else {
      need_mask = k0 + BC > S;
    }
    if (active) {
      if (need_mask)
        tile(std::true_type{}, kst, vst, vprev, k0);
      else
        tile(std::false_type{}, kst, vst, vprev, k0);
      pending = true;
    } else if (pending) {
      flush(vprev);
      pending = false;
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's direct loads landed
    __syncthreads();
  }
  if (pending) flush((kt_end - 1 - kt_begin) % 3);

  // Epilogue: one division per row, RNE to the element type, natural-log LSE.
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int row = wr0 + 32 * h + lq;
    const float l_tot = l[h] + wave_partner(l[h]);
    if (row < S) {
      const float inv = 1.f / l_tot;
      uint16_t *orow = (uint16_t *)a.o + head_off + (size_t)row * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 w;
          w[0] = Ty::pack2(oacc[h][db][4 * j + 0] * inv, oacc[h][db][4 * j + 1] * inv);
          w[1] = Ty::pack2(oacc[h][db][4 * j + 2] * inv, oacc[h][db][4 * j + 3] * inv);
          *(u32x2 *)(orow + 32 * db + 8 * j + 4 * lg) = w;
        }
      }
      if (lg == 0)
        a.lse[(size_t)bh * S + row] =
            (m[h] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    }
  }
}

#ifndef FA_BC128
#define FA_BC128 64
#endif
template <class Ty, int D, int MASK>
struct Instance {
  static constexpr int NW = 4;
  static constexpr int BC = D == 128 ? FA_BC128 : 64;
  static constexpr int NH = D <= 128 ? 2 : 1;
  static constexpr int BR = 32 * NH * NW;
  static bool run(const FwdArgs *a, hipStream_t stream, bool launch, LaunchInfo *info,
                  hipError_t *err) {
    static char name[96];
    static const char *mk[3] = {"none", "causal", "window"};
    snprintf(name, sizeof(name), "fa_fwd_mfma<%s,d%d,%s,br%d,bc%d>", Ty::kName, D, mk[MASK],
             BR, BC);
    info->name = name;
    info->block_rows = BR;
    info->threads = NW * 64;
    if (!launch) return true;
    const int nq = (a->S + BR - 1) / BR;
    const dim3 grid((unsigned)(nq * a->B * a->H));
    const dim3 block(NW * 64);
    FwdArgs args = *a;
    void *kargs[] = {&args};
    *err = hipLaunchKernel((const void *)&fa_fwd_mfma_kernel<Ty, D, MASK, NW, BC, NH>, grid,
                           block, kargs, 0, stream);
    return true;
  }
};

template <class Ty, int D>
bool by_mask(int mask, const FwdArgs *a, hipStream_t s, bool launch, LaunchInfo *info,
             hipError_t *err) {
  switch (mask) {
    case kMaskNone: return Instance<Ty, D, kMaskNone>::run(a, s, launch, info, err);
    case kMaskCausal: return Instance<Ty, D, kMaskCausal>::run(a, s, launch, info, err);
    case kMaskWindow: return Instance<Ty, D, kMaskWindow>::run(a, s, launch, info, err);
  }
  return false;
}

template <class Ty>
bool by_dim(int d, int mask, const FwdArgs *a, hipStream_t s, bool launch, LaunchInfo *info,
            hipError_t *err) {
  switch (d) {
    case 64: return by_mask<Ty, 64>(mask, a, s, launch, info, err);
    case 128: return by_mask<Ty, 128>(mask, a, s, launch, info, err);
    case 256: return by_mask<Ty, 256>(mask, a, s, launch, info, err);
  }
  return false;
}

}  // namespace

bool mfma_forward(DType dt, int d, int mask, const FwdArgs *a, hipStream_t stream, bool launch,
                  LaunchInfo *info, hipError_t *err) {
  if (dt == kBF16) return by_dim<TBF16>(d, mask, a, stream, launch, info, err);
  if (dt == kF16) return by_dim<TF16>(d, mask, a, stream, launch, info, err);
  return false;
}

}  // namespace fa
