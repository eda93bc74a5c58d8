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
//     [key][d] with a 16-byte-chunk XOR swizzle (see swz below), chosen
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
//   * tiles are loaded PF tiles ahead of the math into free LDS stages (PF+1
//     for K, PF+2 for V because the PV products lag one tile), which hides
//     the L2/HBM latency behind several tiles of math; one barrier per tile;
//   * causal and sliding-window masks skip whole tiles: the work-group visits
//     only key tiles that intersect its rows' visible band, and the
//     elementwise mask (scores set to -inf) runs only on tiles that straddle
//     a band edge of a wave's rows;
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

// Buffer resource words for one head's [S, d] slab (same layout as above),
// for the inline-assembly loads below.
__device__ inline u32x4 rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, bytes, 0x00020000u};
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds_addr + 16 * i (lds_addr is wave-uniform).  Issued as inline assembly
// so that the compiler does not track it: it would otherwise wait for every
// outstanding direct load before each LDS read and each barrier, which
// serialises the multi-tile prefetch.  Completion is awaited explicitly with
// s_waitcnt vmcnt (vector-memory loads complete in issue order).
__device__ inline void load16_to_lds(u32x4 rsrc, uint32_t byte_off, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(byte_off), "s"(rsrc)
      : "memory");  // M0 is only ever set by these statements in this kernel
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

// 16-byte chunk position of chunk c in LDS row r (64 banks of 4 bytes: a
// 256-byte bank line).  The chunk is XORed with f(r), which has two jobs:
//   * 16 consecutive rows reading the same logical chunk (the K operand, one
//     ds_read_b128 per lane, 16 lanes per LDS cycle) must land in 16
//     different 16-byte bank groups, so f must be a bijection on 16
//     consecutive rows (on 8 row pairs for d = 64, whose 128-byte rows share
//     a bank line in pairs);
//   * the transposing V reads fetch 4 consecutive keys x 4 consecutive chunks
//     per half wave, so the 4 keys must also differ in the chunk bits above
//     the lowest two, which a plain XOR with the low row bits does not give
//     (it only permutes chunks within groups of four).
// Hence the low row bits go to the high chunk bits: f = 4*(r&3) + (r>>2 & 3)
// for rows of at least 256 bytes; for d = 64 the same rotation applied to the
// row-pair index (r>>1) & 7.
template <int D>
__device__ __host__ constexpr int swz(int r, int c) {
  return D >= 128 ? (c ^ (4 * (r & 3) + ((r >> 2) & 3)))
                  : (c ^ (4 * ((r >> 1) & 1) + ((r >> 2) & 3)));
}

template <class Ty, int D, int MASK, int NW, int BC, int NH, int PF>
__global__ __launch_bounds__(NW * 64, 1) void fa_fwd_mfma_kernel(FwdArgs a) {
  constexpr int QW = 32 * NH;          // query rows per wave
  constexpr int BR = QW * NW;          // query rows per work-group
  constexpr int NKB = BC / 32;         // 32-key blocks per key tile
  constexpr int NKS = D / 16;          // contraction steps of S^T = K Q^T
  constexpr int NDB = D / 32;          // 32-wide d blocks of O^T
  constexpr int NPS = BC / 16;         // contraction steps of O^T = V^T P^T
  constexpr int KCH = D / 8;           // 16-byte chunks per K/V row
  constexpr int TILE_CHUNKS = BC * KCH;  // 16-byte chunks per K or V tile
  constexpr int LOADS_PER_WAVE = TILE_CHUNKS / 64 / NW;  // direct loads per tensor
  static_assert(D % 32 == 0 && BC % 32 == 0 && BC % 16 == 0, "tile shape");
  static_assert(KCH >= 8, "swizzle needs >= 8 chunks per LDS row");
  static_assert(TILE_CHUNKS % (64 * NW) == 0, "tile must split evenly over the waves");

  // Tiles are loaded PF tiles ahead of the one being computed.  K needs PF+1
  // stages; V needs PF+2 because the PV products of tile t are issued during
  // tile t+1.
  constexpr int NKST = PF + 1, NVST = PF + 2;
  constexpr int LOADS_PER_TILE = 2 * LOADS_PER_WAVE;  // per wave, K and V
  static_assert(LOADS_PER_TILE * (PF - 1) < 64, "vmcnt range");
  __shared__ u32x4 k_lds[NKST][TILE_CHUNKS];
  __shared__ u32x4 v_lds[NVST][TILE_CHUNKS];

  const int tid = threadIdx.x;
  // readfirstlane makes the wave index (and everything derived from it) a
  // scalar, so per-wave tile decisions become scalar branches.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const u32x4 rk = rsrc_words((const uint16_t *)a.k + head_off, head_bytes);
  const u32x4 rv = rsrc_words((const uint16_t *)a.v + head_off, head_bytes);

  // The softmax runs on c * s with c > 0: a negative scale is applied by
  // flipping the sign bits of Q (exact in bf16 and fp16), and a zero scale
  // becomes 1e-30, whose products with finite scores are far below fp32
  // resolution of the exponent's result (every weight is still exactly 1),
  // while c * (-inf) stays -inf for masked scores.
  const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);
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
  // Q never meets the vector ALU again: keep it in accumulation registers
  // (MFMA reads its A/B operands from AGPRs too), leaving VGPRs to the softmax.
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+a"(qreg[h][ks]));

  // Key tiles this work-group visits.
  const int ntk = (S + BC - 1) / BC;
  int kt_begin = 0, kt_end = ntk;
  if (MASK != kMaskNone) {
    const int last_row = min(q0 + BR, S) - 1;
    kt_end = last_row / BC + 1;
    if (MASK == kMaskWindow) kt_begin = max(0, q0 - a.window + 1) / BC;
  }

  // Direct loads of tile kt into K stage kst and V stage vst.  Chunk position
  // p of a stage holds row p / KCH, logical chunk c with swz(row, c) == p % KCH
  // (swz is an involution in c).
  auto load_tile = [&](int kt, int kst, int vst) __attribute__((always_inline)) {
    const int k0 = kt * BC;
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int blk = wave * LOADS_PER_WAVE + i;  // 64-chunk block of the tile
      const int pos = 64 * blk + lane;
      const int r = pos / KCH, cc = swz<D>(r, pos % KCH);
      const uint32_t off = (uint32_t)((k0 + r) * D + 8 * cc) * 2u;
      load16_to_lds(rk, off, (uint32_t)(uintptr_t)&k_lds[kst][64 * blk]);
      load16_to_lds(rv, off, (uint32_t)(uintptr_t)&v_lds[vst][64 * blk]);
    }
  };

  f32x16 oacc[NH][NDB];
  f32x16 sacc[NH][NKB];
  u32x4 pk[NH][NPS];  // packed weights of the previous tile, awaiting their PV product
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
  // O accumulators and scores stay in VGPRs (the file is built with the
  // VGPR-destination MFMA form): the softmax and the rare rescale then read
  // them directly, without AGPR copies.
  // The PV products lag one tile: pk / alpha hold the previous tile's
  // weights and factors until the next tile (or the epilogue) multiplies them
  // in.  Initially the weights are zero, and so is the V stage they meet.

  // Per-lane LDS byte offsets.  The swizzle XOR is split into a per-lane base
  // and a compile-time part so every operand read is "lane pointer +
  // immediate".  K operand of step ks, key block kb: row 32*kb + lq, logical
  // chunk 2*ks + lg; one base per ks % KSW.
  constexpr int KSW = D >= 128 ? 8 : 4;
  int k_base[KSW];
#pragma unroll
  for (int j = 0; j < KSW; ++j) k_base[j] = lq * (D * 2) + 16 * swz<D>(lq, 2 * j + lg);

  // V^T operand of step kk, d block db, part i2: lane (group G = lane/16,
  // n = lane%16) names row key = 16*kk + 8*i2 + tr_key (tr_key = 4*lg + n/4)
  // at column d = 32*db + 16*(G&1) + 4*(n&3) and receives keys
  // 16*kk + 8*i2 + 4*lg + 0..3 of column 32*db + lane%32.  The swizzle
  // depends on the row only through its low four bits and leaves chunk bits
  // above the fourth alone, so the offset is a lane base chosen by (i2, the
  // low two bits of db) plus the constant 16*kk rows and 16*(db & ~3) chunks.
  constexpr int NVB = D >= 128 ? 8 : 4;
  int v_base[NVB];
  {
    const int tr_key = 4 * lg + ((lane & 15) >> 2);
    const int tr_c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int j = 0; j < NVB; ++j) {
      const int key = 8 * (j & 1) + tr_key;
      v_base[j] = key * (D * 2) + 16 * swz<D>(key, 4 * (j >> 1) + tr_c) + 8 * (lane & 1);
    }
  }
  auto v_off = [](int kk, int db) constexpr { return 16 * kk * (D * 2) + 64 * (db & ~3); };

  auto s_phase = [&](int kst) __attribute__((always_inline)) {
    const char *kl = (const char *)&k_lds[kst][0];
    const char *kp[KSW];
#pragma unroll
    for (int j = 0; j < KSW; ++j) kp[j] = kl + k_base[j];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[h][kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 op =
            *(const u32x4 *)(kp[ks % KSW] + kb * (32 * D * 2) + 16 * 2 * KSW * (ks / KSW));
#pragma unroll
        for (int h = 0; h < NH; ++h) sacc[h][kb] = Ty::mfma(op, qreg[h][ks], sacc[h][kb]);
      }
    // scores go to the vector ALU next: keep them in VGPRs
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) asm volatile("" : "+v"(sacc[h][kb]));
  };

  // O_h^T += V^T P_h^T for every half, each V operand read once.
  auto o_phase = [&](int vst) __attribute__((always_inline)) {
    const char *vl = (const char *)&v_lds[vst][0];
    const char *vp[NVB];
#pragma unroll
    for (int j = 0; j < NVB; ++j) vp[j] = vl + v_base[j];
#pragma unroll
    for (int kk = 0; kk < NPS; ++kk)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x4 op;
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const u32x2 v2 =
              lds_read_tr16((const FA_LDS void *)(vp[2 * (db & 3) + i2] + v_off(kk, db)));
          op[2 * i2] = v2[0];
          op[2 * i2 + 1] = v2[1];
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) oacc[h][db] = Ty::mfma(op, pk[h][kk], oacc[h][db]);
      }
  };

  auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
      if (__any(alpha[h] != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[h][db] *= alpha[h];
      }
  };

  // Elementwise mask of the raw scores (tiles straddling a band edge):
  // invisible (query, key) pairs become -inf.
  auto apply_mask = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int row = wr0 + 32 * h + lq;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * lg + (r & 3);
          if (!key_visible<MASK>(key, row, S, a.window)) sacc[h][kb][r] = -INFINITY;
        }
    }
  };

  // Online softmax, in pieces that the pipeline below places next to MFMA work.
  // head(h): row maximum of half h's raw scores, new offset and factor.
  // exps(h, kk0, kk1): weights of steps [kk0, kk1) against that offset,
  //   packed for the PV product, with their fp32 sum kept in lpart[h].
  // finish(h): l <- l * alpha + lpart.
  float m_use[NH], lpart[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    m_use[h] = 0.f;
    lpart[h] = -0.f;
  }
  auto sm_head = [&](int h, const f32x16 (&sc)[NKB]) __attribute__((always_inline)) {
    float t4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        t4[r >> 2] = fmaxf(t4[r >> 2], fmaxf(fmaxf(sc[kb][r], sc[kb][r + 1]),
                                             fmaxf(sc[kb][r + 2], sc[kb][r + 3])));
    float tmax = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, tmax),
                                                     __builtin_bit_cast(uint32_t, tmax),
                                                     false, false);
    tmax = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]),
                 __builtin_bit_cast(float, (uint32_t)sw[1])) * c;  // c > 0 keeps order
    const float m_old = m[h];
    const float m_new = tmax > m_old + TAU ? tmax : m_old;
    m_use[h] = m_new == -INFINITY ? 0.f : m_new;          // row fully masked so far
    alpha[h] = __builtin_amdgcn_exp2f(m_old - m_use[h]);  // 1 if unchanged, 0 from -inf
    m[h] = m_new;
    lpart[h] = -0.f;
  };
  auto sm_exps = [&](int h, const f32x16 (&sc)[NKB], u32x4 (&pk_out)[NPS], int kk0, int kk1)
                     __attribute__((always_inline)) {
    float s4[4] = {-0.f, -0.f, -0.f, -0.f};  // -0 + x == x folds away
#pragma unroll
    for (int kk = kk0; kk < kk1; ++kk) {
      const int kb = kk >> 1, base = 8 * (kk & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][base + 2 * j], c, -m_use[h]));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][base + 2 * j + 1], c, -m_use[h]));
        pk_out[kk][j] = Ty::pack2(p0, p1);
        s4[j] += p0 + p1;
      }
    }
    lpart[h] += (s4[0] + s4[1]) + (s4[2] + s4[3]);
  };
  auto sm_finish = [&](int h) __attribute__((always_inline)) {
    l[h] = l[h] * alpha[h] + lpart[h];
  };

  // Software pipeline over key tiles (t = current tile):
  //   phase A: S(t) = K_t Q^T on MFMA, next to the second softmax piece of
  //            tile t-1 (half 1 when a wave has two halves, the second half
  //            of the keys otherwise);
  //   phase B: O += V_{t-1}^T P(t-1)^T on MFMA (both halves share each V
  //            operand), next to the first softmax piece of tile t.
  // Every piece is independent of the MFMAs it issues beside, so the vector
  // ALU and the matrix core work at the same time inside one wave.  The
  // leftover pieces of the last tile run after the loop.
  constexpr int SPLIT = NH == 2 ? NPS : NPS / 2;  // steps done in phase B (NH == 1)
  f32x16 sprev[NKB];  // scores of tile t-1 still awaiting their second piece
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sprev[kb][r] = -INFINITY;

  auto second_piece = [&]() __attribute__((always_inline)) {
    if (NH == 2) {
      sm_head(1, sprev);
      sm_exps(1, sprev, pk[1], 0, NPS);
      sm_finish(1);
    } else {
      sm_exps(0, sprev, pk[0], SPLIT, NPS);
      sm_finish(0);
    }
  };

  auto tile = [&](bool masked, int kst, int vprev, int k0) __attribute__((always_inline)) {
    s_phase(kst);
    second_piece();
    if (masked) apply_mask(k0);
    rescale();  // factors of tile t-1, now complete
    o_phase(vprev);
    // first piece of tile t: half 0 (or the first keys of the only half)
    u32x4 pk0_new[NPS];
#pragma unroll
    for (int i = 0; i < NPS; ++i) pk0_new[i] = pk[0][i];
    sm_head(0, sacc[0]);
    sm_exps(0, sacc[0], pk0_new, 0, SPLIT);
    if (NH == 2) sm_finish(0);
#pragma unroll
    for (int i = 0; i < NPS; ++i) pk[0][i] = pk0_new[i];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sprev[kb] = sacc[NH - 1][kb];
  };

  // Zero the V stage that the first tile's (empty) pending product reads, so
  // that its zero weights never meet uninitialised LDS.
  for (int i = tid; i < TILE_CHUNKS; i += NW * 64) v_lds[NVST - 1][i] = u32x4{};
  // Prefetches past the last tile read an index beyond the sequence: the
  // buffer range check turns them into zero fills of a free stage, so every
  // tile issues the same number of loads and the waits below are constants
  // (no branch splits the loop body).
  const int kt_none = ntk + PF;
  auto tile_or_none = [&](int kt) { return kt < kt_end ? kt : kt_none; };
#pragma unroll
  for (int i = 0; i < PF; ++i) load_tile(tile_or_none(kt_begin + i), i, i);
  // Wait for the first tile only (and the zero fill); the later prefetches
  // stay in flight.
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LOADS_PER_TILE * (PF - 1)) : "memory");
  __builtin_amdgcn_s_barrier();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int it = kt - kt_begin;
    const int kst = it % NKST, vprev = (it + NVST - 1) % NVST;
    load_tile(tile_or_none(kt + PF), (it + PF) % NKST, (it + PF) % NVST);

    // Every wave runs every tile of the work-group's range; a tile that lies
    // outside a wave's band is simply fully masked (weights 0, factor 1).
    // That costs a few percent of MFMA work on band edges but keeps a single
    // copy of each phase in the loop.
    const int k0 = kt * BC;
    bool need_mask;
    if (MASK == kMaskCausal)
      need_mask = k0 + BC - 1 > wr0;
    else if (MASK == kMaskWindow)
      need_mask = k0 + BC - 1 > wr0 || k0 <= wr1 - a.window;
    else
      need_mask = k0 + BC > S;
    tile(need_mask, kst, vprev, k0);

    // Tile kt+1 must have landed (this wave's share); tiles kt+2 .. kt+PF may
    // still be in flight.
    // Tile kt+1 has landed once at most PF-1 tiles' loads are outstanding.
    // Every LDS read of this tile was consumed by an MFMA above, so after the
    // barrier the stages read here may be overwritten.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS_PER_TILE * (PF - 1)) : "memory");
    __builtin_amdgcn_s_barrier();
  }
  // The last tile: its second softmax piece, then its PV products.
  second_piece();
  rescale();
  if (kt_begin < kt_end) o_phase((kt_end - 1 - kt_begin) % NVST);

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

#ifndef FA_BC64
#define FA_BC64 64
#endif
#ifndef FA_BC128
#define FA_BC128 32
#endif
#ifndef FA_BC256
#define FA_BC256 32
#endif
#ifndef FA_PF
#define FA_PF 2
#endif
template <class Ty, int D, int MASK>
struct Instance {
  static constexpr int NW = 4;
  static constexpr int BC = D == 64 ? FA_BC64 : D == 128 ? FA_BC128 : FA_BC256;
  static constexpr int NH = D <= 128 ? 2 : 1;
  static constexpr int PF = D == 256 && FA_PF > 3 ? 3 : FA_PF;  // LDS budget
  static constexpr int BR = 32 * NH * NW;
  static bool run(const FwdArgs *a, hipStream_t stream, bool launch, LaunchInfo *info,
                  hipError_t *err) {
    static char name[96];
    static const char *mk[3] = {"none", "causal", "window"};
    snprintf(name, sizeof(name), "fa_fwd_mfma<%s,d%d,%s,br%d,bc%d,pf%d>", Ty::kName, D,
             mk[MASK], BR, BC, PF);
    info->name = name;
    info->block_rows = BR;
    info->threads = NW * 64;
    if (!launch) return true;
    const int nq = (a->S + BR - 1) / BR;
    const dim3 grid((unsigned)(nq * a->B * a->H));
    const dim3 block(NW * 64);
    FwdArgs args = *a;
    void *kargs[] = {&args};
    *err = hipLaunchKernel((const void *)&fa_fwd_mfma_kernel<Ty, D, MASK, NW, BC, NH, PF>, grid,
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
