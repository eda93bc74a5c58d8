// Exact attention forward for bf16 / fp16 inputs on CDNA4 (gfx950) matrix cores.
//
// Method: the tiled forward pass with the online softmax ("FlashAttention: Why
// Tiling Attention Makes Transformers Fast Without Changing the Result",
// sections "Online softmax: correct as you go" and "The tiled forward pass";
// aicomputerinstitute.com grade-12 flash-attention chapter, section "Tiling
// and the running (online) softmax").  Per query row the kernel keeps a
// running offset m (the role of the running maximum), a running denominator
// l and an unnormalised fp32 output accumulator; for every visible key tile
// it adds the tile's exponentiated scores exp(s - m), moves m up to the
// tile's maximum (rescaling l and the accumulator by exp(m_old - m_new)) when
// those weights would grow too large, and divides by l once after the last
// tile.  Score and probability
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
//     half), halving LDS traffic per flop;
//   * the vector-ALU softmax work of a tile is spread over the MFMAs of two
//     phases (see the tile loop below), so that the matrix core runs while
//     the wave issues it;
//   * tiles are loaded PF tiles ahead of the math into free LDS stages (PF+1
//     for K, PF+2 for V because the PV products lag one tile), which hides
//     the L2/HBM latency behind several tiles of math; one barrier per tile;
//   * causal and sliding-window masks skip whole tiles: the work-group visits
//     only key tiles that intersect its rows' visible band, and the
//     elementwise mask (scores set to -inf) runs only on tiles that straddle
//     a band edge of a wave's rows;
//   * scores are scaled into base 2 (scale * log2 e) so that every exponential
//     is one v_exp_f32, with the scale folded into the exponent's FMA;
//   * lazy offset: the exponentials of a tile are taken against the row's
//     current offset m without first looking at the tile's maximum.  Only a
//     lane whose tile weight sum exceeds a cap (2^32 for bf16 weights, which
//     share fp32's exponent range; 2^8 for fp16), or a row that has no
//     offset yet, sends the wave to a rare branch that takes the true row
//     maximum of the tile, moves m up to it, rescales the accumulator and
//     denominator by exp(m_old - m_new) and recomputes the tile's weights.
//     Every final O = acc / l and LSE = m + log l uses one m per row, so the
//     result is unchanged up to rounding (the deferred-rescaling idea of the
//     "What FlashAttention-2 changed" section, taken one step further: the
//     common path computes no row maximum at all);
//   * l sums the fp32 weights (before they are rounded to the input dtype
//     for the PV product), so the logsumexp is not limited by bf16
//     precision.  The key-split instances (small grids) also keep lt, the
//     sum of the rounded weights the PV product actually used, and
//     normalise O by it: O is then an exact convex combination of V rows
//     with weights p~/sum p~, and a row dominated by one key returns that
//     key's V row exactly, where dividing by the fp32 sum carries the
//     dominant weight's rounding (up to 2^-8 of |V| in bf16, when the lazy
//     offset left that weight inexact) into O.  The other instances divide
//     by l: the second sum costs about 7% of their throughput;
//   * heavy query tiles (the last ones, under a causal or window mask) are
//     dispatched first; consecutive work-groups take different heads, so with
//     the round-robin placement over the 8 XCDs all query tiles of one head
//     land on the same XCD and share its L2;
//   * grids too small to fill the chip split the keys as well: the waves of
//     a work-group form NR row groups times NK key groups, key group g takes
//     every NK-th key tile of the work-group's band (each group with LDS
//     stages of its own, all groups in step), and at the end the NK partial
//     results of each row are merged through LDS with the same rescaling
//     algebra (m = max m_g, l = sum l_g 2^(m_g - m), O = sum O_g 2^(m_g - m)
//     / l).  This is the extra parallelism over the sequence of the chapter's
//     "What FlashAttention-2 changed" section, taken along the keys, so that
//     a short sequence's last query tile no longer runs all of its key tiles
//     one after another on one wave.
#include "fa_gfx950.h"

#include <math.h>
#include <stdio.h>

#include <type_traits>

namespace fa {
namespace {

using namespace tile;

// As load16_to_lds (M0 handling included), for an LDS address that is
// already wave-uniform (a scalar): no v_readfirstlane per load.
__device__ inline void load16_to_lds_s(u32x4 rsrc, uint32_t byte_off, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(byte_off), "s"(rsrc)
      : "memory");
}

// f(stage phase P, it + P) for P = P0 .. N-1, each with a compile-time phase.
template <int P0, int N, class F>
__device__ inline __attribute__((always_inline)) void unroll_steps(F &f, int it) {
  if constexpr (P0 < N) {
    f(std::integral_constant<int, P0>{}, it + P0);
    unroll_steps<P0 + 1, N>(f, it);
  }
}

// Offset-move cap: a lane's tile weight sum above it sends the wave to the
// offset update.  bf16 weights share fp32's exponent range, so they may grow
// to 2^32 before the offset has to move (the accumulator then stays below
// 2^52 times the largest |V|); fp16 weights must stay below 65504, so they
// move it at 2^8.
template <class Ty> struct WeightCap;
template <> struct WeightCap<TBF16> { static constexpr float value = 4294967296.0f; };
template <> struct WeightCap<TF16> { static constexpr float value = 256.0f; };

template <class Ty, int D, int MASK, int NW, int NK, int BC, int NH, int PF>
__global__ __launch_bounds__(NW * 64, 1) void fa_fwd_mfma_kernel(FwdArgs a) {
  constexpr int NR = NW / NK;          // row groups (one wave each per key group)
  constexpr int QW = 32 * NH;          // query rows per wave
  constexpr int BR = QW * NR;          // query rows per work-group
  constexpr int NKB = BC / 32;         // 32-key blocks per key tile
  constexpr int NKS = D / 16;          // contraction steps of S^T = K Q^T
  constexpr int NDB = D / 32;          // 32-wide d blocks of O^T
  constexpr int NPS = BC / 16;         // contraction steps of O^T = V^T P^T
  constexpr int KCH = D / 8;           // 16-byte chunks per K/V row
  constexpr int TILE_CHUNKS = BC * KCH;  // 16-byte chunks per K or V tile
  // The NR waves of a key group load its tiles together.
  constexpr int LOADS_PER_WAVE = TILE_CHUNKS / 64 / NR;  // direct loads per tensor
  static_assert(NW % NK == 0, "key groups must split the waves evenly");
  static_assert(D % 32 == 0 && BC % 32 == 0 && BC % 16 == 0, "tile shape");
  static_assert(KCH >= 8, "swizzle needs >= 8 chunks per LDS row");
  static_assert(TILE_CHUNKS % (64 * NR) == 0, "tile must split evenly over a group's waves");

  // Tiles are loaded PF tiles ahead of the one being computed.  K needs PF+1
  // stages; V needs PF+2 because the PV products of tile t are issued during
  // tile t+1.  Both get NST = PF+2 stages so that one index, it % NST with
  // it = kt - kt_begin, names the stages of a tile; the tile loop is unrolled
  // NST times, which makes every stage offset a compile-time immediate of the
  // LDS instructions.
  constexpr int NST = PF + 2;
  constexpr int NVST = NST;
  constexpr int LOADS_PER_TILE = 2 * LOADS_PER_WAVE;  // per wave, K and V
  static_assert(LOADS_PER_TILE * (PF - 1) < 64, "vmcnt range");
  // K and V stages per key group (separate arrays: each operand read's LDS
  // offset then stays within the 16-bit immediate of the instruction).
  __shared__ u32x4 k_lds[NK][NST][TILE_CHUNKS];
  __shared__ u32x4 v_lds[NK][NST][TILE_CHUNKS];

  const int tid = threadIdx.x;
  // readfirstlane makes the wave index (and everything derived from it) a
  // scalar, so per-wave tile decisions become scalar branches.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // row group and key group (compile-time 0 without a key split)
  const int rg = NK == 1 ? wave : wave % NR, kg = NK == 1 ? 0 : wave / NR;
  const int lq = lane & 31, lg = lane >> 5;
  const int S = a.S;
  const int BH = a.B * a.H;
  const int nq = (S + BR - 1) / BR;

  // Work-group b runs on XCD b % 8.  Masked launches take one query tile of
  // each head at a time, heaviest first (their tiles differ in work).
  // Unmasked ones, whose tiles are all alike, run every query tile of one
  // head in a row on its XCD, so the XCD's resident work-groups share few
  // heads' K and V in its L2.
  int slot = blockIdx.x % BH, qt = blockIdx.x / BH;
  if (MASK != kMaskNone) {
    qt = nq - 1 - qt;
  } else if (BH % 8 == 0) {
    const int xcd = blockIdx.x % 8, l = blockIdx.x / 8;
    slot = (l / nq) * 8 + xcd;
    qt = l % nq;
  }
  const HeadPair hp = head_of_slot(slot, a.B, a.H, a.Hkv);
  const int bh = hp.q;
  const int q0 = qt * BR;

  const size_t head_off = (size_t)bh * (size_t)S * D;     // q, o (elements)
  const size_t kv_off = (size_t)hp.kv * (size_t)S * D;    // k, v (elements)
  const uint32_t head_bytes = (uint32_t)S * D * 2u;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t *)a.q + head_off, head_bytes);
  const u32x4 rk = rsrc_words((const uint16_t *)a.k + kv_off, head_bytes);
  const u32x4 rv = rsrc_words((const uint16_t *)a.v + kv_off, head_bytes);

  // The softmax runs on c * s with c > 0: a negative scale is applied by
  // flipping the sign bits of Q (exact in bf16 and fp16), and a zero scale
  // becomes 1e-30, whose products with finite scores are far below fp32
  // resolution of the exponent's result (every weight is still exactly 1),
  // while c * (-inf) stays -inf for masked scores.
  const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);
  const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  // Q^T as the B operand: lane holds Q[row][16*ks + 8*lg .. +7] for every ks.
  const int wr0 = q0 + rg * QW;    // first query row of this wave
  const int wr1 = wr0 + QW - 1;    // last query row of this wave
  u32x4 qreg[NH][NKS];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qreg[h][ks] = load16(rq, (uint32_t)((wr0 + 32 * h + lq) * D + 16 * ks + 8 * lg) * 2u);

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
  // LDS byte address of this wave's first 64-chunk block in stage 0 of its
  // key group's K and V: wave-uniform, so every direct load's LDS address is
  // a scalar plus a compile-time offset.
  const uint32_t k_lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)&k_lds[kg][0][64 * rg * LOADS_PER_WAVE]);
  const uint32_t v_lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)&v_lds[kg][0][64 * rg * LOADS_PER_WAVE]);
  constexpr uint32_t STAGE_BYTES = TILE_CHUNKS * 16;
  constexpr uint32_t GROUP_BYTES = NST * STAGE_BYTES;  // one key group's stages
  auto load_tile = [&](int kt, int kst, int vst) __attribute__((always_inline)) {
    const int k0 = kt * BC;
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int blk = rg * LOADS_PER_WAVE + i;  // 64-chunk block of the tile
      const int pos = 64 * blk + lane;
      const int r = pos / KCH, cc = swz<D>(r, pos % KCH);
      const uint32_t off = (uint32_t)((k0 + r) * D + 8 * cc) * 2u;
      load16_to_lds_s(rk, off, k_lds0 + kst * STAGE_BYTES + 1024u * i);
      load16_to_lds_s(rv, off, v_lds0 + vst * STAGE_BYTES + 1024u * i);
    }
  };

  f32x16 oacc[NH][NDB];
  f32x16 sacc[NH][NKB];
  u32x4 pk[NH][NPS];  // packed weights of the previous tile, awaiting their PV product
  float m[NH], l[NH], lt[NH];
  float m_use[NH], lpart[NH], ltpart[NH];  // offset the exponents use; a tile's weight sums
#pragma unroll
  for (int h = 0; h < NH; ++h) {
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[h][i] = f32x16{};
#pragma unroll
    for (int i = 0; i < NPS; ++i) pk[h][i] = u32x4{};
    m[h] = -INFINITY;  // running offset, base 2 (equal in lanes q and q^32)
    l[h] = 0.f;        // this lane's share of the running denominator (fp32 weights)
    lt[h] = 0.f;       // the same over the rounded weights
    m_use[h] = 0.f;
    lpart[h] = -0.f;
    ltpart[h] = -0.f;
  }
  // O accumulators and scores stay in VGPRs (the file is built with the
  // VGPR-destination MFMA form): the softmax and the rare rescale then read
  // them directly, without AGPR copies.
  // The PV products lag one tile: pk holds the previous tile's weights until
  // the next tile (or the epilogue) multiplies them in.  Initially the
  // weights are zero, and so is the V stage they meet.

  // Per-lane LDS byte offsets.  The swizzle XOR is split into a per-lane base
  // and a compile-time part so every operand read is "lane pointer +
  // immediate"; the bases include the offset of the wave's key group, so
  // operand reads address the stages as those of key group 0.  K operand of
  // step ks, key block kb: row 32*kb + lq, logical chunk 2*ks + lg; one base
  // per ks % KSW.
  constexpr int KSW = D >= 128 ? 8 : 4;
  const int group_off = kg * (int)GROUP_BYTES;
  int k_base[KSW];
#pragma unroll
  for (int j = 0; j < KSW; ++j)
    k_base[j] = group_off + lq * (D * 2) + 16 * swz<D>(lq, 2 * j + lg);

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
      v_base[j] = group_off + key * (D * 2) + 16 * swz<D>(key, 4 * (j >> 1) + tr_c) +
                  8 * (lane & 1);
    }
  }
  // The V stages follow the K stages in LDS.  With several key groups or
  // d = 256 they reach past 64 KB, beyond the 16-bit offset of an LDS
  // instruction: the bases then carry the V array's LDS address themselves
  // (opaque to the compiler, which would otherwise fold it back into the
  // constant and add it with a vector instruction before each read), so
  // that the stage and step stay in the offset field.
  constexpr bool V_FAR = sizeof(k_lds) + NST * STAGE_BYTES > 65536;
  uint32_t v_at[NVB];
#pragma unroll
  for (int j = 0; j < NVB; ++j) {
    v_at[j] = (V_FAR ? (uint32_t)(uintptr_t)&v_lds[0][0][0] : 0u) + (uint32_t)v_base[j];
    if (V_FAR) asm volatile("" : "+v"(v_at[j]));
  }
  auto v_off = [](int kk, int db) constexpr { return 16 * kk * (D * 2) + 64 * (db & ~3); };

  // K operand of score step st = (ks, kb): 16 bytes per lane.
  auto read_k = [&](const char *kl, int st) __attribute__((always_inline)) {
    const int ks = st / NKB, kb = st % NKB;
    return *(const u32x4 *)(kl + k_base[ks % KSW] + kb * (32 * D * 2) + 16 * 2 * KSW * (ks / KSW));
  };
  // V^T operand of product step st = (kk, db) from the V stage at byte
  // offset vs of the V array: two transposing reads.
  auto read_v = [&](uint32_t vs, int st) __attribute__((always_inline)) {
    const int kk = st / NDB, db = st % NDB;
    u32x4 op;
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const uint32_t o = v_at[2 * (db & 3) + i2] + vs + v_off(kk, db);
      const u32x2 v2 = lds_read_tr16(
          V_FAR ? (const FA_LDS void *)(uintptr_t)o
                : (const FA_LDS void *)((const char *)&v_lds[0][0][0] + o));
      op[2 * i2] = v2[0];
      op[2 * i2 + 1] = v2[1];
    }
    return op;
  };
  // O_h^T += V^T P_h^T for every half, without interleaved work (last tile).
  auto o_phase = [&](int vst) __attribute__((always_inline)) {
    const uint32_t vl = (uint32_t)vst * STAGE_BYTES;
#pragma unroll
    for (int st = 0; st < NPS * NDB; ++st) {
      const u32x4 op = read_v(vl, st);
#pragma unroll
      for (int h = 0; h < NH; ++h)
        oacc[h][st % NDB] = Ty::mfma(op, pk[h][st / NDB], oacc[h][st % NDB]);
    }
  };

  // Elementwise mask of the raw scores of a tile that straddles an edge of
  // this wave's visible band or lies outside it: invisible (query, key)
  // pairs become -inf.  The band test is made once per 32-row half (scalar
  // branches): a half that sees none of the tile's keys is set to -inf
  // outright, and a half that straddles an edge tests, per score, only the
  // inequality of that edge (key <= row at the diagonal, key > row - window
  // at a window's lower edge, key < S at the end of the sequence).
  auto apply_mask = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int r0 = wr0 + 32 * h, r1 = r0 + 31;  // the half's rows
      const int kl = k0 + BC - 1;                  // the tile's last key
      bool none_visible, upper = false, lower = false, tail = false;
      if (MASK == kMaskNone) {
        none_visible = k0 >= S;
        tail = kl >= S;
      } else {
        none_visible = k0 > r1;
        upper = kl > r0;
        if (MASK == kMaskWindow) {
          none_visible = none_visible || kl <= r0 - a.window;
          lower = k0 <= r1 - a.window;
        }
      }
      // Score (kb, r) of this lane holds key k0 + 4 * lg + off(kb, r) of
      // row r0 + lq; each edge test compares the compile-time offset with
      // one per-lane bound (no index arithmetic per score).
      const int kbase = k0 + 4 * lg, row = r0 + lq;
      auto off = [](int kb, int r) constexpr { return 32 * kb + 8 * (r >> 2) + (r & 3); };
      if (none_visible) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[h][kb][r] = -INFINITY;
        continue;
      }
      if (upper) {  // key > row
        const int t = row - kbase;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (off(kb, r) > t) sacc[h][kb][r] = -INFINITY;
      }
      if (MASK == kMaskWindow && lower) {  // key <= row - window
        const int t = row - a.window - kbase;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (off(kb, r) <= t) sacc[h][kb][r] = -INFINITY;
      }
      if (MASK == kMaskNone && tail) {  // key >= S
        const int t = S - kbase;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (off(kb, r) >= t) sacc[h][kb][r] = -INFINITY;
      }
    }
  };

  // Online softmax, in units that the pipeline below places between MFMAs.
  // Contraction step kk of the PV product covers, in each lane, the 8 scores
  // sc[kk/2][8*(kk%2) .. +7]; weights are exp2(c*s - offset).
  //   argument unit (phase B of tile t): four exponent arguments c*s - offset
  //     of one half and step, from the tile's scores;
  //   weight unit: two weights from saved arguments, packed for the PV
  //     product and added to the lane's sums.  The weights of the first NPS/2
  //     steps (at most UAB units) are made in the second half of phase B of
  //     tile t, once the products of tile t-1 have read those registers; the
  //     rest in phase A of tile t+1;
  //   finish (end of phase A of tile t+1): the lane's tile sums, the test
  //     that sends the wave to the offset update, and the denominators.
  // Only exponent arguments and weights cross from one tile to the next, so
  // no score registers are copied along the loop.
  float xdef[NH][NPS][8];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int i = 0; i < NPS; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) xdef[h][i][j] = -INFINITY;

  constexpr int KKB = NPS / 2;                 // steps whose weights phase B may make
  constexpr int UAB_ALL = NH * KKB * 4;
  constexpr int UAB = 8 < UAB_ALL ? 8 : UAB_ALL;  // weight units phase B makes
  constexpr int UA = NH * NPS * 4 - UAB;       // weight units left to phase A
  constexpr float CAP = WeightCap<Ty>::value;
  float s4a[NH][4], s4t[NH][4];  // a tile's partial sums, fp32 and rounded weights
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) s4a[h][j] = s4t[h][j] = -0.f;
  auto sums_start = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) s4a[h][j] = s4t[h][j] = -0.f;  // -0 + x == x folds away
  };
  // Weight units in step-major order: r -> (half (r/4) % NH, step r/(4 NH),
  // pair r % 4); phase B makes r < UAB, phase A the rest.  Each unit runs in
  // two stages: the exponentials of unit r are issued together with the pack
  // and sums of unit r - 1 (w_exp(r), then w_fin(r - 1)), so that neither
  // waits on the other's latency (a wave runs alone on its SIMD: nothing
  // else hides an exponential's latency from the pack that reads it).
  float pe[2][2];
  auto w_exp = [&](int r) __attribute__((always_inline)) {
    const int h = (r / 4) % NH, kk = r / (4 * NH), j = r % 4;
    pe[r & 1][0] = __builtin_amdgcn_exp2f(xdef[h][kk][2 * j]);
    pe[r & 1][1] = __builtin_amdgcn_exp2f(xdef[h][kk][2 * j + 1]);
    pin(pe[r & 1][0]);
    pin(pe[r & 1][1]);
  };
  auto w_fin = [&](int r) __attribute__((always_inline)) {
    const int h = (r / 4) % NH, kk = r / (4 * NH), j = r % 4;
    const float p0 = pe[r & 1][0], p1 = pe[r & 1][1];
    pk[h][kk][j] = Ty::pack2(p0, p1);
    s4a[h][j] += p0 + p1;
    if constexpr (NK > 1) s4t[h][j] = Ty::add2(pk[h][kk][j], s4t[h][j]);
    pin(pk[h][kk][j]);
    pin(s4a[h][j]);
    if constexpr (NK > 1) pin(s4t[h][j]);
  };
  auto a_unit = [&](int u) __attribute__((always_inline)) {
    w_exp(u + UAB);
    if (u > 0) w_fin(u - 1 + UAB);
  };
  auto a_unit_last = [&]() __attribute__((always_inline)) { if (UA > 0) w_fin(UA - 1 + UAB); };

  // Offset update, off the common path.  The weights above were taken
  // against the current offset without looking at the tile's maximum.  A
  // lane whose tile sum exceeds CAP may hold a weight above CAP, and a row
  // that has seen no visible key yet has no offset; either sends the wave
  // here.  The row maximum t of the exponent arguments is taken over both
  // lanes of each row; a row with an offset moves it up by max(t, 0),
  // scaling its accumulator and denominator by exp2(-shift); a row without
  // one takes the maximum itself (its accumulator and denominator are still
  // 0).  The tile's weights are then recomputed against the new offset, so
  // every weight of a row stays at most CAP times its offset's weight.  The
  // accumulator holds the tiles before this one (their products were all
  // issued in the phase before), so the rescale and the recomputed weights
  // agree.
  auto settle = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float t = xdef[h][0][0];
#pragma unroll
      for (int kk = 0; kk < NPS; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) t = fmaxf(t, xdef[h][kk][j]);
      t = fmaxf(t, wave_partner(t));
      const bool fresh = m[h] == -INFINITY;
      const float shift = fresh ? (t == -INFINITY ? 0.f : t) : fmaxf(t, 0.f);
      const float alpha = fresh ? 1.f : __builtin_amdgcn_exp2f(-shift);
      if (!(fresh && t == -INFINITY)) m[h] = m_use[h] + shift;
      m_use[h] = m[h] == -INFINITY ? 0.f : m[h];
      float sum = 0.f, sumt = 0.f;
#pragma unroll
      for (int kk = 0; kk < NPS; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(xdef[h][kk][2 * j] - shift);
          const float p1 = __builtin_amdgcn_exp2f(xdef[h][kk][2 * j + 1] - shift);
          pk[h][kk][j] = Ty::pack2(p0, p1);
          sum += p0 + p1;
          if constexpr (NK > 1) sumt = Ty::add2(pk[h][kk][j], sumt);
        }
      lpart[h] = sum;
      ltpart[h] = sumt;
      l[h] *= alpha;
      if constexpr (NK > 1) lt[h] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[h][db] *= alpha;
    }
  };
  // `force` (the finish of the first tile) always takes the update: every row
  // gets its offset there, except under a window, where a row's first
  // visible key can lie in a later tile; `fresh` says that the finished tile
  // may hold some of this wave's rows' first visible keys, and only then are
  // rows without an offset looked for.
  auto a_finish = [&](bool force, bool fresh) __attribute__((always_inline)) {
    bool trig = false;
    uint64_t votes = 0;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      lpart[h] = (s4a[h][0] + s4a[h][1]) + (s4a[h][2] + s4a[h][3]);
      votes |= __builtin_amdgcn_ballot_w64(lpart[h] > CAP);
      if constexpr (NK > 1) ltpart[h] = (s4t[h][0] + s4t[h][1]) + (s4t[h][2] + s4t[h][3]);

      if (MASK == kMaskWindow && fresh) trig = trig || m[h] == -INFINITY;
    }
    if (force || votes != 0 ||
        (MASK == kMaskWindow && fresh && __builtin_amdgcn_ballot_w64(trig) != 0))
      settle();
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      l[h] += lpart[h];
      pin(l[h]);
      if constexpr (NK > 1) {
        lt[h] += ltpart[h];
        pin(lt[h]);
      }
    }
  };

  // Argument units, in step-major order: u -> (step u / (2 NH), half
  // (u / 2) % NH, four arguments 4 * (u % 2) ..), so the first steps'
  // arguments are ready before their weight units.
  constexpr int UB = 2 * NPS * NH;
  auto b_unit = [&](int u) __attribute__((always_inline)) {
    const int kk = u / (2 * NH), h = (u / 2) % NH, part = u % 2;
    const int kb = kk >> 1, base = 8 * (kk & 1) + 4 * part;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xdef[h][kk][4 * part + i] = fmaf(sacc[h][kb][base + i], c, -m_use[h]);
      pin(xdef[h][kk][4 * part + i]);
    }
  };

  // One tile, software-pipelined (t = this tile):
  //   phase A: S(t) = K_t Q^T on MFMA, next to the remaining weight units of
  //            tile t-1, its finish (offset test and the rare update) under
  //            the last few score MFMAs, the direct loads of tile t+PF, and
  //            the first V operand reads of phase B;
  //   phase B: O += V_{t-1}^T P(t-1)^T on MFMA (both halves share each V
  //            operand), next to the argument units of tile t in its first
  //            half and tile t's first weight units in its second half,
  //            after the products that read those weight registers.
  // Both phases are written as a sequence of steps (operand read RPD steps
  // ahead, one MFMA, its share of the ALU units) separated by scheduling
  // fences, so the instruction stream alternates matrix and vector work in
  // this order: the matrix core runs each MFMA while the wave issues the ALU
  // work behind it.
  constexpr int NSA = NKS * NKB, MA = NSA * NH;  // score steps, MFMAs
  constexpr int NSB = NPS * NDB, MB = NSB * NH;  // product steps, MFMAs
  constexpr int NDMA = 2 * LOADS_PER_WAVE;       // direct loads per tile
  constexpr int RPD = 2;                         // operand reads run RPD steps ahead
  constexpr int UA_PRE = 1 < UA ? 1 : UA;        // units before the first MFMA
  // Tile with stage phase P = it % NST: K in stage P, the previous tile's V
  // in stage P-1, loads of tile it+PF into stage P+PF.
  auto tile = [&](bool masked, bool first, bool fresh, auto phase_c, int k0, int lkt)
                  __attribute__((always_inline)) {
    constexpr int P = decltype(phase_c)::value;
    constexpr int kst = P, vprev = (P + NST - 1) % NST, lks = (P + PF) % NST, lvs = lks;
    const char *kl = (const char *)&k_lds[0][kst][0];
    constexpr uint32_t vl = vprev * STAGE_BYTES;
    const int lk0 = lkt * BC;
    // Direct load d of tile t+PF (K and V alternate), issued after MFMA 2d+1
    // of phase A (placements over both phases, or all at once, measured no
    // better).
    auto dma = [&](int d) __attribute__((always_inline)) {
      const int i = d >> 1;
      const int blk = rg * LOADS_PER_WAVE + i;
      const int pos = 64 * blk + lane;
      const int r = pos / KCH, cc = swz<D>(r, pos % KCH);
      const uint32_t off = (uint32_t)((lk0 + r) * D + 8 * cc) * 2u;
      if (d & 1)
        load16_to_lds_s(rv, off, v_lds0 + lvs * STAGE_BYTES + 1024u * i);
      else
        load16_to_lds_s(rk, off, k_lds0 + lks * STAGE_BYTES + 1024u * i);
    };
    // (one per MFMA, from the first, when there are more loads than half the
    // score MFMAs)
    auto dma_slot = [](int d) constexpr { return 2 * NDMA <= MA ? 2 * d + 1 : d; };
    static_assert(NDMA <= MA, "direct loads must fit between the score MFMAs");
    // ---- phase A ----
    u32x4 kop[RPD + 1];
#pragma unroll
    for (int st = 0; st < RPD && st < NSA; ++st) kop[st] = read_k(kl, st);
    // The first operand's LDS latency is covered by the first exponentials,
    // which need no operand; the fence keeps the reads in step order.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UA_PRE; ++u) a_unit(u);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 vop[RPD + 1];
    // The finish of the previous tile runs after score MFMA FIN, so that the
    // last score MFMAs (which it does not depend on) cover its vector work
    // and branch, and the first V operands of phase B are read in the last
    // RPD slots: the product phase then starts without waiting.
    // (with fewer than 8 score MFMAs, after the first half of them)
    constexpr int FIN = MA >= 8 ? MA - 4 : MA / 2;
    static_assert(FIN >= 1 || UA <= UA_PRE, "weight units need score MFMAs before the finish");
#pragma unroll
    for (int st = 0; st < NSA; ++st) {
      if (st + RPD < NSA) kop[(st + RPD) % (RPD + 1)] = read_k(kl, st + RPD);
      const int ks = st / NKB, kb = st % NKB;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int mi = st * NH + h;
        sacc[h][kb] = Ty::mfma(kop[st % (RPD + 1)], qreg[h][ks], ks == 0 ? f32x16{} : sacc[h][kb]);
        if (mi < FIN) {
#pragma unroll
          for (int u = UA_PRE + mi * (UA - UA_PRE) / FIN; u < UA_PRE + (mi + 1) * (UA - UA_PRE) / FIN; ++u)
            a_unit(u);
        }
        if (mi == FIN) {
          a_unit_last();
          a_finish(first, fresh);
        }
        if (mi >= MA - RPD) vop[mi - (MA - RPD)] = read_v(vl, mi - (MA - RPD));
#pragma unroll
        for (int d = 0; d < NDMA; ++d)
          if (dma_slot(d) == mi) dma(d);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (FIN >= MA) {
      a_unit_last();
      a_finish(first, fresh);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- phase B ----
    if (masked) apply_mask(k0);  // per-wave scalar branch at a fence point
    sums_start();
#pragma unroll
    for (int st = 0; st < NSB; ++st) {
      if (st + RPD < NSB) vop[(st + RPD) % (RPD + 1)] = read_v(vl, st + RPD);
      const int kk = st / NDB, db = st % NDB;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int mi = st * NH + h;
        oacc[h][db] = Ty::mfma(vop[st % (RPD + 1)], pk[h][kk], oacc[h][db]);
        if (mi < MB / 2) {
#pragma unroll
          for (int u = mi * UB / (MB / 2); u < (mi + 1) * UB / (MB / 2); ++u) b_unit(u);
        } else {
          const int q = mi - MB / 2;
#pragma unroll
          for (int r = q * UAB / (MB / 2); r < (q + 1) * UAB / (MB / 2); ++r) {
            w_exp(r);
            if (r > 0) w_fin(r - 1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (UAB > 0) w_fin(UAB - 1);
  };

  // Zero the V stage that the first tile's (empty) pending product reads, so
  // that its zero weights never meet uninitialised LDS.
  for (int i = tid; i < NK * TILE_CHUNKS; i += NW * 64)
    v_lds[i / TILE_CHUNKS][NVST - 1][i % TILE_CHUNKS] = u32x4{};
  // Prefetches past the last tile read an index beyond the sequence: the
  // buffer range check turns them into zero fills of a free stage, so every
  // tile issues the same number of loads and the waits below are constants
  // (no branch splits the loop body).  Key group g's step `it` is tile
  // kt_begin + g + NK * it.
  const int kt_none = ntk + PF * NK;
  auto tile_of = [&](int it) { return kt_begin + kg + NK * it; };
  auto tile_or_none = [&](int kt) { return kt < kt_end ? kt : kt_none; };
#pragma unroll
  for (int i = 0; i < PF; ++i) load_tile(tile_or_none(tile_of(i)), i, i);
  __builtin_amdgcn_sched_barrier(0);  // nothing that waits for Q before these loads
  // Wait for the first tile only (and the zero fill); the later prefetches
  // stay in flight.
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LOADS_PER_TILE * (PF - 1)) : "memory");
  __builtin_amdgcn_s_barrier();
  // Kernel arguments arrive through scalar loads, which share the counter
  // of LDS reads.  Using every argument-derived value the loops or the
  // epilogue read (buffer descriptors, output pointers) once here settles
  // the compiler's bookkeeping of those loads before the loops: a scalar load
  // still pending at a loop entry, or feeding an inline-assembly operand in
  // a loop, makes it wait for lgkmcnt(0), which also drains the LDS operand
  // reads that run ahead of the MFMAs.
  asm volatile("" ::"s"(rk), "s"(rv), "s"(a.o), "s"(a.lse));
  // The sign flip, then Q into accumulation registers: Q never meets the
  // vector ALU again, and MFMA reads its A/B operands from AGPRs too, which
  // leaves the VGPRs to the softmax.  Both wait for the Q loads, so they come
  // after the first tiles' loads are issued (the fence above keeps them
  // there): Q and those tiles are then fetched in one round trip.
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qreg[h][ks] ^= qflip;
      asm volatile("" : "+a"(qreg[h][ks]));
    }

  // The work-group's steps run in groups of NST, each copy of the tile with
  // its own compile-time stage phase; the loop leaves at the first step past
  // the last one (a scalar branch per step).  Every key group takes the same
  // number of steps (the largest group's share, so the barriers match), a
  // group with fewer tiles finishing with one past its last visible one: its
  // loads read the out-of-range index (zero fill) and all its scores are
  // masked, so it contributes weight 0 and factor 1.
  //
  // Every wave of a key group runs every tile of that group (the loads are
  // shared within the group; every wave takes the same number of steps).
  // A wave masks a tile
  // elementwise when the tile straddles an edge of its rows' band or lies
  // outside it; a tile outside the band is simply fully masked (weights 0,
  // factor 1).
  const int n_steps = (kt_end - kt_begin + NK - 1) / NK;
  // Under a window, whether tile kt (of this wave's key group) can hold the
  // first key of some row of this wave that the group sees: rows wr0..wr1
  // first see keys wr0 - W + 1 .. wr1 - W + 1, and a key group's first tile
  // at or after such a key starts at most NK - 1 tiles after the tile that
  // holds it.
  auto fresh_window = [&](int kt) __attribute__((always_inline)) {
    if (MASK != kMaskWindow) return false;
    const int k0 = kt * BC;
    return k0 + BC - 1 >= wr0 - a.window + 1 && k0 <= wr1 - a.window + 1 + (NK - 1) * BC;
  };
  auto need_mask = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BC;
    if (kt >= kt_end) return true;
    if (MASK == kMaskCausal) return k0 + BC - 1 > wr0;
    if (MASK == kMaskWindow) return k0 + BC - 1 > wr0 || k0 <= wr1 - a.window;
    return k0 + BC > S;
  };
  // One tile and the end-of-tile synchronisation.  Tile kt+1 has landed
  // (this wave's share) once at most PF-1 tiles' loads are outstanding; the
  // barrier extends that to the whole work-group.  Every LDS read of this
  // tile was consumed by an MFMA above, so after the barrier the stages read
  // here may be overwritten.
  // Steps 0 .. it_hi hold the tiles this wave can see any key of.  Under a
  // causal or window mask the tiles after it (keys past the wave's last row)
  // it only loads for (its share of the work-group's tiles) and synchronises
  // on: no MFMA, no softmax.  Every wave still takes n_steps steps, so the
  // barriers match.  Under a key split every wave runs every step.
  int it_hi = n_steps - 1;
  if (NK == 1 && MASK != kMaskNone) it_hi = min(it_hi, min(wr1, S - 1) / BC - kt_begin);
  auto sync = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS_PER_TILE * (PF - 1)) : "memory");
    __builtin_amdgcn_s_barrier();
  };
  auto step = [&](auto phase_c, int it) __attribute__((always_inline)) {
    const int kt = tile_of(it);
    // (the finish in step `it` is that of tile_of(it - 1), none in step 0;
    // the first tile's always takes the offset update)
    tile(need_mask(kt), it == 1, it > 0 && fresh_window(tile_of(it - 1)), phase_c, kt * BC,
         tile_or_none(tile_of(it + PF)));
    sync();
  };
  auto step_if = [&](auto phase_c, int it) __attribute__((always_inline)) {
    if (it <= it_hi) step(phase_c, it);
  };
  for (int it = 0; it <= it_hi; it += NST) unroll_steps<0, NST>(step_if, it);
  // The last visible tile: its remaining weights, then its PV products (its
  // V stage is that of step it_hi).
  if (it_hi >= 0) {
#pragma unroll
    for (int u = 0; u < UA; ++u) a_unit(u);
    a_unit_last();
    a_finish(it_hi == 0, fresh_window(tile_of(it_hi)));
    o_phase(it_hi % NST);
  }
  // The rest of the work-group's steps: loads and synchronisation only.
  for (int it = it_hi + 1; it < n_steps; ++it) {
    const int st = (it + PF) % NST;
    load_tile(tile_or_none(tile_of(it + PF)), st, st);
    sync();
  }
  // Zero-fill loads issued past the last tile may still be writing LDS.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Row statistics of the rows this wave holds: offset m (base 2) and the
  // full denominators (both lanes of a row).
  float l_tot[NH], lt_tot[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    l_tot[h] = l[h] + wave_partner(l[h]);
    lt_tot[h] = NK > 1 ? lt[h] + wave_partner(lt[h]) : l_tot[h];
  }

  if constexpr (NK > 1) {
    // Merge of the key groups' partial results: m = max m_g,
    // l = sum l_g 2^(m_g - m), O = sum O_g 2^(m_g - m) (a group that saw no
    // visible key of a row has m_g = -inf and factor 0).  The work is shared
    // out by accumulator block: block b = h * NDB + db of a row group is
    // merged, normalised and stored by key group b % NK, which reads the
    // other groups' partials of that block from LDS.  Every wave writes the
    // blocks it hands on and its row statistics, then all waves merge at once.
    // The stages are reused for the partials (accumulators in the K stages,
    // row statistics in the V stages) once every wave is done with them (the
    // zero-fill loads past the last tile have landed: see the wait above).
    // The partials are stored in the register layout (16 bytes per lane,
    // consecutive lanes), so the stores and reads are conflict-free.  The
    // terms are summed in key-group order whichever group merges, so the
    // result does not depend on which wave does it.
    constexpr int NBLK = NH * NDB;      // accumulator blocks per wave
    // With fewer blocks than key groups, groups NBLK.. merge nothing and
    // every block has a slot of its own per writer; otherwise a group writes
    // only the other groups' blocks, packed.
    constexpr bool SPARSE = NBLK % NK != 0;
    constexpr int NOUT = SPARSE ? NBLK : NBLK - NBLK / NK;  // slots per writing wave
    static_assert(!SPARSE || NBLK < NK, "blocks must split evenly over the key groups");
    static_assert(NW * NOUT * 4096 <= (int)sizeof(k_lds), "merge space (accumulators)");
    static_assert(NW * NH * 1024 <= (int)sizeof(v_lds), "merge space (statistics)");
    char *mbuf = (char *)&k_lds[0][0][0];
    char *sbuf = (char *)&v_lds[0][0][0];
    // byte offset of block b as written by key group g of this row group
    // (a group writes the blocks of the other groups, in block order)
    auto slot = [&](int g, int b) __attribute__((always_inline)) {
      const int j = SPARSE ? b : (b / NK) * (NK - 1) + (b % NK) - (b % NK > g ? 1 : 0);
      return ((g * NR + rg) * NOUT + j) * 4096;
    };
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int bl = h * NDB + db;
        if (bl % NK == kg) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16 &o = oacc[h][db];
          *(f32x4 *)(mbuf + slot(kg, bl) + (j * 64 + lane) * 16) =
              f32x4{o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
        }
      }
      *(f32x4 *)(sbuf + (((kg * NR + rg) * NH + h) * 64 + lane) * 16) =
          f32x4{m[h], l_tot[h], lt_tot[h], 0.f};
    }
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float mg[NK], lgs[NK], ltg[NK];
      float mm = -INFINITY;
#pragma unroll
      for (int g = 0; g < NK; ++g) {
        const f32x4 ml = *(const f32x4 *)(sbuf + (((g * NR + rg) * NH + h) * 64 + lane) * 16);
        mg[g] = ml[0];
        lgs[g] = ml[1];
        ltg[g] = ml[2];
        mm = fmaxf(mm, mg[g]);
      }
      float f[NK], lsum = 0.f, ltsum = 0.f;
#pragma unroll
      for (int g = 0; g < NK; ++g) {
        f[g] = mg[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg[g] - mm);
        lsum = fmaf(f[g], lgs[g], lsum);
        ltsum = fmaf(f[g], ltg[g], ltsum);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int bl = h * NDB + db;
        if (bl % NK != kg) continue;
        f32x16 acc;
#pragma unroll
        for (int g = 0; g < NK; ++g) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4 o;
            if (g == kg)
              o = f32x4{oacc[h][db][4 * j], oacc[h][db][4 * j + 1], oacc[h][db][4 * j + 2],
                        oacc[h][db][4 * j + 3]};
            else
              o = *(const f32x4 *)(mbuf + slot(g, bl) + (j * 64 + lane) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[4 * j + e] = g == 0 ? o[e] * f[0] : fmaf(f[g], o[e], acc[4 * j + e]);
          }
        }
        oacc[h][db] = acc;
      }
      m[h] = mm;
      l_tot[h] = lsum;
      lt_tot[h] = ltsum;
    }
  }

  // Epilogue: one division per row, RNE to the element type, natural-log LSE
  // (under a key split, each key group stores the blocks it merged, and the
  // group holding a half's first block its LSE).
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int row = wr0 + 32 * h + lq;
    if (row < S) {
      const float inv = 1.f / lt_tot[h];
      uint16_t *orow = (uint16_t *)a.o + head_off + (size_t)row * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if (NK > 1 && (h * NDB + db) % NK != kg) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 w;
          w[0] = Ty::pack2(oacc[h][db][4 * j + 0] * inv, oacc[h][db][4 * j + 1] * inv);
          w[1] = Ty::pack2(oacc[h][db][4 * j + 2] * inv, oacc[h][db][4 * j + 3] * inv);
          *(u32x2 *)(orow + 32 * db + 8 * j + 4 * lg) = w;
        }
      }
      if (lg == 0 && (NK == 1 || (h * NDB) % NK == kg))
        a.lse[(size_t)bh * S + row] =
            (m[h] + __builtin_amdgcn_logf(l_tot[h])) * 0.69314718055994531f;
    }
  }
}

// One kernel instance: NW waves per work-group as NK key groups of NR = NW/NK
// row groups.  NK = 1 is the plain decomposition (one work-group per 256
// query rows at d <= 128); NK > 1 splits each work-group's key tiles over
// the key groups, for grids too small to fill the chip.
template <class Ty, int D, int MASK, int NK>
struct Instance {
  // Key splits (d <= 128): 8 waves of 32 rows, two per SIMD (169 registers
  // at d = 64, about 200 at d = 128), so that a step's softmax work is split
  // over twice the waves.  The d = 128 sliding window: 2 waves of 64 rows,
  // two work-groups per compute unit, so that a barrier couples only the two
  // waves of a 128-row band (their band edges, and so their masked tiles,
  // fall on different steps) and a work-group's band holds 2 tiles more than
  // a wave's instead of 6.  Everything else: 4 waves, one per SIMD.
  static constexpr int NW = (D <= 128 && NK > 1) ? 8
                            : (D == 128 && MASK == kMaskWindow) ? 2 : 4;
  static constexpr int BC = NK > 1 ? 32 : D == 64 ? 64 : 32;  // keys per tile
  static constexpr int NH = (D <= 128 && NK > 1) ? 1 : D <= 128 ? 2 : 1;
  static constexpr int PF = 2;
  static constexpr int BR = 32 * NH * (NW / NK);
  static bool run(const FwdArgs *a, hipStream_t stream, bool launch, LaunchInfo *info,
                  hipError_t *err) {
    static char name[96];
    static const char *mk[3] = {"none", "causal", "window"};
    if (NK > 1)
      snprintf(name, sizeof(name), "fa_fwd_mfma<%s,d%d,%s,br%d,bc%d,pf%d,keysplit%d>",
               Ty::kName, D, mk[MASK], BR, BC, PF, NK);
    else
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
    *err = hipLaunchKernel((const void *)&fa_fwd_mfma_kernel<Ty, D, MASK, NW, NK, BC, NH, PF>,
                           grid, block, kargs, 0, stream);
    return true;
  }
};

// Key groups for a launch of these sizes: 1 unless the plain grid has fewer
// work-groups than the chip has compute units (256), in which case the keys
// are split 4 ways at d = 64 (64-row work-groups) and 2 ways at d = 128
// (128-row work-groups), within the 128 KB of LDS the split stages need.
constexpr int kComputeUnits = 256;
template <int D>
int key_groups(const FwdArgs *a) {
  if (!a || D > 128) return 1;
  const int64_t plain = (int64_t)((a->S + 255) / 256) * a->B * a->H;
  if (plain >= kComputeUnits) return 1;
  return D == 64 ? 4 : 2;
}

template <class Ty, int D, int MASK>
bool by_split(const FwdArgs *a, hipStream_t s, bool launch, LaunchInfo *info, hipError_t *err) {
  if constexpr (D <= 128) {
    if (key_groups<D>(a) > 1)
      return Instance<Ty, D, MASK, D == 64 ? 4 : 2>::run(a, s, launch, info, err);
  }
  return Instance<Ty, D, MASK, 1>::run(a, s, launch, info, err);
}

template <class Ty, int D>
bool by_mask(int mask, const FwdArgs *a, hipStream_t s, bool launch, LaunchInfo *info,
             hipError_t *err) {
  switch (mask) {
    case kMaskNone: return by_split<Ty, D, kMaskNone>(a, s, launch, info, err);
    case kMaskCausal: return by_split<Ty, D, kMaskCausal>(a, s, launch, info, err);
    case kMaskWindow: return by_split<Ty, D, kMaskWindow>(a, s, launch, info, err);
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
