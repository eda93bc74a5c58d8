// Backward pass of exact attention on gfx950: gradients dQ, dK, dV from Q, K,
// V, the forward output O, its logsumexp and the output gradient dO.
//
// The method is the one in "FlashAttention: Why Tiling Attention Makes
// Transformers Fast Without Changing the Result" (Dev.to), section "The
// backward pass: recompute instead of storing": nothing of size S x S is
// stored; every score block is recomputed on chip from Q and K, its
// probabilities are rebuilt from the stored row statistic (P = exp(scale *
// q.k - LSE), exact because LSE is the final normaliser), and
//   dV = P^T dO,   dP = dO V^T,
//   dS = P * (dP - D) with D[i] = dO_i . O_i  (the softmax Jacobian's row
//        term: sum_j P_ij dP_ij = dO_i . (sum_j P_ij V_j) = dO_i . O_i),
//   dQ = scale * dS K,   dK = scale * dS^T Q
// are accumulated tile by tile.
//
// Three launches, all deterministic (no atomics):
//   * row terms: D[i] = dO_i . O_i into a caller-provided fp32 buffer;
//   * dK/dV: one work-group per 128 keys of one key/value head; each wave
//     owns 32 keys, keeps their K and V rows in registers as MFMA operands
//     and streams the query tiles (Q, dO, LSE, D through LDS) of every query
//     head that reads this key/value head;
//   * dQ: one work-group per 128 query rows; each wave owns 32 rows, keeps
//     their Q and dO rows in registers and streams K/V tiles through LDS, as
//     the forward kernel does.
// The MFMA layouts are the forward kernel's: score blocks come out of
// v_mfma_f32_32x32x16 so that each lane holds 16 entries of one column, the
// accumulator of P (or dS) is directly the operand of the next product once
// packed, and the transposed operands (dO^T, Q^T, K^T) are read with
// ds_read_b64_tr_b16 from row-major LDS tiles under the same 64-bank swizzle.
#include "fa_tile_ops.h"

#include <math.h>
#include <stdio.h>

namespace fa {
namespace {

using namespace tile;

constexpr float LOG2E = 1.4426950408889634f;

// Direct loads of a [32 rows][D] tile (rows row0.., of one head's slab) into
// an LDS tile, this wave's share: chunk position p of the tile holds row
// p / KCH, logical chunk c with swz(row, c) == p % KCH.
template <int D, int NW>
__device__ inline void load_rows_tile(u32x4 rsrc, int row0, u32x4 *lds_tile, int wave,
                                      int lane) {
  constexpr int KCH = D / 8, CHUNKS = 32 * KCH, LPW = CHUNKS / 64 / NW;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int blk = wave * LPW + i;
    const int pos = 64 * blk + lane;
    const int r = pos / KCH, cc = swz<D>(r, pos % KCH);
    load16_to_lds(rsrc, (uint32_t)((row0 + r) * D + 8 * cc) * 2u,
                  (uint32_t)(uintptr_t)&lds_tile[64 * blk]);
  }
}

// Store a transposed accumulator (lane: one column index `col` of the
// output rows, registers: d values 32*db + 8*(r/4) + 4*lg + (r%4), NB
// blocks) as 32*NB values of the row `col` of a row-major slab, starting at
// row_ptr, RNE to the element type.
template <class Ty, int NB>
__device__ inline void store_rowmajor(uint16_t *row_ptr, const f32x16 (&acc)[NB], float mul,
                                      int lg) {
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 w;
      w[0] = Ty::pack2(acc[db][4 * j + 0] * mul, acc[db][4 * j + 1] * mul);
      w[1] = Ty::pack2(acc[db][4 * j + 2] * mul, acc[db][4 * j + 3] * mul);
      *(u32x2 *)(row_ptr + 32 * db + 8 * j + 4 * lg) = w;
    }
}

// ---------------------------------------------------------------------------
// Row terms: D[i] = sum_t dO[i, t] * O[i, t] (fp32), D/8 lanes per row.
template <class Ty, int D>
__global__ __launch_bounds__(256) void fa_bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int64_t rows = (int64_t)a.B * a.H * a.S;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int c = tid % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = *(const u32x4 *)((const uint16_t *)a.o + row * D + 8 * c);
    const u32x4 g = *(const u32x4 *)((const uint16_t *)a.dout + row * D + 8 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2 ov = Ty::unpack2(o[j]), gv = Ty::unpack2(g[j]);
      acc = fmaf(ov[0], gv[0], fmaf(ov[1], gv[1], acc));
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK and dV: one work-group per 32*NW keys of one key/value head and
// 1/DSPLIT of the head dimension.  With DSPLIT = 2 (d = 256, where whole-d
// accumulators do not fit beside the K and V operands) the two work-groups of
// a key tile both compute S and dP over the whole d and each accumulates dK
// and dV for its half of the columns: 1.5 times the matrix work of whole-d
// accumulation, and the same query stream read twice (the two work-groups
// are adjacent in launch order, so the second read mostly hits L2).
//
// Software pipeline over the query tiles u of the work-group's stream (one
// wave, 32 keys; the same for every wave):
//   phase 1 of step u: S(u) = Q_u K^T and dP(u) = dO_u V^T on the matrix
//     core, with the vector work of tile u-1 beside them: dS(u-1) =
//     P(u-1) * (dP(u-1) - D) and its packing;
//   phase 2 of step u: dV += dO_{u-1}^T P(u-1) and dK += Q_{u-1}^T dS(u-1),
//     with the weights of tile u beside them: P(u) = exp2(c S(u) - LSE log2 e)
//     and their packing.
// Each phase is a fixed sequence of steps (operand read RPD steps ahead, one
// MFMA, its share of the vector work) separated by scheduling fences, so
// the matrix core runs while the wave issues the vector work.  Query tiles
// stream through NST = 4 LDS stages, loaded PF = 2 tiles ahead; the step
// loop is unrolled over the 4 stage phases so every LDS offset and register
// buffer choice is a compile-time constant.  Tiles past the end of the
// stream read out of range (zero fill) and contribute nothing: with Q and
// dO zero, dP, D and dO^T P all vanish.
template <class Ty, int D, int MASK, int NW, int DSPLIT>
__global__ __launch_bounds__(NW * 64, 1) void fa_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BKV = 32 * NW;  // keys per work-group
  constexpr int BQ = 32;        // query rows per streamed tile
  constexpr int NKS = D / 16, NDB = D / 32 / DSPLIT, KCH = D / 8;  // NDB: d blocks owned
  constexpr int TILE_CHUNKS = BQ * KCH;
  constexpr int LPW = TILE_CHUNKS / 64 / NW;       // 16-byte loads per wave per tile and tensor
  constexpr int LOADS = 2 * LPW + 1;               // per wave per tile (Q, dO, one statistic)
  constexpr int NST = 4, PF = 2, RPD = 3;
  constexpr int NS1 = 2 * NKS;                     // phase-1 MFMAs (S and dP)
  constexpr int NS2 = 4 * NDB;                     // phase-2 MFMAs (dV and dK, 2 key halves)
  static_assert(TILE_CHUNKS % (64 * NW) == 0, "tile must split evenly over the waves");
  static_assert(NW == 4, "one statistic load per wave: lse, D and two spares");
  __shared__ u32x4 q_lds[NST][TILE_CHUNKS];
  __shared__ u32x4 do_lds[NST][TILE_CHUNKS];
  __shared__ float stat_lds[NST][4][64];           // [stage][lse, D, spare, spare][row]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, lg = lane >> 5;
  const int S = a.S, H = a.H, Hkv = a.Hkv, group = H / Hkv;
  const int n_kv = a.B * Hkv;
  const int kvi = blockIdx.x % n_kv;  // key/value head (b * Hkv + hk)
  const int kt = blockIdx.x / n_kv / DSPLIT;  // key tile; the first ones see the most rows
  const int dh = (blockIdx.x / n_kv) % DSPLIT;  // part of d owned: columns 32*NDB*dh ...
  const int b = kvi / Hkv, hk = kvi - b * Hkv;
  const int k0 = kt * BKV, kw0 = k0 + 32 * wave;
  const float c = a.scale_log2;

  const size_t kv_off = (size_t)kvi * (size_t)S * D;
  const uint32_t head_bytes = (uint32_t)S * D * 2u;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t *)a.k + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t *)a.v + kv_off, head_bytes);
  // This wave's keys as the B operand of S = Q K^T and dP = dO V^T: lane
  // (key kw0 + lq, group lg) holds row chunk 2*ks + lg of K and V.
  u32x4 kreg[NKS], vreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const uint32_t off = (uint32_t)((kw0 + lq) * D + 16 * ks + 8 * lg) * 2u;
    kreg[ks] = load16(rk, off);
    vreg[ks] = load16(rv, off);
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+a"(kreg[ks]), "+a"(vreg[ks]));

  // Query tiles that can see a key of this work-group.
  const int nqt_all = (S + BQ - 1) / BQ;
  int qt_begin = 0, qt_end = nqt_all;
  if (MASK != kMaskNone) qt_begin = k0 / BQ;  // rows i >= key
  if (MASK == kMaskWindow) {
    const int last_row = min(S - 1, k0 + BKV - 1 + a.window - 1);  // i < key + window
    qt_end = min(qt_end, last_row / BQ + 1);
  }
  const int nq = max(qt_end - qt_begin, 0);
  const int total = group * nq;  // (query head of the group, query tile) pairs

  TileOffsets<D> off(lane);
  // transposed operands address this work-group's columns 32*NDB*dh ...
  // (a multiple of 128 columns: the swizzle permutes only the low 16 chunks)
  if (DSPLIT > 1) {
#pragma unroll
    for (int j = 0; j < TileOffsets<D>::NVB; ++j) off.tr_base[j] += 64 * NDB * dh;
  }
  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dkacc[i] = dvacc[i] = f32x16{};

  // Stream cursors (wave-uniform scalars, no division): the member j of the
  // query-head group and the query tile qt of the tile being loaded and of
  // the tile being finished.  j == group means past the end: a row beyond
  // the sequence, whose loads zero-fill.
  struct Cursor {
    int j, qt;
  };
  auto advance = [&](Cursor &c) __attribute__((always_inline)) {
    const bool wrap = c.qt + 1 == qt_end;
    c.qt = wrap ? qt_begin : c.qt + 1;
    c.j += wrap ? 1 : 0;
  };
  auto row0_of = [&](const Cursor &c) __attribute__((always_inline)) {
    return c.j < group ? c.qt * BQ : S + BQ;
  };
  Cursor ld{0, qt_begin}, fin{0, qt_begin};
  // Sources of the tile under the load cursor, set once per tile.
  struct Src {
    u32x4 q, dout, stat;
    int row0;
  } src;
  auto set_src = [&]() __attribute__((always_inline)) {
    const int bh = b * H + hk * group + (ld.j < group ? ld.j : 0);
    const size_t q_off = (size_t)bh * (size_t)S * D;
    src.q = rsrc_words((const uint16_t *)a.q + q_off, head_bytes);
    src.dout = rsrc_words((const uint16_t *)a.dout + q_off, head_bytes);
    const float *st = wave == 1 ? a.delta : a.lse;  // waves 2, 3: spare copies
    src.stat = rsrc_words(st + (size_t)bh * S, (uint32_t)S * 4u);
    src.row0 = row0_of(ld);
  };
  // Direct load d (of this wave's LOADS per tile) of the tile under the load
  // cursor, into stage st.
  auto dma = [&](int st, int d) __attribute__((always_inline)) {
    if (d < 2 * LPW) {
      const int i = d % LPW;
      const int blk = wave * LPW + i;
      const int pos = 64 * blk + lane;
      const int r = pos / KCH, cc = swz<D>(r, pos % KCH);
      const uint32_t o = (uint32_t)((src.row0 + r) * D + 8 * cc) * 2u;
      if (d < LPW)
        load16_to_lds(src.q, o, (uint32_t)(uintptr_t)&q_lds[st][64 * blk]);
      else
        load16_to_lds(src.dout, o, (uint32_t)(uintptr_t)&do_lds[st][64 * blk]);
    } else {
      load4_to_lds(src.stat, (uint32_t)(src.row0 + lane) * 4u,
                   (uint32_t)(uintptr_t)&stat_lds[st][wave][0]);
    }
  };

  // Pipeline registers.  Scores of the current tile; dP of the current and
  // previous tile (by parity); fp32 weights of the newest tile; packed
  // weights by parity; packed dS of the previous tile.
  f32x16 sacc;
  f32x16 dpacc[2];
  float pw[16];
  u32x4 ppk[2][2], dspk[2];
  dpacc[0] = dpacc[1] = f32x16{};

  // The finished tile's rows: row0 + 8*(r/4) + 4*lg + (r%4) for
  // accumulator register r.
  auto edge_of = [&](int row0) __attribute__((always_inline)) {
    if (MASK == kMaskNone) return false;
    bool e = row0 < kw0 + 31;
    if (MASK == kMaskWindow) e = e || row0 + BQ - 1 > kw0 - 1 + a.window;
    return e;
  };
  auto fix_mask = [&](int row0, u32x4 (&pk)[2]) __attribute__((always_inline)) {
    // row = row0 + 4*lg + off(r): key <= row is off(r) >= t, and under a
    // window key > row - window is off(r) < t + window (one per-lane bound,
    // compile-time offsets)
    const int t = kw0 + lq - row0 - 4 * lg;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 8 * (r >> 2) + (r & 3);
      bool vis = off >= t;
      if (MASK == kMaskWindow) vis = vis && off < t + a.window;
      if (!vis) pw[r] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j) pk[kk][j] = Ty::pack2(pw[8 * kk + 2 * j], pw[8 * kk + 2 * j + 1]);
  };

  // One pipeline step u with stage phase P (= u % NST).  HAS_PREV: tile u-1
  // exists (dS, dV, dK work); HAS_CUR: tile u exists (S, dP, weights).
  auto step = [&](auto phase_c, auto has_prev_c, auto has_cur_c, int u)
                  __attribute__((always_inline)) {
    constexpr int P = decltype(phase_c)::value;
    constexpr bool HAS_PREV = decltype(has_prev_c)::value, HAS_CUR = decltype(has_cur_c)::value;
    constexpr int par = P & 1;
    constexpr int cur = P, prev = (P + NST - 1) % NST, ldst = (P + PF) % NST;
    const char *qc = (const char *)&q_lds[cur][0];
    const char *dc = (const char *)&do_lds[cur][0];
    const char *qp = (const char *)&q_lds[prev][0];
    const char *dp = (const char *)&do_lds[prev][0];
    set_src();
    // ---- phase 1: S(u), dP(u) | dS(u-1) ----
    // Row terms D of tile u-1, four at a time; at d = 256 each group is read
    // a few steps before its first use rather than all up front, which keeps
    // the registers within the file.
    float dl[16];
    auto load_dl = [&](int q4) __attribute__((always_inline)) {
      const float4 d4 = *(const float4 *)&stat_lds[prev][1][8 * q4 + 4 * lg];
      dl[4 * q4 + 0] = d4.x;
      dl[4 * q4 + 1] = d4.y;
      dl[4 * q4 + 2] = d4.z;
      dl[4 * q4 + 3] = d4.w;
    };
    constexpr bool LATE_DL = D == 256;
    // first phase-1 step that uses group q4, and the step that reads it
    auto dl_use = [](int q4) constexpr { return ((4 * q4 + 1) * NS1 + 15) / 16 - 1; };
    auto dl_read = [&](int q4) constexpr { return dl_use(q4) > 4 ? dl_use(q4) - 4 : 0; };
    if (HAS_PREV && !LATE_DL) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) load_dl(q4);
    }
    u32x4 rop[RPD + 1];
    auto read_row = [&](int st) __attribute__((always_inline)) {
      return off.row_op((st & 1) ? dc : qc, st >> 1);
    };
    if (HAS_CUR) {
#pragma unroll
      for (int st = 0; st < RPD; ++st) rop[st] = read_row(st);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NS1; ++st) {
      if (HAS_CUR) {
        if (st + RPD < NS1) rop[(st + RPD) % (RPD + 1)] = read_row(st + RPD);
        const int ks = st >> 1;
        if (st & 1)
          dpacc[par] = Ty::mfma(rop[st % (RPD + 1)], vreg[ks], ks == 0 ? f32x16{} : dpacc[par]);
        else
          sacc = Ty::mfma(rop[st % (RPD + 1)], kreg[ks], ks == 0 ? f32x16{} : sacc);
      }
      // direct loads of tile u+PF, spread over the phase
#pragma unroll
      for (int d = 0; d < LOADS; ++d)
        if ((d * NS1) / LOADS == st) dma(ldst, d);
      if (HAS_PREV && LATE_DL) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          if (dl_read(q4) == st) load_dl(q4);
      }
      if (HAS_PREV) {
#pragma unroll
        for (int r = st * 16 / NS1; r < (st + 1) * 16 / NS1; ++r) {
          const float v = pw[r] * (dpacc[par ^ 1][r] - dl[r]);
          pw[r] = v;  // pw now holds dS(u-1)
          if (r & 1) {
            dspk[r >> 3][(r & 7) >> 1] = Ty::pack2(pw[r - 1], v);
            pin(dspk[r >> 3][(r & 7) >> 1]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- phase 2: dV, dK of tile u-1 | weights of tile u ----
    float lv[16];
    if (HAS_CUR) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 l4 = *(const float4 *)&stat_lds[cur][0][8 * q4 + 4 * lg];
        lv[4 * q4 + 0] = l4.x * LOG2E;
        lv[4 * q4 + 1] = l4.y * LOG2E;
        lv[4 * q4 + 2] = l4.z * LOG2E;
        lv[4 * q4 + 3] = l4.w * LOG2E;
      }
    }
    // step st: key half kk = st / (2*NDB), d block db = (st / 2) % NDB,
    // dV (even st) or dK (odd st)
    u32x4 top[RPD + 1];
    auto read_tr = [&](int st) __attribute__((always_inline)) {
      const int kk = st / (2 * NDB), db = (st >> 1) % NDB;
      return off.tr_op((st & 1) ? qp : dp, kk, db);
    };
    if (HAS_PREV) {
#pragma unroll
      for (int st = 0; st < RPD; ++st) top[st] = read_tr(st);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NS2; ++st) {
      if (HAS_PREV) {
        if (st + RPD < NS2) top[(st + RPD) % (RPD + 1)] = read_tr(st + RPD);
        const int kk = st / (2 * NDB), db = (st >> 1) % NDB;
        if (st & 1)
          dkacc[db] = Ty::mfma(top[st % (RPD + 1)], dspk[kk], dkacc[db]);
        else
          dvacc[db] = Ty::mfma(top[st % (RPD + 1)], ppk[par ^ 1][kk], dvacc[db]);
      }
      if (HAS_CUR) {
#pragma unroll
        for (int r = st * 16 / NS2; r < (st + 1) * 16 / NS2; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, -lv[r]));
          pw[r] = p;
          if (r & 1) {
            ppk[par][r >> 3][(r & 7) >> 1] = Ty::pack2(pw[r - 1], p);
            pin(ppk[par][r >> 3][(r & 7) >> 1]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    advance(ld);
    if (HAS_CUR) {
      if (MASK != kMaskNone) {
        const int row0 = row0_of(fin);
        if (edge_of(row0)) fix_mask(row0, ppk[par]);
      }
      advance(fin);
    }
    (void)u;
    // Tile u+1 has landed once only tile u+PF's loads are outstanding.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS * (PF - 1)) : "memory");
    __builtin_amdgcn_s_barrier();
  };

  // Settle the bookkeeping of the kernel-argument scalar loads before the
  // loop (see the forward kernel).
  asm volatile("" ::"s"(a.q), "s"(a.dout), "s"(a.lse), "s"(a.delta));
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using T = std::true_type;
  using F = std::false_type;
  if (total > 0) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      set_src();
#pragma unroll
      for (int d = 0; d < LOADS; ++d) dma(u, d);
      advance(ld);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS * (PF - 1)) : "memory");
    __builtin_amdgcn_s_barrier();
    step(I0{}, F{}, T{}, 0);
    // steps 1 .. n_main (a multiple of NST, padded with empty tiles), then
    // the last step, which only finishes tile n_main
    const int n_main = (total - 1 + NST - 1) / NST * NST;
    for (int u = 1; u <= n_main; u += NST) {
      step(I1{}, T{}, T{}, u);
      step(I2{}, T{}, T{}, u + 1);
      step(I3{}, T{}, T{}, u + 2);
      step(I0{}, T{}, T{}, u + 3);
    }
    step(I1{}, T{}, F{}, n_main + 1);
  }

  // dK = scale * dS^T Q; each lane holds this work-group's d values of key
  // kw0 + lq.
  const int key = kw0 + lq;
  if (key < S) {
    const size_t o = kv_off + (size_t)key * D + 32 * NDB * dh;
    store_rowmajor<Ty, NDB>((uint16_t *)a.dk + o, dkacc, a.scale, lg);
    store_rowmajor<Ty, NDB>((uint16_t *)a.dv + o, dvacc, 1.f, lg);
  }
}

// ---------------------------------------------------------------------------
// dQ: one work-group per 32*NW query rows of one query head.
//
// The same software pipeline as the dK/dV kernel, over the key tiles t the
// work-group visits (each wave: its 32 rows against the tile's 32 keys):
//   phase 1 of step t: first the chain S^T(t) = K_t Q^T on the matrix core,
//     with dS^T(t-1) = P(t-1) * (dP^T(t-1) - D) and its packing beside; then
//     the chain dP^T(t) = V_t dO^T, with the weights of tile t,
//     P = exp2(c S^T(t) - LSE log2 e), beside (S^T(t) is complete by then,
//     and a dependent MFMA chain issues at the full rate);
//   phase 2 of step t: dQ^T += K_{t-1}^T dS^T(t-1) on the matrix core.
// This keeps the vector work of a tile beside the 16 MFMAs of phase 1 rather
// than the 8 of phase 2.
// Keys past the sequence read as zero rows: their dS^T column is multiplied
// by a zero K row, so they need no mask; causal and window edges get a
// fix-up on the tiles that straddle them.
template <class Ty, int D, int MASK, int NW>
__global__ __launch_bounds__(NW * 64, 1) void fa_bwd_dq_kernel(BwdArgs a) {
  constexpr int BR = 32 * NW;  // query rows per work-group
  constexpr int BC = 32;       // keys per streamed tile
  constexpr int NKS = D / 16, NDB = D / 32, KCH = D / 8;
  constexpr int TILE_CHUNKS = BC * KCH;
  constexpr int LPW = TILE_CHUNKS / 64 / NW;
  constexpr int LOADS = 2 * LPW;                   // K and V, per wave per tile
  constexpr int NST = 4, PF = 2, RPD = 3;
  constexpr int NS1 = 2 * NKS;                     // S^T and dP^T MFMAs
  constexpr int NS2 = 2 * NDB;                     // dQ^T MFMAs (2 key halves)
  static_assert(TILE_CHUNKS % (64 * NW) == 0, "tile must split evenly over the waves");
  __shared__ u32x4 k_lds[NST][TILE_CHUNKS];
  __shared__ u32x4 v_lds[NST][TILE_CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, lg = lane >> 5;
  const int S = a.S;
  const int BH = a.B * a.H;
  const int nqt = (S + BR - 1) / BR;
  const HeadPair hp = head_of_slot(blockIdx.x % BH, a.B, a.H, a.Hkv);
  int qt = blockIdx.x / BH;
  if (MASK != kMaskNone) qt = nqt - 1 - qt;  // heaviest query tiles first
  const int q0 = qt * BR, wr0 = q0 + 32 * wave, wr1 = wr0 + 31;
  const int row = wr0 + lq;  // this lane's query row
  const float c = a.scale_log2;

  const size_t q_off = (size_t)hp.q * (size_t)S * D, kv_off = (size_t)hp.kv * (size_t)S * D;
  const uint32_t head_bytes = (uint32_t)S * D * 2u;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t *)a.q + q_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const uint16_t *)a.dout + q_off, head_bytes);
  const u32x4 rk = rsrc_words((const uint16_t *)a.k + kv_off, head_bytes);
  const u32x4 rv = rsrc_words((const uint16_t *)a.v + kv_off, head_bytes);
  // This wave's rows as the B operand of S^T = K Q^T and dP^T = V dO^T.
  u32x4 qreg[NKS], doreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const uint32_t o = (uint32_t)(row * D + 16 * ks + 8 * lg) * 2u;
    qreg[ks] = load16(rq, o);
    doreg[ks] = load16(rdo, o);
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+a"(qreg[ks]), "+a"(doreg[ks]));
  const float lse2 = row < S ? a.lse[(size_t)hp.q * S + row] * LOG2E : 0.f;
  const float drow = row < S ? a.delta[(size_t)hp.q * S + row] : 0.f;

  // Key tiles this work-group visits (as in the forward pass).
  const int ntk = (S + BC - 1) / BC;
  int kt_begin = 0, kt_end = ntk;
  if (MASK != kMaskNone) {
    kt_end = (min(q0 + BR, S) - 1) / BC + 1;
    if (MASK == kMaskWindow) kt_begin = max(0, q0 - a.window + 1) / BC;
  }
  const int total = kt_end - kt_begin;

  const TileOffsets<D> off(lane);
  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};

  // Direct loads of stream tile u (key tile kt_begin + u; past the end an
  // out-of-range tile, zero-filled) into stage st.
  auto dma = [&](int u, int st, int d) __attribute__((always_inline)) {
    const int kt = u < total ? kt_begin + u : ntk + 1;
    const int i = d % LPW;
    const int blk = wave * LPW + i;
    const int pos = 64 * blk + lane;
    const int r = pos / KCH, cc = swz<D>(r, pos % KCH);
    const uint32_t o = (uint32_t)((kt * BC + r) * D + 8 * cc) * 2u;
    if (d < LPW)
      load16_to_lds(rk, o, (uint32_t)(uintptr_t)&k_lds[st][64 * blk]);
    else
      load16_to_lds(rv, o, (uint32_t)(uintptr_t)&v_lds[st][64 * blk]);
  };

  f32x16 sacc, dpacc[2];
  float pw[16];
  u32x4 dspk[2];
  dpacc[0] = dpacc[1] = f32x16{};

  // S^T accumulator register r of tile u holds key k0 + 8*(r/4) + 4*lg + (r%4).
  auto edge_of = [&](int u) __attribute__((always_inline)) {
    const int k0 = (kt_begin + u) * BC;
    if (MASK == kMaskCausal) return k0 + BC - 1 > wr0;
    if (MASK == kMaskWindow) return k0 + BC - 1 > wr0 || k0 <= wr1 - a.window;
    return false;
  };
  auto fix_mask = [&](int u) __attribute__((always_inline)) {
    // key = k0 + 4*lg + off(r): key <= row is off(r) <= t, and under a
    // window key > row - window is off(r) > t - window
    const int t = row - (kt_begin + u) * BC - 4 * lg;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 8 * (r >> 2) + (r & 3);
      bool vis = off <= t;
      if (MASK == kMaskWindow) vis = vis && off > t - a.window;
      if (!vis) pw[r] = 0.f;
    }
  };

  auto step = [&](auto phase_c, auto has_prev_c, auto has_cur_c, int u)
                  __attribute__((always_inline)) {
    constexpr int P = decltype(phase_c)::value;
    constexpr bool HAS_PREV = decltype(has_prev_c)::value, HAS_CUR = decltype(has_cur_c)::value;
    constexpr int par = P & 1;
    constexpr int cur = P, prev = (P + NST - 1) % NST, ld = (P + PF) % NST;
    const char *kc = (const char *)&k_lds[cur][0];
    const char *vc = (const char *)&v_lds[cur][0];
    const char *kp = (const char *)&k_lds[prev][0];
    // ---- phase 1: S^T(u) | dS^T(u-1), then dP^T(u) | weights of tile u ----
    u32x4 rop[RPD + 1];
    auto read_row = [&](int st) __attribute__((always_inline)) {
      return off.row_op(st >= NKS ? vc : kc, st % NKS);
    };
    if (HAS_CUR) {
#pragma unroll
      for (int st = 0; st < RPD; ++st) rop[st] = read_row(st);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NS1; ++st) {
      if (HAS_CUR) {
        if (st + RPD < NS1) rop[(st + RPD) % (RPD + 1)] = read_row(st + RPD);
        const int ks = st % NKS;
        if (st >= NKS)
          dpacc[par] = Ty::mfma(rop[st % (RPD + 1)], doreg[ks], ks == 0 ? f32x16{} : dpacc[par]);
        else
          sacc = Ty::mfma(rop[st % (RPD + 1)], qreg[ks], ks == 0 ? f32x16{} : sacc);
      }
#pragma unroll
      for (int d = 0; d < LOADS; ++d)
        if ((d * NS1) / LOADS == st) dma(u + PF, ld, d);
      if (HAS_PREV && st < NKS) {
#pragma unroll
        for (int r = st * 16 / NKS; r < (st + 1) * 16 / NKS; ++r) {
          const float v = pw[r] * (dpacc[par ^ 1][r] - drow);
          pw[r] = v;  // pw now holds dS^T(u-1)
          if (r & 1) {
            dspk[r >> 3][(r & 7) >> 1] = Ty::pack2(pw[r - 1], v);
            pin(dspk[r >> 3][(r & 7) >> 1]);
          }
        }
      }
      if (HAS_CUR && st >= NKS) {
        const int q = st - NKS;
#pragma unroll
        for (int r = q * 16 / NKS; r < (q + 1) * 16 / NKS; ++r) {
          pw[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, -lse2));
          pin(pw[r]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- phase 2: dQ^T of tile u-1 ----
    u32x4 top[RPD + 1];
    auto read_tr = [&](int st) __attribute__((always_inline)) {
      return off.tr_op(kp, st / NDB, st % NDB);
    };
    if (HAS_PREV) {
#pragma unroll
      for (int st = 0; st < RPD && st < NS2; ++st) top[st] = read_tr(st);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NS2; ++st) {
      if (HAS_PREV) {
        if (st + RPD < NS2) top[(st + RPD) % (RPD + 1)] = read_tr(st + RPD);
        const int kk = st / NDB, db = st % NDB;
        dqacc[db] = Ty::mfma(top[st % (RPD + 1)], dspk[kk], dqacc[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (HAS_CUR && MASK != kMaskNone) {
      if (edge_of(u)) fix_mask(u);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS * (PF - 1)) : "memory");
    __builtin_amdgcn_s_barrier();
  };

  // Settle the loads the loop reads (kernel arguments, the row's statistics)
  // before it: a compiler-tracked load still pending at a use inside the
  // loop makes it wait for vmcnt(0) there, which also drains the direct loads
  // that run ahead.
  asm volatile("" ::"s"(rk), "s"(rv), "s"(a.dq), "v"(lse2), "v"(drow));
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using T = std::true_type;
  using F = std::false_type;
  if (total > 0) {
#pragma unroll
    for (int u = 0; u < PF; ++u)
#pragma unroll
      for (int d = 0; d < LOADS; ++d) dma(u, u, d);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS * (PF - 1)) : "memory");
    __builtin_amdgcn_s_barrier();
    step(I0{}, F{}, T{}, 0);
    const int n_main = (total - 1 + NST - 1) / NST * NST;
    for (int u = 1; u <= n_main; u += NST) {
      step(I1{}, T{}, T{}, u);
      step(I2{}, T{}, T{}, u + 1);
      step(I3{}, T{}, T{}, u + 2);
      step(I0{}, T{}, T{}, u + 3);
    }
    step(I1{}, T{}, F{}, n_main + 1);
  }

  if (row < S)
    store_rowmajor<Ty, D / 32>((uint16_t *)a.dq + q_off + (size_t)row * D, dqacc, a.scale, lg);
}

// ---------------------------------------------------------------------------
template <class Ty, int D, int MASK>
bool run_backward(const BwdArgs *a, hipStream_t stream, bool launch, LaunchInfo *info,
                  hipError_t *err) {
  constexpr int NW = 4;
  static char name[96];
  static const char *mk[3] = {"none", "causal", "window"};
  snprintf(name, sizeof(name), "fa_bwd_mfma<%s,d%d,%s,bkv%d,bq%d>", Ty::kName, D, mk[MASK],
           32 * NW, 32 * NW);
  info->name = name;
  info->block_rows = 32 * NW;
  info->threads = NW * 64;
  if (!launch) return true;
  BwdArgs args = *a;
  void *kargs[] = {&args};
  const int64_t rows = (int64_t)a->B * a->H * a->S;
  const int rpb = 256 / (D / 8);
  *err = hipLaunchKernel((const void *)&fa_bwd_delta_kernel<Ty, D>,
                         dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), kargs, 0, stream);
  if (*err != hipSuccess) return true;
  const int nkt = (a->S + 32 * NW - 1) / (32 * NW);
  constexpr int DSPLIT = D == 256 ? 2 : 1;
  *err = hipLaunchKernel((const void *)&fa_bwd_dkdv_kernel<Ty, D, MASK, NW, DSPLIT>,
                         dim3((unsigned)(nkt * DSPLIT * a->B * a->Hkv)), dim3(NW * 64), kargs, 0,
                         stream);
  if (*err != hipSuccess) return true;
  *err = hipLaunchKernel((const void *)&fa_bwd_dq_kernel<Ty, D, MASK, NW>,
                         dim3((unsigned)(nkt * a->B * a->H)), dim3(NW * 64), kargs, 0, stream);
  return true;
}

template <class Ty, int D>
bool bwd_by_mask(int mask, const BwdArgs *a, hipStream_t s, bool launch, LaunchInfo *info,
                 hipError_t *err) {
  switch (mask) {
    case kMaskNone: return run_backward<Ty, D, kMaskNone>(a, s, launch, info, err);
    case kMaskCausal: return run_backward<Ty, D, kMaskCausal>(a, s, launch, info, err);
    case kMaskWindow: return run_backward<Ty, D, kMaskWindow>(a, s, launch, info, err);
  }
  return false;
}

template <class Ty>
bool bwd_by_dim(int d, int mask, const BwdArgs *a, hipStream_t s, bool launch, LaunchInfo *info,
                hipError_t *err) {
  switch (d) {
    case 64: return bwd_by_mask<Ty, 64>(mask, a, s, launch, info, err);
    case 128: return bwd_by_mask<Ty, 128>(mask, a, s, launch, info, err);
    case 256: return bwd_by_mask<Ty, 256>(mask, a, s, launch, info, err);
  }
  return false;
}

}  // namespace

bool mfma_backward(DType dt, int d, int mask, const BwdArgs *a, hipStream_t stream, bool launch,
                   LaunchInfo *info, hipError_t *err) {
  if (dt == kBF16) return bwd_by_dim<TBF16>(d, mask, a, stream, launch, info, err);
  if (dt == kF16) return bwd_by_dim<TF16>(d, mask, a, stream, launch, info, err);
  return false;
}

}  // namespace fa
