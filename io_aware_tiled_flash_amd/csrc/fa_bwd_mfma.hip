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
//     head that reads this key/value head.  At d = 256 (where K, V and
//     whole-d accumulators exceed a wave's registers) one work-group per 64
//     keys, whose waves work in pairs: one computes S, the other dP, they
//     exchange the fp32 tiles through LDS and each accumulates dK and dV for
//     half of the columns;
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
// dK and dV: one work-group per 32*NW keys of one key/value head.
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
template <class Ty, int D, int MASK, int NW>
__global__ __launch_bounds__(NW * 64, 1) void fa_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BKV = 32 * NW;  // keys per work-group
  constexpr int BQ = 32;        // query rows per streamed tile
  constexpr int NKS = D / 16, NDB = D / 32, KCH = D / 8;
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
  int kvi = blockIdx.x % n_kv;  // key/value head (b * Hkv + hk)
  int kt = blockIdx.x / n_kv;   // key tile; the first ones see the most rows
  if (MASK == kMaskNone && n_kv % 8 == 0) {
    // no imbalance to order by: each XCD (work-group b goes to XCD b % 8)
    // runs a head's key tiles in a row, so they share its query stream in
    // that XCD's L2
    const int nkt = gridDim.x / n_kv, xcd = blockIdx.x % 8, l = blockIdx.x / 8;
    kvi = (l / nkt) * 8 + xcd;
    kt = l % nkt;
  }
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

  const TileOffsets<D> off(lane);
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
    float dl[16];
    if (HAS_PREV) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 d4 = *(const float4 *)&stat_lds[prev][1][8 * q4 + 4 * lg];
        dl[4 * q4 + 0] = d4.x;
        dl[4 * q4 + 1] = d4.y;
        dl[4 * q4 + 2] = d4.z;
        dl[4 * q4 + 3] = d4.w;
      }
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

  // dK = scale * dS^T Q; each lane holds d values of key kw0 + lq.
  const int key = kw0 + lq;
  if (key < S) {
    store_rowmajor<Ty, NDB>((uint16_t *)a.dk + kv_off + (size_t)key * D, dkacc, a.scale, lg);
    store_rowmajor<Ty, NDB>((uint16_t *)a.dv + kv_off + (size_t)key * D, dvacc, 1.f, lg);
  }
}

// ---------------------------------------------------------------------------
// dK and dV by wave pairs: one work-group per 32*NP keys of one key/value
// head, 2*NP waves.  The two waves of a pair own the same 32 keys: the first
// (role 0) keeps their K rows in registers and computes S = Q K^T, the
// second (role 1) keeps their V rows and computes dP = dO V^T, each over the
// whole d.  Role 0 turns S into the weights P, role 1 turns dP into
// X = dP - D; each writes its fp32 tile to LDS and reads its partner's, both
// form dS = P * X, and each accumulates dV += dO^T P and dK += Q^T dS for its
// half of the columns.  A pair's matrix work per tile is the four products
// once (no recomputation) and each wave holds one of K, V and half of the
// accumulators, which is what lets the head width reach 256.
//
// The pipeline is the whole-d kernel's: phase 1 of step u runs the S(u) or
// dP(u) chain beside dS(u-1) and its packing, phase 2 runs dV and dK of tile
// u-1 beside the wave's own P(u) or X(u), written to the exchange buffer at
// the end of the step.  The tile loop is compiled once per role, so every
// LDS offset is a compile-time constant.  With XB = 2 exchange buffers (by
// tile parity) the step's one barrier orders each write after the partner's
// read of the same buffer; with XB = 1 (where LDS holds only one) a second
// barrier after phase 1 does.
template <class Ty, int D, int MASK, int NP, int XB>
__global__ __launch_bounds__(NP * 128, 1) void fa_bwd_dkdv_pair_kernel(BwdArgs a) {
  constexpr int NW = 2 * NP;      // waves
  constexpr int BKV = 32 * NP;    // keys per work-group
  constexpr int BQ = 32;          // query rows per streamed tile
  constexpr int NKS = D / 16, NDB = D / 64, KCH = D / 8;  // NDB: d blocks per role
  constexpr int TILE_CHUNKS = BQ * KCH;
  constexpr int LPW = TILE_CHUNKS / 64 / NW;  // 16-byte loads per wave per tile and tensor
  constexpr int LOADS = 2 * LPW + 1;          // per wave per tile (Q, dO, one statistic)
  constexpr int NST = 4, PF = 2, RPD = 3;
  constexpr int NS1 = NKS;                    // phase-1 MFMAs (S or dP)
  constexpr int NS2 = 4 * NDB;                // phase-2 MFMAs (dV and dK, 2 key halves)
  static_assert(TILE_CHUNKS % (64 * NW) == 0, "tile must split evenly over the waves");
  // [tensor: Q, dO][stage]: the dO stages follow the Q stages
  __shared__ u32x4 tiles[2][NST][TILE_CHUNKS];
  __shared__ float stat_lds[NST][2][64];      // [stage][LSE, D][row]
  // [buffer][pair][role][part][lane]: a wave's 16 fp32 values per lane, in
  // four parts of four, part-major so that one part is 1 KB of consecutive
  // lanes
  __shared__ f32x4 x_lds[XB][NP][2][4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave % NP, role = wave / NP;
  const int lq = lane & 31, lg = lane >> 5;
  const int S = a.S, H = a.H, Hkv = a.Hkv, group = H / Hkv;
  const int n_kv = a.B * Hkv;
  int kvi = blockIdx.x % n_kv;  // key/value head (b * Hkv + hk)
  int kt = blockIdx.x / n_kv;   // key tile; the first ones see the most rows
  if (MASK == kMaskNone && n_kv % 8 == 0) {
    // no imbalance to order by: each XCD (work-group b goes to XCD b % 8)
    // runs a head's key tiles in a row, so they share its query stream in
    // that XCD's L2
    const int nkt = gridDim.x / n_kv, xcd = blockIdx.x % 8, l = blockIdx.x / 8;
    kvi = (l / nkt) * 8 + xcd;
    kt = l % nkt;
  }
  const int b = kvi / Hkv, hk = kvi - b * Hkv;
  const int k0 = kt * BKV, kw0 = k0 + 32 * pair;
  const float c = a.scale_log2;

  const size_t kv_off = (size_t)kvi * (size_t)S * D;
  const uint32_t head_bytes = (uint32_t)S * D * 2u;
  // This wave's keys as the B operand of its product: lane (key kw0 + lq,
  // group lg) holds row chunk 2*ks + lg of K (role 0) or V (role 1).
  const __amdgpu_buffer_rsrc_t rkv =
      make_rsrc((const uint16_t *)(role ? a.v : a.k) + kv_off, head_bytes);
  u32x4 kvreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    kvreg[ks] = load16(rkv, (uint32_t)((kw0 + lq) * D + 16 * ks + 8 * lg) * 2u);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+a"(kvreg[ks]));

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

  const TileOffsets<D> off(lane);
  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dkacc[i] = dvacc[i] = f32x16{};

  // Stream cursors, as in the whole-d kernel.
  struct Cursor {
    int j, qt;
  };
  auto advance = [&](Cursor &cu) __attribute__((always_inline)) {
    const bool wrap = cu.qt + 1 == qt_end;
    cu.qt = wrap ? qt_begin : cu.qt + 1;
    cu.j += wrap ? 1 : 0;
  };
  auto row0_of = [&](const Cursor &cu) __attribute__((always_inline)) {
    return cu.j < group ? cu.qt * BQ : S + BQ;
  };
  Cursor ld{0, qt_begin}, fin{0, qt_begin};
  struct Src {
    u32x4 q, dout, stat;
    int row0;
  } src;
  auto set_src = [&]() __attribute__((always_inline)) {
    const int bh = b * H + hk * group + (ld.j < group ? ld.j : 0);
    const size_t q_off = (size_t)bh * (size_t)S * D;
    src.q = rsrc_words((const uint16_t *)a.q + q_off, head_bytes);
    src.dout = rsrc_words((const uint16_t *)a.dout + q_off, head_bytes);
    // waves 0 and 1 load LSE and D; the others load the same rows again into
    // the same slots (identical bytes), which keeps every wave's load count
    // equal for the counted waits
    const float *st = (wave & 1) ? a.delta : a.lse;
    src.stat = rsrc_words(st + (size_t)bh * S, (uint32_t)S * 4u);
    src.row0 = row0_of(ld);
  };
  auto dma = [&](int st, int d) __attribute__((always_inline)) {
    if (d < 2 * LPW) {
      const int i = d % LPW;
      const int blk = wave * LPW + i;
      const int pos = 64 * blk + lane;
      const int r = pos / KCH, cc = swz<D>(r, pos % KCH);
      const uint32_t o = (uint32_t)((src.row0 + r) * D + 8 * cc) * 2u;
      if (d < LPW)
        load16_to_lds(src.q, o, (uint32_t)(uintptr_t)&tiles[0][st][64 * blk]);
      else
        load16_to_lds(src.dout, o, (uint32_t)(uintptr_t)&tiles[1][st][64 * blk]);
    } else {
      load4_to_lds(src.stat, (uint32_t)(src.row0 + lane) * 4u,
                   (uint32_t)(uintptr_t)&stat_lds[st][wave & 1][0]);
    }
  };

  // Pipeline registers: the product of the current tile (S or dP), the
  // wave's own fp32 values of the newest tile (P or X), packed P and dS of
  // the previous tile.
  f32x16 acc1;
  float own[16];
  u32x4 ppk[2], dspk[2];
  // this pair's exchange slots from (pair, role 0, part 0, lane)
  FA_LDS f32x4 *const x_lane =
      (FA_LDS f32x4 *)(uintptr_t)(uint32_t)(uintptr_t)&x_lds[0][pair][0][0][lane];

  auto edge_of = [&](int row0) __attribute__((always_inline)) {
    if (MASK == kMaskNone) return false;
    bool e = row0 < kw0 + 31;
    if (MASK == kMaskWindow) e = e || row0 + BQ - 1 > kw0 - 1 + a.window;
    return e;
  };

  auto run = [&](auto role_c) __attribute__((always_inline)) {
    constexpr int R = decltype(role_c)::value;
    // slot (buffer xb, role rr, part q4) of this pair and lane
    auto x_at = [&](int xb, int rr, int q4) __attribute__((always_inline)) {
      return x_lane + ((xb * NP * 2 + rr) * 4 + q4) * 64;
    };
    // Per-lane operand offsets: this role's row operand (Q for role 0, dO
    // for role 1), and the transposed Q and dO operands of its half of the
    // columns.  Where the dO stages lie beyond the 16-bit immediate of the
    // LDS reads (FAR, d = 256), the role's offsets carry the distance from
    // the Q stages so that every stage and step offset stays an immediate;
    // otherwise the tile pointers carry it and the offsets are the common
    // ones.
    constexpr int TSZ = (int)sizeof(tiles[0]);
    constexpr bool FAR = 2 * TSZ > 65536;
    int rb[TileOffsets<D>::KSW], tq[TileOffsets<D>::NVB], td[TileOffsets<D>::NVB];
#pragma unroll
    for (int j = 0; j < TileOffsets<D>::KSW; ++j) rb[j] = off.row_base[j] + (FAR ? R * TSZ : 0);
#pragma unroll
    for (int j = 0; j < TileOffsets<D>::NVB; ++j) {
      tq[j] = off.tr_base[j] + (FAR ? 64 * NDB * R : 0);
      td[j] = tq[j] + (FAR ? TSZ : 0);
    }
    auto row_op = [&](const char *tile, int ks) __attribute__((always_inline)) {
      constexpr int KSW = TileOffsets<D>::KSW;
      return *(const u32x4 *)(tile + rb[ks % KSW] + 16 * 2 * KSW * (ks / KSW));
    };
    auto tr_op = [&](const char *tile, const int (&base)[TileOffsets<D>::NVB], int kk, int db)
                     __attribute__((always_inline)) {
      u32x4 op;
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const u32x2 v2 = lds_read_tr16((const FA_LDS void *)(tile + base[2 * (db & 3) + i2] +
                                                             16 * kk * (D * 2) + 64 * (db & ~3)));
        op[2 * i2] = v2[0];
        op[2 * i2 + 1] = v2[1];
      }
      return op;
    };
    auto step = [&](auto phase_c, auto has_prev_c, auto has_cur_c)
                    __attribute__((always_inline)) {
      constexpr int P = decltype(phase_c)::value;
      constexpr bool HAS_PREV = decltype(has_prev_c)::value,
                     HAS_CUR = decltype(has_cur_c)::value;
      constexpr int cur = P, prev = (P + NST - 1) % NST, ldst = (P + PF) % NST;
      constexpr int xw = XB == 2 ? (P & 1) : 0, xr = XB == 2 ? ((P + 1) & 1) : 0;
      const char *rc = (const char *)&tiles[FAR ? 0 : R][cur][0];
      const char *qpc = (const char *)&tiles[0][prev][0] + (FAR ? 0 : 64 * NDB * R);
      const char *dpc = (const char *)&tiles[FAR ? 0 : 1][prev][0] + (FAR ? 0 : 64 * NDB * R);
      set_src();
      // ---- phase 1: S(u) or dP(u) | dS(u-1) ----
      float xv[16];
      if (HAS_PREV) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v4 = *x_at(xr, 1 - R, q4);
          xv[4 * q4 + 0] = v4.x;
          xv[4 * q4 + 1] = v4.y;
          xv[4 * q4 + 2] = v4.z;
          xv[4 * q4 + 3] = v4.w;
        }
      }
      u32x4 rop[RPD + 1];
      if (HAS_CUR) {
#pragma unroll
        for (int st = 0; st < RPD; ++st) rop[st] = row_op(rc, st);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NS1; ++st) {
        if (HAS_CUR) {
          if (st + RPD < NS1) rop[(st + RPD) % (RPD + 1)] = row_op(rc, st + RPD);
          acc1 = Ty::mfma(rop[st % (RPD + 1)], kvreg[st], st == 0 ? f32x16{} : acc1);
        }
#pragma unroll
        for (int d = 0; d < LOADS; ++d)
          if ((d * NS1) / LOADS == st) dma(ldst, d);
        if (HAS_PREV) {
          // dS = P * X (the same product on both waves); P is the own
          // values on role 0 and the partner's on role 1
#pragma unroll
          for (int r = st * 16 / NS1; r < (st + 1) * 16 / NS1; ++r) {
            const float p = R == 0 ? own[r] : xv[r];
            const float ds = own[r] * xv[r];
            own[r] = ds;
            xv[r] = p;
            if (r & 1) {
              dspk[r >> 3][(r & 7) >> 1] = Ty::pack2(own[r - 1], ds);
              ppk[r >> 3][(r & 7) >> 1] = Ty::pack2(xv[r - 1], p);
              pin(dspk[r >> 3][(r & 7) >> 1]);
              pin(ppk[r >> 3][(r & 7) >> 1]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (XB == 1 && HAS_PREV && HAS_CUR) {
        // every wave has read the exchange buffer (the reads were consumed
        // above) before any rewrites it
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      // ---- phase 2: dV, dK of tile u-1 | own values of tile u ----
      float sv[16];
      if (HAS_CUR) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 s4 = *(const float4 *)&stat_lds[cur][R][8 * q4 + 4 * lg];
          const float m = R == 0 ? LOG2E : 1.f;
          sv[4 * q4 + 0] = s4.x * m;
          sv[4 * q4 + 1] = s4.y * m;
          sv[4 * q4 + 2] = s4.z * m;
          sv[4 * q4 + 3] = s4.w * m;
        }
      }
      // step st: key half kk = st / (2*NDB), d block db = (st / 2) % NDB,
      // dV (even st) or dK (odd st)
      u32x4 top[RPD + 1];
      auto read_tr = [&](int st) __attribute__((always_inline)) {
        const int kk = st / (2 * NDB), db = (st >> 1) % NDB;
        return (st & 1) ? tr_op(qpc, tq, kk, db) : tr_op(dpc, td, kk, db);
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
            dvacc[db] = Ty::mfma(top[st % (RPD + 1)], ppk[kk], dvacc[db]);
        }
        if (HAS_CUR) {
#pragma unroll
          for (int r = st * 16 / NS2; r < (st + 1) * 16 / NS2; ++r)
            own[r] = R == 0 ? __builtin_amdgcn_exp2f(fmaf(acc1[r], c, -sv[r])) : acc1[r] - sv[r];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      advance(ld);
      if (HAS_CUR) {
        if (R == 0 && MASK != kMaskNone) {
          // row = row0 + 4*lg + off(r): key <= row is off(r) >= t, and under
          // a window key > row - window is off(r) < t + window
          const int row0 = row0_of(fin);
          if (edge_of(row0)) {
            const int t = kw0 + lq - row0 - 4 * lg;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int o = 8 * (r >> 2) + (r & 3);
              bool vis = o >= t;
              if (MASK == kMaskWindow) vis = vis && o < t + a.window;
              if (!vis) own[r] = 0.f;
            }
          }
        }
        advance(fin);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *x_at(xw, R, q4) = f32x4{own[4 * q4], own[4 * q4 + 1], own[4 * q4 + 2],
                                   own[4 * q4 + 3]};
      }
      // Tile u+1 has landed once only tile u+PF's loads are outstanding; the
      // exchange writes are complete before the barrier publishes them.
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LOADS * (PF - 1)) : "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using T = std::true_type;
    using F = std::false_type;
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      set_src();
#pragma unroll
      for (int d = 0; d < LOADS; ++d) dma(u, d);
      advance(ld);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS * (PF - 1)) : "memory");
    __builtin_amdgcn_s_barrier();
    step(I0{}, F{}, T{});
    const int n_main = (total - 1 + NST - 1) / NST * NST;
    for (int u = 1; u <= n_main; u += NST) {
      step(I1{}, T{}, T{});
      step(I2{}, T{}, T{});
      step(I3{}, T{}, T{});
      step(I0{}, T{}, T{});
    }
    step(I1{}, T{}, F{});
  };

  // Settle the bookkeeping of the kernel-argument scalar loads before the
  // loop (see the forward kernel).
  asm volatile("" ::"s"(a.q), "s"(a.dout), "s"(a.lse), "s"(a.delta));
  if (total > 0) {
    if (role == 0)
      run(std::integral_constant<int, 0>{});
    else
      run(std::integral_constant<int, 1>{});
  }

  // dK = scale * dS^T Q; each lane holds this wave's half of the d values of
  // key kw0 + lq.
  const int key = kw0 + lq;
  if (key < S) {
    const size_t o = kv_off + (size_t)key * D + 32 * NDB * role;
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
  int slot = blockIdx.x % BH, qt = blockIdx.x / BH;
  if (MASK == kMaskNone && BH % 8 == 0) {
    // each XCD runs a head's query tiles in a row (shared K/V in its L2)
    const int xcd = blockIdx.x % 8, l = blockIdx.x / 8;
    slot = (l / nqt) * 8 + xcd;
    qt = l % nqt;
  }
  const HeadPair hp = head_of_slot(slot, a.B, a.H, a.Hkv);
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
  if constexpr (D == 256) {
    // wave pairs, 64 keys per work-group; LDS holds one exchange buffer
    constexpr int NP = 2;
    const int nkt_p = (a->S + 32 * NP - 1) / (32 * NP);
    *err = hipLaunchKernel((const void *)&fa_bwd_dkdv_pair_kernel<Ty, D, MASK, NP, 1>,
                           dim3((unsigned)(nkt_p * a->B * a->Hkv)), dim3(NP * 128), kargs, 0,
                           stream);
  } else {
    *err = hipLaunchKernel((const void *)&fa_bwd_dkdv_kernel<Ty, D, MASK, NW>,
                           dim3((unsigned)(nkt * a->B * a->Hkv)), dim3(NW * 64), kargs, 0,
                           stream);
  }
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
