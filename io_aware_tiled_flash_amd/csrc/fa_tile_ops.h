// LDS operand addressing shared by the backward and decode kernels: per-lane
// byte offsets of MFMA operands read from [32 rows][d] tiles stored under the
// 64-bank swizzle swz<d>.  Internal; not part of the ABI.
#pragma once

#include "fa_gfx950.h"

namespace fa {
namespace tile {

// Per-lane LDS byte offsets of the two operand kinds on a [32 rows][D] tile
// stored under swz<D> (the forward kernel's decomposition):
//   * row operand of step ks: row lq, logical chunk 2*ks + lg (ds_read_b128);
//   * transposed operand of step kk, d block db, part i2: rows
//     16*kk + 8*i2 + 4*lg + 0..3 of column 32*db + lane%32 (two
//     ds_read_b64_tr_b16, one per i2).
template <int D>
struct TileOffsets {
  static constexpr int KSW = D >= 128 ? 8 : 4;
  static constexpr int NVB = D >= 128 ? 8 : 4;
  int row_base[KSW];
  int tr_base[NVB];
  __device__ inline TileOffsets(int lane) {
    const int lq = lane & 31, lg = lane >> 5;
#pragma unroll
    for (int j = 0; j < KSW; ++j) row_base[j] = lq * (D * 2) + 16 * swz<D>(lq, 2 * j + lg);
    const int tr_row = 4 * lg + ((lane & 15) >> 2);
    const int tr_c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int j = 0; j < NVB; ++j) {
      const int r = 8 * (j & 1) + tr_row;
      tr_base[j] = r * (D * 2) + 16 * swz<D>(r, 4 * (j >> 1) + tr_c) + 8 * (lane & 1);
    }
  }
  __device__ inline u32x4 row_op(const char *tile, int ks) const {
    return *(const u32x4 *)(tile + row_base[ks % KSW] + 16 * 2 * KSW * (ks / KSW));
  }
  __device__ inline u32x4 tr_op(const char *tile, int kk, int db) const {
    u32x4 op;
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const u32x2 v2 = lds_read_tr16((const FA_LDS void *)(tile + tr_base[2 * (db & 3) + i2] +
                                                           16 * kk * (D * 2) + 64 * (db & ~3)));
      op[2 * i2] = v2[0];
      op[2 * i2 + 1] = v2[1];
    }
    return op;
  }
};

}  // namespace tile
}  // namespace fa
