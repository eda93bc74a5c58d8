// Device building blocks shared by the gfx950 matrix-core attention kernels
// (forward and backward): element-type traits for the 32x32x16 MFMA, buffer
// loads (into registers or straight into LDS), the transposing LDS read, the
// 64-bank LDS swizzle, and small helpers.  Internal; not part of the ABI.
#pragma once

#include "fa_internal.h"

namespace fa {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


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
  // the two packed values, exactly, as floats (low half first)
  __device__ static inline f32x2 unpack2(uint32_t w) {
    return f32x2{__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u)};
  }
  // acc + both packed values (v_dot2_f32_bf16 against (1, 1): the products
  // are exact, the sum is an fp32 addition)
  __device__ static inline float add2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
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
  // the two packed values, exactly, as floats (low half first)
  __device__ static inline f32x2 unpack2(uint32_t w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
  }
  // acc + both packed values (v_dot2_f32_f16 against (1, 1))
  __device__ static inline float add2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                  __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
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
// M0 (the LDS base of the direct loads) is a reserved register for this
// compiler: it allocates no value to it, and a clobber list naming it is
// ignored (the compiler warns as much), so none is given.  The kernels rely
// on no compiler-generated instruction reading M0; tests/test_isa.py checks
// that in the generated code.
__device__ inline void load16_to_lds(u32x4 rsrc, uint32_t byte_off, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(byte_off), "s"(rsrc)
      : "memory");
}

// 4 bytes per lane from global memory straight into LDS (lane i's bytes land
// at lds_addr + 4 * i), for per-row statistics; awaited like load16_to_lds.
__device__ inline void load4_to_lds(u32x4 rsrc, uint32_t byte_off, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(byte_off), "s"(rsrc)
      : "memory");
}

// ds_read_b64_tr_b16: in every group of 16 lanes, lanes 4k..4k+3 name row k
// (4 elements each, 16 in total); lane n of the group receives column n, i.e.
// element n of rows 0..3.
__device__ inline u32x2 lds_read_tr16(const FA_LDS void *p) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4 *)const_cast<FA_LDS void *>(p)));
}

// An empty use that keeps a value's computation in the code region where it
// is written (the compiler would otherwise sink ALU work past later branches,
// away from the MFMAs it is meant to run beside).
__device__ inline void pin(float x) { asm volatile("" ::"v"(x)); }
__device__ inline void pin(uint32_t x) { asm volatile("" ::"v"(x)); }

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

}  // namespace tile
}  // namespace fa
