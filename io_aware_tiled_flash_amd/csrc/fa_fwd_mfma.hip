// Exact attention forward for bf16 / fp16 inputs on CDNA4 (gfx950) matrix cores.
//
// Method: the tiled forward pass with the online softmax ("FlashAttention: Why
// Tiling Attention Makes Transformers Fast Without Changing the Result",
// sections "Online softmax: correct as you go" and "The tiled forward pass";
// aicomputerinstitute.com grade-12 flash-attention chapter, section "Tiling
// and the running (online) softmax").  Per query row the kernel keeps a
// running maximum m, a running denominator l and an unnormalised fp32 output
// accumulator; for every visible key tile it rescales l and the accumulator by
// exp(m_old - m_new) when the maximum grows, adds the tile's exponentiated
// scores, and divides by l once after the last tile.  Score and probability
// tiles live only in registers.  The work split over the query sequence (one
// work-group per query tile, per batch and head) is the one the same chapter
// describes under "What FlashAttention-2 changed"; each wavefront owns
// distinct query rows, so waves never combine partial results.
//
// gfx950 mapping (one work-group = NW wave64s, 32 query rows per wave):
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{bf16,f16}: lane (q = lane%32, g = lane/32) then
//     holds 16 of the 32 keys of one query column, so a row maximum or sum is
//     a register reduction plus one exchange with lane^32;
//   * Q^T (the B operand) is loaded once into VGPRs;
//   * K tiles are staged in LDS row-major with a 16-byte-chunk XOR swizzle so
//     that the A-operand reads (one 16-byte chunk per lane, 32 rows) are free
//     of bank conflicts;
//   * V tiles are staged in LDS transposed ([d][key]); the transpose happens
//     in registers between the global load and the LDS store.  Keys inside
//     each 16-key group are stored with bits 2 and 3 of the key index swapped,
//     which makes the P^T accumulator layout of S^T usable directly as the B
//     operand of O^T = V^T P^T (a contraction does not care about the order
//     of its summation index, only that both operands agree);
//   * K/V tiles are double-buffered: the global loads of tile t+1 are issued
//     before the math of tile t and written to the other LDS stage after it,
//     with one barrier per tile;
//   * causal and sliding-window masks skip whole tiles: the work-group visits
//     only key tiles that intersect its rows' visible band, a wave skips the
//     math of tiles that are invisible to all of its rows, and elementwise
//     masking runs only on tiles that straddle a band edge;
//   * scores are scaled into base 2 (scale * log2 e folded into one multiply)
//     so every exponential is a single v_exp_f32;
//   * heavy query tiles (the last ones, under a causal or window mask) are
//     dispatched first; consecutive work-groups take different heads, so with
//     the round-robin placement over the 8 XCDs all query tiles of one head
//     land on the same XCD and share its L2.
#include "fa_internal.h"

#include <math.h>

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

__device__ inline float wave_partner(float x) {  // value held by lane ^ 32
  return __shfl_xor(x, 32, 64);
}

template <int MASK>
__device__ inline bool key_visible(int key, int row, int S, int window) {
  if (MASK == kMaskNone) return key < S;
  if (MASK == kMaskCausal) return key <= row;
  return key <= row && key > row - window;
}

template <class Ty, int D, int MASK, int NW, int BC>
__global__ __launch_bounds__(NW * 64, 1) void fa_fwd_mfma_kernel(FwdArgs a) {
  constexpr int NT = NW * 64;          // threads per work-group
  constexpr int BR = 32 * NW;          // query rows per work-group
  constexpr int NKB = BC / 32;         // 32-key blocks per key tile
  constexpr int NKS = D / 16;          // contraction steps of S^T = K Q^T
  constexpr int NDB = D / 32;          // 32-wide d blocks of O^T
  constexpr int NPS = BC / 16;         // contraction steps of O^T = V^T P^T
  constexpr int KCH = D / 8;           // 16-byte chunks per K row
  constexpr int VCH = BC / 8;          // 16-byte chunks per V^T row
  constexpr int K_CHUNKS = BC * D / 8; // 16-byte chunks per K tile
  constexpr int V_BLOCKS = BC * D / 32;  // 4-key x 8-d blocks per V tile
  constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
  constexpr int V_PER_T = (V_BLOCKS + NT - 1) / NT;
  static_assert(D % 32 == 0 && BC % 32 == 0, "tile shape");
  static_assert(VCH >= 8 && KCH >= 8, "swizzle needs >= 8 chunks per LDS row");

  __shared__ u32x4 k_lds[2][BC * KCH];
  __shared__ u32x4 vt_lds[2][D * VCH];

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
  const uint16_t *qh = (const uint16_t *)a.q + head_off;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t *)a.k + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t *)a.v + head_off, head_bytes);

  // Q^T as the B operand: lane holds Q[row][16*ks + 8*lg .. +7] for every ks.
  const int wr0 = q0 + wave * 32;  // first query row of this wave
  const int row = wr0 + lq;
  u32x4 qreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qreg[ks] = load16(rq, (uint32_t)(row * D + 16 * ks + 8 * lg) * 2u);

  // Key tiles this work-group visits.
  const int ntk = (S + BC - 1) / BC;
  int kt_begin = 0, kt_end = ntk;
  if (MASK != kMaskNone) {
    const int last_row = min(q0 + BR, S) - 1;
    kt_end = last_row / BC + 1;
    if (MASK == kMaskWindow) kt_begin = max(0, q0 - a.window + 1) / BC;
  }

  u32x4 kbuf[K_PER_T];
  u32x4 vbuf[V_PER_T][4];

  auto load_tile = [&](int kt) {
    const int k0 = kt * BC;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int ci = tid + i * NT;
      if (K_CHUNKS % NT == 0 || ci < K_CHUNKS) {
        const int r = ci / KCH, c = ci % KCH;
        kbuf[i] = load16(rk, (uint32_t)((k0 + r) * D + 8 * c) * 2u);
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int bi = tid + i * NT;
      if (V_BLOCKS % NT == 0 || bi < V_BLOCKS) {
        const int kg = bi % (BC / 4), dc = bi / (BC / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vbuf[i][r] = load16(rv, (uint32_t)((k0 + 4 * kg + r) * D + 8 * dc) * 2u);
      }
    }
  };

  auto store_tile = [&](int stage) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int ci = tid + i * NT;
      if (K_CHUNKS % NT == 0 || ci < K_CHUNKS) {
        const int r = ci / KCH, c = ci % KCH;
        k_lds[stage][r * KCH + (c ^ (r & 7))] = kbuf[i];
      }
    }
    char *vt_base = (char *)&vt_lds[stage][0];
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int bi = tid + i * NT;
      if (V_BLOCKS % NT == 0 || bi < V_BLOCKS) {
        const int kg = bi % (BC / 4), dc = bi / (BC / 4);
        // key 4*kg+j sits at position 4*swap01(kg)+j inside the d row
        const int kgs = (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1);
        const int chunk = kgs >> 1, half = kgs & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x2 w;
          w[0] = __builtin_amdgcn_perm(vbuf[i][1][e >> 1], vbuf[i][0][e >> 1], sel);
          w[1] = __builtin_amdgcn_perm(vbuf[i][3][e >> 1], vbuf[i][2][e >> 1], sel);
          const int d = 8 * dc + e;
          *(u32x2 *)(vt_base + d * (BC * 2) + ((chunk ^ (d & 7)) << 4) + (half << 3)) = w;
        }
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m = -INFINITY;  // running max of base-2 scores (same in lanes q and q^32)
  float l = 0.f;        // this lane's share of the running denominator

  if (kt_begin < kt_end) {
    load_tile(kt_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int stage = (kt - kt_begin) & 1;
    const bool has_next = kt + 1 < kt_end;
    if (has_next) load_tile(kt + 1);

    const int k0 = kt * BC;
    bool active = true, need_mask;
    if (MASK == kMaskCausal) {
      active = k0 <= wr0 + 31;
      need_mask = k0 + BC - 1 > wr0;
    } else if (MASK == kMaskWindow) {
      active = k0 <= wr0 + 31 && k0 + BC - 1 > wr0 - a.window;
      need_mask = k0 + BC - 1 > wr0 || k0 <= wr0 + 31 - a.window;
    } else {
      need_mask = k0 + BC > S;
    }

    if (active) {
      const u32x4 *kl = k_lds[stage];
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int r = 32 * kb + lq;
          const u32x4 kop = kl[r * KCH + ((2 * ks + lg) ^ (r & 7))];
          sacc[kb] = Ty::mfma(kop, qreg[ks], sacc[kb]);
        }
      }

      // base-2 scores, masking, tile row max
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float s = sacc[kb][r] * a.scale_log2;
          if (need_mask) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * lg + (r & 3);
            s = key_visible<MASK>(key, row, S, a.window) ? s : -INFINITY;
          }
          sacc[kb][r] = s;
          tmax = fmaxf(tmax, s);
        }
      }
      tmax = fmaxf(tmax, wave_partner(tmax));
      const float m_new = fmaxf(m, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // fully masked so far
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);    // 0 while m is -inf
      m = m_new;

      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(sacc[kb][r] - m_use);
          sacc[kb][r] = p;
          lsum += p;
        }
      }
      l = l * alpha + lsum;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      }

      // P^T as the B operand: step kk = 2*kb + s covers accumulator entries
      // 8*s .. 8*s+7 of key block kb.
      u32x4 pk[NPS];
#pragma unroll
      for (int kk = 0; kk < NPS; ++kk) {
        const int kb = kk >> 1, base = 8 * (kk & 1);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pk[kk][j] = Ty::pack2(sacc[kb][base + 2 * j], sacc[kb][base + 2 * j + 1]);
      }

      const u32x4 *vl = vt_lds[stage];
#pragma unroll
      for (int kk = 0; kk < NPS; ++kk) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + lq;
          const u32x4 vop = vl[d * VCH + ((2 * kk + lg) ^ (d & 7))];
          oacc[db] = Ty::mfma(vop, pk[kk], oacc[db]);
        }
      }
    }

    if (has_next) store_tile(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: one division per row, RNE to the element type, natural-log LSE.
  const float l_tot = l + wave_partner(l);
  if (row < S) {
    const float inv = 1.f / l_tot;
    uint16_t *orow = (uint16_t *)a.o + head_off + (size_t)row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w[0] = Ty::pack2(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
        w[1] = Ty::pack2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
        *(u32x2 *)(orow + 32 * db + 8 * j + 4 * lg) = w;
      }
    }
    if (lg == 0)
      a.lse[(size_t)bh * S + row] = (m + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

template <class Ty, int D, int MASK>
struct Instance {
  static constexpr int NW = 4;
  static constexpr int BC = 64;
  static bool run(const FwdArgs *a, hipStream_t stream, bool launch, LaunchInfo *info,
                  hipError_t *err) {
    static char name[96];
    static const char *mk[3] = {"none", "causal", "window"};
    snprintf(name, sizeof(name), "fa_fwd_mfma<%s,d%d,%s,br%d,bc%d>", Ty::kName, D, mk[MASK],
             32 * NW, BC);
    info->name = name;
    info->block_rows = 32 * NW;
    info->threads = NW * 64;
    if (!launch) return true;
    const int nq = (a->S + 32 * NW - 1) / (32 * NW);
    const dim3 grid((unsigned)(nq * a->B * a->H));
    const dim3 block(NW * 64);
    FwdArgs args = *a;
    void *kargs[] = {&args};
    *err = hipLaunchKernel((const void *)&fa_fwd_mfma_kernel<Ty, D, MASK, NW, BC>, grid, block,
                           kargs, 0, stream);
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
