// Shader-clock sampler for the benchmark (measurement support, not part of
// the attention ABI; built into its own library, libfa_clock.so).
//
// The attention kernels' percentage of peak is quoted twice: against the
// published peak (2.4 GHz) and against the peak at the clock the chip
// actually ran at over the timed region.  Under sustained matrix-core load
// the MI355X lowers its shader clock (power limit), so the second figure says
// how much of the gap is clock and how much is the kernel.
//
// fa_clock_sample launches one tiny kernel of `n` work-groups on `stream`.
// Work-group i writes three 64-bit words to dst[3 i .. 3 i + 2]:
//   * the compute unit it ran on: the die (hardware register XCC_ID, 0..7 on
//     MI355X) in bits 0..3, and the shader engine, array and CU fields of
//     the HW_ID register (its bits 8..15) in bits 4..11;
//   * the shader-clock cycle counter (s_memtime: it counts shader clock
//     cycles, so its rate follows the clock; counters of different compute
//     units are not aligned with each other);
//   * the constant-rate real-time counter (s_memrealtime, at the rate
//     fa_clock_realtime_khz returns).
// Two samples taken on one stream before and after a stretch of work give,
// for every compute unit seen in both, the mean shader clock over that
// stretch:
//   (cycles_after - cycles_before) / (real_after - real_before) * real_rate.
// The cycle counter advances only while the compute unit is active, so the
// stretch must be continuous work (idle gaps read as a lower clock).
// n = 1024 work-groups visit almost every one of the 256 compute units.
//
// fa_mfma_ceiling measures what the matrix cores sustain on this part when
// nothing else limits them: every wave runs chains of v_mfma_f32_32x32x16
// (bf16 or fp16) on register operands drawn like the attention inputs
// (roughly standard normal), with no memory traffic in the loop.  Under
// sustained load the part's power limit sets the clock, so this rate, not the
// published peak, is the most any attention kernel can reach on operands of
// that kind.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 32-bit integer hash (the finaliser of MurmurHash3).
__device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

// About standard normal: the centred sum of four uniforms, scaled to unit
// variance (Irwin-Hall), from one 32-bit hash (four 8-bit uniforms).
__device__ inline float normalish(uint32_t h) {
  const float s = (float)(h & 255u) + (float)((h >> 8) & 255u) + (float)((h >> 16) & 255u) +
                  (float)(h >> 24);
  return (s * (1.f / 256.f) - 2.f) * 1.7320508f;
}

// Eight values packed as bf16 (FP16 = false) or fp16 pairs; bf16 keeps the
// upper half of the fp32 pattern.
template <bool FP16>
__device__ inline u32x4 operand(uint32_t key) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x0 = normalish(mix32(key + 2u * j)), x1 = normalish(mix32(key + 2u * j + 1u));
    uint32_t lo, hi;
    if (FP16) {
      lo = __builtin_bit_cast(uint16_t, (_Float16)x0);
      hi = __builtin_bit_cast(uint16_t, (_Float16)x1);
    } else {
      lo = __builtin_bit_cast(uint32_t, x0) >> 16;
      hi = __builtin_bit_cast(uint32_t, x1) >> 16;
    }
    r[j] = lo | (hi << 16);
  }
  return r;
}

template <bool FP16>
__device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (FP16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Per wave and round: 64 products over 8 A and 8 B operands (every product a
// different pair), into 4 independent accumulators.  One float per thread is
// stored at the end so that nothing is optimised away.
template <bool FP16>
__global__ __launch_bounds__(256) void mfma_ceiling_kernel(float *out, int rounds, uint32_t seed) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = operand<FP16>(mix32(seed ^ (t * 64u + 8u * i)));
    b[i] = operand<FP16>(mix32(~seed ^ (t * 64u + 8u * i)));
  }
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[(8 * j + i) & 3] = mfma<FP16>(a[i], b[(i + j) & 7], acc[(8 * j + i) & 3]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 16; ++k) s += acc[i][k];
  out[t] = s;
}

// hwreg(HW_REG_XCC_ID, offset 0, 4 bits): register id 20, size field 4 - 1;
// hwreg(HW_REG_HW_ID): register id 4, all 32 bits
constexpr int kXccIdReg = 20 | (3 << 11);
constexpr int kHwIdReg = 4 | (31 << 11);

__global__ void clock_sample_kernel(uint64_t *dst) {
  if (threadIdx.x != 0) return;
  const uint64_t xcc = __builtin_amdgcn_s_getreg(kXccIdReg) & 0xfu;
  const uint64_t hw = __builtin_amdgcn_s_getreg(kHwIdReg);
  const uint64_t cu_key = xcc | (((hw >> 8) & 0xffu) << 4);
  const uint64_t cycles = __builtin_amdgcn_s_memtime();
  const uint64_t real = __builtin_amdgcn_s_memrealtime();
  dst[3 * blockIdx.x + 0] = cu_key;
  dst[3 * blockIdx.x + 1] = cycles;
  dst[3 * blockIdx.x + 2] = real;
}

}  // namespace

extern "C" {

// dst: device buffer of 3 * n uint64_t; 1 <= n <= 4096.  Returns 0 on
// success, -1 on bad arguments, else the HIP error code of the launch.
int fa_clock_sample(void *dst, int n, void *stream) {
  if (!dst || n < 1 || n > 4096 || (uintptr_t)dst % 8 != 0) return -1;
  hipLaunchKernelGGL(clock_sample_kernel, dim3(n), dim3(64), 0, (hipStream_t)stream,
                     (uint64_t *)dst);
  return (int)hipGetLastError();
}

// Matrix-core ceiling run: n_wg work-groups of 256 threads (4 waves), each
// wave `rounds` x 64 products of 32 x 32 x 16 (32768 flop each); dtype 1 =
// fp16, 2 = bf16 operands.  out: device buffer of 256 * n_wg floats.
// Returns 0, -1 on bad arguments, else the HIP error code of the launch.
int fa_mfma_ceiling(void *out, int n_wg, int rounds, int dtype, unsigned seed, void *stream) {
  if (!out || n_wg < 1 || rounds < 1 || (dtype != 1 && dtype != 2) || (uintptr_t)out % 4 != 0)
    return -1;
  if (dtype == 1)
    hipLaunchKernelGGL(mfma_ceiling_kernel<true>, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                       (float *)out, rounds, (uint32_t)seed);
  else
    hipLaunchKernelGGL(mfma_ceiling_kernel<false>, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                       (float *)out, rounds, (uint32_t)seed);
  return (int)hipGetLastError();
}

// Rate of the real-time counter of the current device in kHz, or -1.
int fa_clock_realtime_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}

}  // extern "C"
