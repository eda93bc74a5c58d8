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
// n = 1024 work-groups visit almost every one of the 256 compute units.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

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

// Rate of the real-time counter of the current device in kHz, or -1.
int fa_clock_realtime_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}

}  // extern "C"
