// clock_stamp.hip -- shader-clock stamps for the benchmark (not part of the
// quantizer / GEMM library).
//
// Each workgroup of one small launch records where it runs (its XCD and its
// compute unit's place in it, from HW_REG_XCC_ID and HW_REG_HW_ID), the
// shader-clock counter (s_memtime, which advances once per shader clock and
// is kept per compute unit) and the constant-rate real-time counter
// (s_memrealtime).  Two launches on the benchmark's stream, one before and one
// after the timed steps, give the average shader clock over the steps of
// every compute unit that ran a workgroup of both: d(memtime) / d(realtime)
// times the real-time counter's rate (hipDeviceAttributeWallClockRate).
#include <hip/hip_runtime.h>
#include <stdint.h>

constexpr int kStampGroups = 2048;   // 8 per compute unit, so most units run one in both launches

__global__ void __launch_bounds__(64) clock_stamp_kernel(uint64_t* out) {
  if (threadIdx.x != 0) return;
  uint32_t xcc, hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  // place: XCD, then HW_ID's compute-unit, shader-array and engine fields
  // (bits 8..15; the wave, SIMD and pipe fields below them are left out)
  out[3 * blockIdx.x + 0] = ((uint64_t)(xcc & 0xF) << 8) | ((hw >> 8) & 0xFF);
  out[3 * blockIdx.x + 1] = t;
  out[3 * blockIdx.x + 2] = r;
}

extern "C" {

// Number of uint64 slots one stamp writes.
int mxclock_stamp_slots(void) { return 3 * kStampGroups; }

// out: device, mxclock_stamp_slots() uint64 values, 8-byte aligned.
int mxclock_stamp(uint64_t* out, hipStream_t stream) {
  if (!out) return -1;
  hipLaunchKernelGGL(clock_stamp_kernel, dim3(kStampGroups), dim3(64), 0, stream, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Rate of the real-time counter in kHz (0 if the query fails).
int mxclock_wall_rate_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}
}
