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
//
// The MFMA ceiling kernel measures the rate the chip sustains for the scaled
// FP4 MFMA alone (v_mfma_scale_f32_32x32x64_f8f6f4, FP4 operands, unit scales)
// on pseudo-random codes, or for the fp16 MFMA of the NVFP4 GEMM on random
// fp16 values, with no memory traffic: one workgroup of four waves
// per compute unit (its LDS request leaves room for no second one), each wave
// cycling 16 independent accumulators over 4 x 4 operand registers, the
// register pattern of the 256 x 256 GEMM tile.  The power drawn by random
// operands sets the clock, so this is the practical compute ceiling of the
// FP4 GEMM on this part, next to the nominal dense peak at 2.4 GHz.  Each
// workgroup also stamps s_memtime and s_memrealtime around its loop, which
// gives the clock during the run and the counter ticks per MFMA.
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

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kCeilGroups = 256;                 // one per compute unit
constexpr int kCeilLds = 96 * 1024;              // more than half of a compute unit's LDS

// Two rounds of an integer hash of (workgroup, thread, register index).
__device__ __forceinline__ uint32_t ceil_hash(uint32_t gid, uint32_t idx, uint32_t salt) {
  uint32_t h = gid * 2654435761u + idx * 40503u + salt;
  h ^= h >> 15; h *= 0x2c1b3c6du; h ^= h >> 12; h *= 0x297a2d39u; h ^= h >> 15;
  return h;
}

// KIND 0: the scaled FP4 MFMA (32x32x64, every nibble an arbitrary E2M1
// code, unit E8M0 scales).  KIND 1: the fp16 MFMA (32x32x16) that the NVFP4
// GEMM runs on, every operand a random fp16 in [1, 2) with a random sign, so
// that products and sums stay finite.
template <int KIND>
__global__ void __launch_bounds__(256) mfma_ceiling_kernel(int iters, uint64_t* stamps, float* sink) {
  extern __shared__ char lds[];
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  v4i fa[4], fb[4];
  for (int i = 0; i < 4; i++)
    for (int k = 0; k < 4; k++) {
      uint32_t h = ceil_hash(gid, 4 * i + k, 0x9e3779b9u), g = ceil_hash(gid, 4 * i + k, 0x165667b1u);
      if (KIND == 1) {   // two fp16 per word: sign, exponent 15 (2^0), random 10-bit mantissa
        h = (h & 0x83FF83FFu) | 0x3C003C00u;
        g = (g & 0x83FF83FFu) | 0x3C003C00u;
      }
      fa[i][k] = (int)h;
      fb[i][k] = (int)g;
    }
  v16f acc[4][4];
  for (int i = 0; i < 4; i++)
    for (int j = 0; j < 4; j++) acc[i][j] = (v16f){};
  const int unit = 0x7f7f7f7f;                   // E8M0 scale 1.0 in every byte
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if constexpr (KIND == 0) {
          const v8i a = __builtin_shufflevector(fa[i], fa[i], 0, 1, 2, 3, -1, -1, -1, -1);
          const v8i b = __builtin_shufflevector(fb[j], fb[j], 0, 1, 2, 3, -1, -1, -1, -1);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 4, 4, 0, unit, 0, unit);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, fa[i]),
                                                             __builtin_bit_cast(v8h, fb[j]), acc[i][j], 0, 0, 0);
        }
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int i = 0; i < 4; i++)
    for (int j = 0; j < 4; j++)
      for (int k = 0; k < 16; k++) s += acc[i][j][k];
  sink[gid] = s;                                 // keeps every MFMA live
  if (threadIdx.x == 0) {
    stamps[2 * blockIdx.x] = t1 - t0;
    stamps[2 * blockIdx.x + 1] = r1 - r0;
  }
  if (s == 1.2345f) lds[threadIdx.x] = 1;        // the LDS request stays in the kernel
}

template <int KIND>
static int launch_ceiling(int iters, uint64_t* stamps, float* sink, hipStream_t stream) {
  if (!stamps || !sink || iters <= 0) return -1;
  if (hipFuncSetAttribute((const void*)mfma_ceiling_kernel<KIND>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kCeilLds) != hipSuccess)
    return -5;
  hipLaunchKernelGGL(mfma_ceiling_kernel<KIND>, dim3(kCeilGroups), dim3(256), kCeilLds, stream, iters, stamps, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" {

// Sizes of the ceiling run's buffers: uint64 stamp slots and float sink slots.
int mxclock_ceiling_stamp_slots(void) { return 2 * kCeilGroups; }
int mxclock_ceiling_sink_slots(void) { return 256 * kCeilGroups; }
// Scaled FP4 MFMAs (32x32x64) one launch issues, per iteration.
long long mxclock_ceiling_mfmas_per_iter(void) { return (long long)kCeilGroups * 4 * 16; }

// stamps, sink: device buffers of the sizes above.  Per workgroup, stamps
// receives the s_memtime and s_memrealtime differences over its loop.
// kind 0: scaled FP4 32x32x64 (FLOP per MFMA 2 * 32 * 32 * 64); kind 1: fp16
// 32x32x16 (2 * 32 * 32 * 16).
int mxclock_mfma_ceiling(int kind, int iters, uint64_t* stamps, float* sink, hipStream_t stream) {
  if (kind == 0) return launch_ceiling<0>(iters, stamps, sink, stream);
  if (kind == 1) return launch_ceiling<1>(iters, stamps, sink, stream);
  return -1;
}

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
