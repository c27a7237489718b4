// noise.hip -- signal and quantization-noise sums of a quantized operand.
//
// "FP4 All the Way: Fully Quantized Training of LLMs", abstract: quantized
// training stops being effective once the gradient norm falls below about
// sqrt(3) times the quantization noise.  The two norms come from one pass
// over the input and its codes: y = the operand's contraction rows (rotated
// by the block Hadamard when the tensor is), Q(y) = the exactly dequantized
// value (E2M1 x scale, NVFP4 x tensor scale; exact in binary64), and
//   stats[0] = sum y^2, stats[1] = sum (Q(y) - y)^2,
//   stats[2] = elements of blocks with a NaN scale byte (left out),
// all in binary64 (squares accumulated with fused multiply-adds).  Each
// workgroup writes its three partial sums, and one
// workgroup adds the partials in a fixed order, so the result does not
// depend on scheduling.
//
// A thread takes 32 consecutive contraction elements of one operand row (16
// for NVFP4 without rotation when the contraction is not a multiple of 32).
// Along axis 1 neighbouring threads take neighbouring units of a row (16-byte
// loads); along axis 0 they take neighbouring operand rows, i.e. neighbouring
// input columns, so every load instruction reads whole lines of x.
#include "fp4_device.h"
#include "mxfp4_internal.h"

namespace mxfp4 {

struct NoiseArgs {
  const uint16_t* x;
  int64_t ldx;
  int64_t rows, K;          // quantized operand [rows, K]
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;          // NVFP4 tensor scale (device)
  int64_t units;            // rows * K / U
  FastDiv div;              // by K / U (axis 1) or rows (axis 0), when units < 2^31
  int small;                // units < 2^31: 32-bit unit indices
  int vec;                  // axis 1: x 16-byte aligned and ldx % 8 == 0
  double* partials;         // 3 per workgroup
};

template <int FMT, bool HAD, int AXIS, int U>
__global__ void __launch_bounds__(256) noise_kernel(NoiseArgs a) {
  constexpr int BS = (FMT == FMT_MX) ? 32 : 16;
  const double st = (FMT == FMT_NV) ? (double)a.ts[0] : 1.0;
  const int64_t nu = a.K / U;                     // units per operand row
  double s0 = 0.0, s1 = 0.0, n = 0.0;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < a.units; u += (int64_t)gridDim.x * 256) {
    int64_t i, b;
    if (a.small) {
      const uint32_t qd = fastdiv((uint32_t)u, a.div), rm = (uint32_t)u - qd * a.div.d;
      if (AXIS == 1) { i = qd; b = rm; } else { b = qd; i = rm; }
    } else if (AXIS == 1) {
      i = u / nu; b = u - i * nu;
    } else {
      b = u / a.rows; i = u - b * a.rows;
    }
    const int64_t k0 = b * U;
    float y[U];
    if (AXIS == 1) {
      const uint16_t* src = a.x + i * a.ldx + k0;
      if (a.vec) {
#pragma unroll
        for (int q = 0; q < U / 8; q++) {
          const u32v4 v = *(const u32v4*)(src + 8 * q);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            y[8 * q + 2 * j] = __uint_as_float(v[j] << 16);
            y[8 * q + 2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < U; j++) y[j] = __uint_as_float((uint32_t)src[j] << 16);
      }
    } else {
      const uint16_t* src = a.x + k0 * a.ldx + i;
#pragma unroll
      for (int j = 0; j < U; j++) y[j] = __uint_as_float((uint32_t)src[(int64_t)j * a.ldx] << 16);
    }
    if constexpr (HAD) fwht32_inlane(y);
    // codes: U / 2 bytes, 8-byte aligned (K / 2 and k0 / 2 are multiples of 8)
    uint32_t cw[U / 8];
    {
      const uint2* cp = (const uint2*)(a.codes + i * (a.K / 2) + k0 / 2);
#pragma unroll
      for (int q = 0; q < U / 16; q++) {
        const uint2 v = cp[q];
        cw[2 * q] = v.x;
        cw[2 * q + 1] = v.y;
      }
    }
    // E2M1 codes -> exact binary32 values (hardware convert, unit scale)
    float g[U];
#pragma unroll
    for (int q = 0; q < U / 8; q++) {
      const f32x2 g0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[q], 1.0f, 0);
      const f32x2 g1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[q], 1.0f, 1);
      const f32x2 g2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[q], 1.0f, 2);
      const f32x2 g3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[q], 1.0f, 3);
      g[8 * q + 0] = g0[0]; g[8 * q + 1] = g0[1]; g[8 * q + 2] = g1[0]; g[8 * q + 3] = g1[1];
      g[8 * q + 4] = g2[0]; g[8 * q + 5] = g2[1]; g[8 * q + 6] = g3[0]; g[8 * q + 7] = g3[1];
    }
    const uint8_t* srow = a.scales + i * (a.K / BS) + k0 / BS;
#pragma unroll
    for (int blk = 0; blk < U / BS; blk++) {
      const uint32_t sb = srow[blk];
      const bool nan_scale = (FMT == FMT_MX) ? (sb == 0xFFu) : ((sb & 0x7Fu) == 0x7Fu);
      if (nan_scale) {
        n += BS;
        continue;
      }
      const double sc = (FMT == FMT_MX) ? (double)e8m0_value(sb) : (double)e4m3_value(sb) * st;
#pragma unroll
      for (int j = 0; j < BS; j++) {
        const int e = blk * BS + j;
        const double q = (double)g[e] * sc;
        const double yv = (double)y[e];
        const double d = q - yv;
        s0 = __builtin_fma(yv, yv, s0);      // yv * yv is exact: the same as a multiply and an add
        s1 = __builtin_fma(d, d, s1);
      }
    }
  }
  block_sum3(s0, s1, n, a.partials + 3 * (int64_t)blockIdx.x);
}

// Fixed-order sum of the partials: 1024 threads, thread t adds partials t,
// t + 1024, ... (four loads in flight), then butterflies within each wave and
// the 16 wave sums in a fixed order.
__global__ void __launch_bounds__(1024) noise_finalize_kernel(const double* __restrict__ partials, int64_t nparts,
                                                              double* __restrict__ stats) {
  __shared__ double red[3][16];
  double a = 0.0, b = 0.0, c = 0.0;
  int64_t p = threadIdx.x;
  for (; p + 3 * 1024 < nparts; p += 4 * 1024) {
    double v[4][3];
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
      for (int j = 0; j < 3; j++) v[q][j] = partials[3 * (p + q * 1024) + j];
#pragma unroll
    for (int q = 0; q < 4; q++) { a += v[q][0]; b += v[q][1]; c += v[q][2]; }
  }
  for (; p < nparts; p += 1024) {
    a += partials[3 * p];
    b += partials[3 * p + 1];
    c += partials[3 * p + 2];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
    c += __shfl_xor(c, off, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][w] = a; red[1][w] = b; red[2][w] = c; }
  __syncthreads();
  if (threadIdx.x < 3) {
    double t = 0.0;
    for (int k = 0; k < 16; k++) t += red[threadIdx.x][k];
    stats[threadIdx.x] = t;
  }
}

void launch_noise_finalize(const double* partials, int64_t nparts, double* stats, hipStream_t s) {
  hipLaunchKernelGGL(noise_finalize_kernel, dim3(1), dim3(1024), 0, s, partials, nparts, stats);
}

// One unit per thread up to 2^16 workgroups (16.7 M units), so that many
// loads are in flight; larger operands loop.
constexpr int kNoiseMaxWGs = 65536;

static int noise_unit(int fmt, int hadamard, int64_t K) {
  return (fmt == FMT_NV && !hadamard && K % 32 != 0) ? 16 : 32;
}

static int64_t noise_wgs(int fmt, int hadamard, int64_t rows, int64_t K) {
  const int64_t units = rows * (K / noise_unit(fmt, hadamard, K));
  int64_t g = (units + 255) / 256;
  if (g > kNoiseMaxWGs) g = kNoiseMaxWGs;
  return g < 1 ? 1 : g;
}

size_t noise_workspace_bytes(int fmt, int hadamard, int64_t rows, int64_t K) {
  return (size_t)noise_wgs(fmt, hadamard, rows, K) * 3 * sizeof(double);
}

template <int FMT, bool HAD, int AXIS, int U>
static void launch_noise_t(const NoiseArgs& a, int64_t g, hipStream_t s) {
  hipLaunchKernelGGL((noise_kernel<FMT, HAD, AXIS, U>), dim3((unsigned)g), dim3(256), 0, s, a);
}

template <int FMT, bool HAD>
static void launch_noise_axis(const NoiseArgs& a, int axis, int u, int64_t g, hipStream_t s) {
  if (u == 16) {
    if constexpr (FMT == FMT_NV && !HAD) {
      if (axis == 1) launch_noise_t<FMT, HAD, 1, 16>(a, g, s);
      else launch_noise_t<FMT, HAD, 0, 16>(a, g, s);
    }
    return;
  }
  if (axis == 1) launch_noise_t<FMT, HAD, 1, 32>(a, g, s);
  else launch_noise_t<FMT, HAD, 0, 32>(a, g, s);
}

hipError_t launch_noise(const uint16_t* x, int64_t ldx, int axis, int fmt, int hadamard, int64_t rows, int64_t K,
                        const uint8_t* codes, const uint8_t* scales, const float* ts, double* stats,
                        double* partials, hipStream_t stream) {
  NoiseArgs a;
  a.x = x;
  a.ldx = ldx;
  a.rows = rows;
  a.K = K;
  a.codes = codes;
  a.scales = scales;
  a.ts = ts;
  const int u = noise_unit(fmt, hadamard, K);
  a.units = rows * (K / u);
  a.small = a.units < ((int64_t)1 << 31) ? 1 : 0;
  a.div = make_fastdiv(a.small ? (uint32_t)(axis == 1 ? K / u : (rows > 0 ? rows : 1)) : 1u);
  a.vec = (((uintptr_t)x & 15) == 0 && ldx % 8 == 0) ? 1 : 0;
  a.partials = partials;
  const int64_t g = noise_wgs(fmt, hadamard, rows, K);
  if (fmt == FMT_MX) {
    if (hadamard) launch_noise_axis<FMT_MX, true>(a, axis, u, g, stream);
    else launch_noise_axis<FMT_MX, false>(a, axis, u, g, stream);
  } else {
    if (hadamard) launch_noise_axis<FMT_NV, true>(a, axis, u, g, stream);
    else launch_noise_axis<FMT_NV, false>(a, axis, u, g, stream);
  }
  launch_noise_finalize(partials, g, stats, stream);
  return hipGetLastError();
}

}  // namespace mxfp4
