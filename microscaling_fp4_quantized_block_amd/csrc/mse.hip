// mse.hip -- round-to-nearest quantization with MSE-fitted scales.
//
// The digest of "Bridging the Gap Between Promise and Performance for
// Microscaling FP4 Quantization" (step 1) fits the quantization grid for
// mean squared error by optimizing the block scales and the tensor scale in
// turn.  The procedure, as this library reads it:
//   block step:  each block keeps, among the scales at and below its absmax
//                scale, the one whose round-to-nearest encoding has the
//                smallest sum of (y - Q(y))^2 over its elements (Q(y) exactly
//                dequantized); ties keep the larger scale; elements are
//                encoded as the absmax quantizer encodes them for that scale.
//                Only a few scales below the absmax one can ever win, and the
//                search here tries exactly those:
//                  MXFP4: e0 and e0 - 1.  At e0 - 2 the grid tops out at
//                    1.5 * 2^e0 while the block maximum exceeds 3 * 2^e0, so
//                    its own error grows by more than 2.25 * 4^e0, and the 31
//                    others can gain at most (2^e0 / 8)^2 each (0.48 * 4^e0 in
//                    all) over e0 - 1;
//                  NVFP4: the absmax E4M3 byte b0 and the five below it.  A
//                    linear-programming bound over every mantissa pattern of b0
//                    (and the subnormal bytes) and every block maximum shows
//                    that no block prefers b0 - 6 or less to b0; b0 - 5 does
//                    win for some blocks.
//                The per-candidate error is summed in binary64 (runs of 8
//                elements, then (S0 + S1) + (S2 + S3) or S0 + S1); near ties
//                may resolve differently from an exact sum, which is within
//                the rounding of that sum either way;
//   tensor step: (NVFP4) the least-squares tensor scale sum(y p) / sum(p^2)
//                for the block step's bytes and codes, p = E4M3 x E2M1, the
//                sums in binary64 (per unit of 32 elements, per operand row,
//                rows in 256 contiguous ranges, the ranges in turn: a fixed
//                order, so the same input gives the same bits), rounded to
//                binary32, at least 2^-117, unchanged if sum(y p) <= 0;
//   schedule:    block step with the absmax tensor scale, then `iters`
//                times (tensor step, block step).
// One thread per unit of 32 contraction elements (16 for NVFP4 without
// rotation when K is not a multiple of 32), addressed as in noise.hip; MXFP4
// transposed inputs that the tiled transposing quantizer takes go there
// instead (quantize.hip: the same block step, one lane per block).
#include "fp4_device.h"
#include "mse_device.h"
#include "mxfp4_internal.h"

namespace mxfp4 {

struct MseArgs {
  const uint16_t* x;
  int64_t ldx;
  int64_t rows, K;
  uint8_t* codes;
  uint8_t* scales;
  const float* st;          // NVFP4 tensor scale (device)
  int64_t units;
  FastDiv div;
  int small, vec;
  double* unit_parts;       // NVFP4: 2 per unit, [rows][K / U]
};

template <int FMT, bool HAD, int AXIS, int U>
__global__ void __launch_bounds__(256) mse_block_kernel(MseArgs a) {
  constexpr int BS = (FMT == FMT_MX) ? 32 : 16;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= a.units) return;
  const float st = (FMT == FMT_NV) ? a.st[0] : 1.0f;
  const int64_t nu = a.K / U;
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
  uint32_t words[U / 8];
  uint32_t bytes[U / BS];
#pragma unroll
  for (int blk = 0; blk < U / BS; blk++) {
    uint32_t cw[BS / 8];
    bytes[blk] = mse_block<FMT, BS>(y + blk * BS, st, cw);
#pragma unroll
    for (int q = 0; q < BS / 8; q++) words[blk * (BS / 8) + q] = cw[q];
  }
  uint8_t* cdst = a.codes + i * (a.K / 2) + k0 / 2;
  if constexpr (U == 32) *(u32v4*)cdst = (u32v4){words[0], words[1], words[2], words[3]};
  else *(uint2*)cdst = make_uint2(words[0], words[1]);
  uint8_t* sdst = a.scales + i * (a.K / BS) + k0 / BS;
#pragma unroll
  for (int blk = 0; blk < U / BS; blk++) sdst[blk] = (uint8_t)bytes[blk];
  if constexpr (FMT == FMT_NV) {
    // this unit's terms of the least-squares tensor scale, elements in turn
    double un = 0.0, ud = 0.0;
#pragma unroll
    for (int blk = 0; blk < U / BS; blk++) {
      if ((bytes[blk] & 0x7Fu) == 0x7Fu) continue;
      const double sb = (double)e4m3_value(bytes[blk]);
#pragma unroll
      for (int q = 0; q < BS / 8; q++) {
        float g[8];
        decode8(words[blk * (BS / 8) + q], g);
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const double p = (double)g[j] * sb;
          un += (double)y[blk * BS + 8 * q + j] * p;
          ud += p * p;
        }
      }
    }
    double* up = a.unit_parts + 2 * (i * nu + b);
    up[0] = un;
    up[1] = ud;
  }
}

// Operand row sums of the unit terms, units in turn.
__global__ void __launch_bounds__(256) mse_row_kernel(const double* __restrict__ unit_parts, int64_t rows,
                                                      int64_t nu, double* __restrict__ row_parts) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  const double* up = unit_parts + 2 * i * nu;
  double rn = 0.0, rd = 0.0;
  for (int64_t b = 0; b < nu; b++) {
    rn += up[2 * b];
    rd += up[2 * b + 1];
  }
  row_parts[2 * i] = rn;
  row_parts[2 * i + 1] = rd;
}

// Rows in 256 contiguous ranges in turn, the ranges in turn; new tensor scale.
__global__ void __launch_bounds__(256) mse_tensor_kernel(const double* __restrict__ row_parts, int64_t rows,
                                                         float* __restrict__ st) {
  __shared__ double part[2][256];
  const int t = threadIdx.x;
  double sn = 0.0, sd = 0.0;
  for (int64_t i = (int64_t)t * rows / 256; i < (int64_t)(t + 1) * rows / 256; i++) {
    sn += row_parts[2 * i];
    sd += row_parts[2 * i + 1];
  }
  part[0][t] = sn;
  part[1][t] = sd;
  __syncthreads();
  if (t == 0) {
    double num = 0.0, den = 0.0;
    for (int r = 0; r < 256; r++) {
      num += part[0][r];
      den += part[1][r];
    }
    if (num > 0.0 && den > 0.0) {
      const float s = (float)(num / den);
      st[0] = s < 0x1p-117f ? 0x1p-117f : s;
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP4 with a fixed grid scale (the digest of "Bridging the Gap Between
// Promise and Performance for Microscaling FP4 Quantization", step 1: for
// MXFP4 with Hadamard rotations one fixed scale of the quantization grid
// serves every model; the value is the caller's alpha): each block's E8M0
// exponent is the smallest e with 6 * 2^e >= RN(alpha * absmax), then the
// absmax quantizer's round-to-nearest for that scale.  One thread per block of
// 32, addressed and loaded as in the MSE block kernel.
// ---------------------------------------------------------------------------
template <bool HAD, int AXIS>
__global__ void __launch_bounds__(256) grid_block_kernel(MseArgs a, float alpha) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= a.units) return;
  const int64_t nu = a.K / 32;
  int64_t i, b;
  if (a.small) {
    const uint32_t qd = fastdiv((uint32_t)u, a.div), rm = (uint32_t)u - qd * a.div.d;
    if (AXIS == 1) { i = qd; b = rm; } else { b = qd; i = rm; }
  } else if (AXIS == 1) {
    i = u / nu; b = u - i * nu;
  } else {
    b = u / a.rows; i = u - b * a.rows;
  }
  const int64_t k0 = b * 32;
  float y[32];
  if (AXIS == 1) {
    const uint16_t* src = a.x + i * a.ldx + k0;
    if (a.vec) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const u32v4 v = *(const u32v4*)(src + 8 * q);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          y[8 * q + 2 * j] = __uint_as_float(v[j] << 16);
          y[8 * q + 2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; j++) y[j] = __uint_as_float((uint32_t)src[j] << 16);
    }
  } else {
    const uint16_t* src = a.x + k0 * a.ldx + i;
#pragma unroll
    for (int j = 0; j < 32; j++) y[j] = __uint_as_float((uint32_t)src[(int64_t)j * a.ldx] << 16);
  }
  if constexpr (HAD) fwht32_inlane(y);
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 32; j++) m = max(m, __float_as_uint(y[j]) & 0x7FFFFFFFu);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  uint32_t byte = 0xFFu;
  if (m < 0x7F800000u) {
    const float scaled = alpha * __uint_as_float(m);
    const uint32_t sb = __float_as_uint(scaled);
    byte = sb >= 0x7F800000u ? 254u : mx_scale_byte_from_f32bits(sb);   // an overflowed product takes e = 127
#pragma unroll
    for (int q = 0; q < 4; q++) w[q] = cvt8(y + 8 * q, e8m0_as_cvt_scale(byte));
  }
  *(u32v4*)(a.codes + i * (a.K / 2) + k0 / 2) = (u32v4){w[0], w[1], w[2], w[3]};
  a.scales[i * (a.K / 32) + b] = (uint8_t)byte;
}

hipError_t launch_quantize_grid(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                                float alpha, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  // the row and tiled transposing quantizers take every input they can (they
  // differ from the plain quantizer only in the scale byte)
  if (launch_quantize_grid_fast(x, R, C, ldx, hadamard, axis, alpha, codes, scales, stream)) return hipGetLastError();
  const int64_t rows = axis == 1 ? R : C, K = axis == 1 ? C : R;
  MseArgs a{};
  a.x = x;
  a.ldx = ldx;
  a.rows = rows;
  a.K = K;
  a.codes = codes;
  a.scales = scales;
  a.units = rows * (K / 32);
  a.small = a.units < ((int64_t)1 << 31) ? 1 : 0;
  a.div = make_fastdiv(a.small ? (uint32_t)(axis == 1 ? K / 32 : rows) : 1u);
  a.vec = (((uintptr_t)x & 15) == 0 && ldx % 8 == 0) ? 1 : 0;
  const unsigned g = (unsigned)((a.units + 255) / 256);
  if (hadamard) {
    if (axis == 1) hipLaunchKernelGGL((grid_block_kernel<true, 1>), dim3(g), dim3(256), 0, stream, a, alpha);
    else hipLaunchKernelGGL((grid_block_kernel<true, 0>), dim3(g), dim3(256), 0, stream, a, alpha);
  } else {
    if (axis == 1) hipLaunchKernelGGL((grid_block_kernel<false, 1>), dim3(g), dim3(256), 0, stream, a, alpha);
    else hipLaunchKernelGGL((grid_block_kernel<false, 0>), dim3(g), dim3(256), 0, stream, a, alpha);
  }
  return hipGetLastError();
}

static int mse_unit(int fmt, int hadamard, int64_t K) {
  return (fmt == FMT_NV && !hadamard && K % 32 != 0) ? 16 : 32;
}

static size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

size_t quantize_mse_workspace_bytes(int fmt, int hadamard, int64_t R, int64_t C, int axis) {
  if (fmt != FMT_NV) return 0;
  const int64_t rows = axis == 1 ? R : C, K = axis == 1 ? C : R;
  const int64_t units = rows * (K / mse_unit(fmt, hadamard, K));
  return align16(quantize_workspace_bytes(fmt, R, C)) + align16((size_t)units * 16) + (size_t)rows * 16;
}

template <int FMT, bool HAD, int AXIS, int U>
static void launch_block_t(const MseArgs& a, hipStream_t s) {
  const int64_t g = (a.units + 255) / 256;
  hipLaunchKernelGGL((mse_block_kernel<FMT, HAD, AXIS, U>), dim3((unsigned)g), dim3(256), 0, s, a);
}

template <int FMT, bool HAD>
static void launch_block(const MseArgs& a, int axis, int u, hipStream_t s) {
  if (u == 16) {
    if constexpr (FMT == FMT_NV && !HAD) {
      if (axis == 1) launch_block_t<FMT, HAD, 1, 16>(a, s);
      else launch_block_t<FMT, HAD, 0, 16>(a, s);
    }
    return;
  }
  if (axis == 1) launch_block_t<FMT, HAD, 1, 32>(a, s);
  else launch_block_t<FMT, HAD, 0, 32>(a, s);
}

hipError_t launch_quantize_mse(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int hadamard,
                               int axis, int iters, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                               void* workspace, hipStream_t stream) {
  const int64_t rows = axis == 1 ? R : C, K = axis == 1 ? C : R;
  const int u = mse_unit(fmt, hadamard, K);
  MseArgs a;
  a.x = x;
  a.ldx = ldx;
  a.rows = rows;
  a.K = K;
  a.codes = codes;
  a.scales = scales;
  a.st = tensor_scale;
  a.units = rows * (K / u);
  a.small = a.units < ((int64_t)1 << 31) ? 1 : 0;
  a.div = make_fastdiv(a.small ? (uint32_t)(axis == 1 ? K / u : rows) : 1u);
  a.vec = (((uintptr_t)x & 15) == 0 && ldx % 8 == 0) ? 1 : 0;
  a.unit_parts = nullptr;
  double* row_parts = nullptr;
  if (fmt == FMT_NV) {
    uint8_t* w = (uint8_t*)workspace;
    launch_tensor_scale(x, R, C, ldx, hadamard, axis, tensor_scale, (uint32_t*)w, stream);
    a.unit_parts = (double*)(w + align16(quantize_workspace_bytes(fmt, R, C)));
    row_parts = (double*)((uint8_t*)a.unit_parts + align16((size_t)a.units * 16));
  }
  const int rounds = fmt == FMT_NV ? iters : 0;
  for (int r = 0; r <= rounds; r++) {
    if (r > 0) {
      hipLaunchKernelGGL(mse_row_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, a.unit_parts,
                         rows, K / u, row_parts);
      hipLaunchKernelGGL(mse_tensor_kernel, dim3(1), dim3(256), 0, stream, row_parts, rows, tensor_scale);
    }
    if (fmt == FMT_MX) {
      // transposed inputs go through the tiled transposing quantizer when it
      // takes them (same candidates, encodings and sums as the block kernel)
      if (launch_quantize_mse_mx_fast(x, R, C, ldx, hadamard, axis, codes, scales, stream)) continue;
      if (hadamard) launch_block<FMT_MX, true>(a, axis, u, stream);
      else launch_block<FMT_MX, false>(a, axis, u, stream);
    } else {
      if (hadamard) launch_block<FMT_NV, true>(a, axis, u, stream);
      else launch_block<FMT_NV, false>(a, axis, u, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace mxfp4
