// mse_device.h -- the block step of round-to-nearest quantization with
// MSE-fitted scales (the digest of "Bridging the Gap Between Promise and
// Performance for Microscaling FP4 Quantization", step 1), shared by the
// block kernels of mse.hip and the MXFP4 mode of the row and transposing
// quantizers.  The candidate windows, the tie rule and the summation order
// are described at the top of mse.hip.
#pragma once

#include "fp4_device.h"

namespace mxfp4 {

// Runs of 8 squared errors in turn, then the fixed pairing.
template <int BS>
__device__ __forceinline__ double mse_tree(const double (&d2)[BS]) {
  double s[BS / 8];
#pragma unroll
  for (int r = 0; r < BS / 8; r++) {
    s[r] = 0.0;
#pragma unroll
    for (int j = 0; j < 8; j++) s[r] += d2[8 * r + j];
  }
  if constexpr (BS == 16) return s[0] + s[1];
  else return (s[0] + s[1]) + (s[2] + s[3]);
}

// Codes of 8 consecutive elements (one 32-bit word) for the FP4 conversion
// scale sc: MXFP4 y with the E8M0 scale; NVFP4 RN(y inv) with unit scale.
__device__ __forceinline__ uint32_t cvt8(const float* v, float sc) {
  uint32_t p = 0;
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0], v[1], sc, 0);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2], v[3], sc, 1);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4], v[5], sc, 2);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6], v[7], sc, 3);
  return p;
}

// E2M1 codes of one word -> exact binary32 values.
__device__ __forceinline__ void decode8(uint32_t w, float* g) {
  const f32x2 g0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2 g1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2 g2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2 g3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  g[0] = g0[0]; g[1] = g0[1]; g[2] = g1[0]; g[3] = g1[1];
  g[4] = g2[0]; g[5] = g2[1]; g[6] = g3[0]; g[7] = g3[1];
}

// Block step for one block of BS elements y: scale byte and code words.
template <int FMT, int BS>
__device__ __forceinline__ uint32_t mse_block(const float* y, float st, uint32_t (&cw)[BS / 8]) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < BS; j++) m = max(m, __float_as_uint(y[j]) & 0x7FFFFFFFu);
  if (m >= 0x7F800000u) {
#pragma unroll
    for (int q = 0; q < BS / 8; q++) cw[q] = 0u;
    return FMT == FMT_MX ? 0xFFu : 0x7Fu;
  }
  double best = __builtin_inf();
  uint32_t best_byte = 0;
  if constexpr (FMT == FMT_MX) {
    const uint32_t b0 = mx_scale_byte_from_f32bits(m);
#pragma unroll 1
    for (int c = 0; c < 2; c++) {            // e0, e0 - 1 (lower exponents never win)
      if ((int)b0 - c < 0) break;
      const uint32_t byte = b0 - c;
      uint32_t w[BS / 8];
      double d2[BS];
      const double sc = (double)e8m0_value(byte);
#pragma unroll
      for (int q = 0; q < BS / 8; q++) {
        w[q] = cvt8(y + 8 * q, e8m0_as_cvt_scale(byte));
        float g[8];
        decode8(w[q], g);
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const double d = (double)y[8 * q + j] - (double)g[j] * sc;
          d2[8 * q + j] = d * d;
        }
      }
      const double E = mse_tree<BS>(d2);
      if (E < best) {
        best = E;
        best_byte = byte;
#pragma unroll
        for (int q = 0; q < BS / 8; q++) cw[q] = w[q];
      }
    }
    return best_byte;
  } else {
    const float amax = __uint_as_float(m);
    const float den = 6.0f * st;
    const uint32_t b0 = e4m3_round_up_byte(__fdiv_rn(amax, den));
    if (b0 == 0) {
      float z[BS];
#pragma unroll
      for (int j = 0; j < BS; j++) z[j] = __builtin_copysignf(0.0f, y[j]);
#pragma unroll
      for (int q = 0; q < BS / 8; q++) cw[q] = cvt8(z + 8 * q, 1.0f);
      return 0u;
    }
#pragma unroll 1
    for (int c = 0; c < 6; c++) {            // b0 .. b0 - 5 (lower bytes never win)
      if ((int)b0 - c < 1) break;
      const uint32_t byte = b0 - c;
      const float sb = e4m3_value(byte);
      const float inv = __fdiv_rn(1.0f, sb * st);
      const double sbst = (double)sb * (double)st;
      uint32_t w[BS / 8];
      double d2[BS];
#pragma unroll
      for (int q = 0; q < BS / 8; q++) {
        float xs[8];
#pragma unroll
        for (int j = 0; j < 8; j++) xs[j] = y[8 * q + j] * inv;
        w[q] = cvt8(xs, 1.0f);
        float g[8];
        decode8(w[q], g);
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const double d = (double)y[8 * q + j] - (double)g[j] * sbst;
          d2[8 * q + j] = d * d;
        }
      }
      const double E = mse_tree<BS>(d2);
      if (E < best) {
        best = E;
        best_byte = byte;
#pragma unroll
        for (int q = 0; q < BS / 8; q++) cw[q] = w[q];
      }
    }
    return best_byte;
  }
}

}  // namespace mxfp4
