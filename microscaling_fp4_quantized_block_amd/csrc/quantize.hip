// quantize.hip -- fused microscaling FP4 quantizer kernels for gfx950.
//
// The quantizer of the method: optional block-diagonal 32x32 Hadamard
// rotation ("Bridging the Gap Between Promise and Performance for
// Microscaling FP4 Quantization", abstract: block-wise Hadamard transforms
// computed online for activations and fused into weights), per-block absmax,
// shared scale (MXFP4 power-of-two E8M0 per 32, same abstract; NVFP4 E4M3 per
// 16 plus an FP32 tensor scale, "FP4 All the Way: Fully Quantized Training of
// LLMs", abstract, and the digest of the MR-GPTQ paper, step 1), rounding to
// E2M1 -- nearest on the forward pass, stochastic on the backward and update
// passes (FP4 All the Way, abstract) -- then nibble packing.
//
// The work is bound by HBM bandwidth (2 bytes in, ~0.53 bytes out per
// element), so the kernels are built around 16-byte coalesced loads, integer
// absmax on raw bit patterns, quad-level DPP reductions and the hardware
// FP4 conversion for round-to-nearest (v_cvt_scalef32_pk_fp4_*, which
// rounds x / 2^e to nearest-even with saturation).
//
// axis = 1 (rows): each lane owns 8 consecutive elements of one row, so a
//   32-block spans a quad of 4 lanes (16-block: 2 lanes).
// axis = 0 (transposed): each lane owns two adjacent columns and 32
//   consecutive rows, so both column blocks sit in one lane's registers and the
//   output (contraction along rows) is written as whole 16-byte block rows.
#include "fp4_device.h"
#include "mxfp4_internal.h"

namespace mxfp4 {

// ---------------------------------------------------------------------------
// Hadamard helpers.  Butterfly h: (x[i], x[i+h]) -> (x[i] + x[i+h], x[i] - x[i+h])
// for i & h == 0, strides 1, 2, 4, 8, 16 in that order, then multiply by
// RN_f32(1/sqrt(32)) = 0x3E3504F3.
// ---------------------------------------------------------------------------
constexpr uint32_t kHadamardScaleBits = 0x3E3504F3u;

// in-lane stages (h = 1, 2, 4) on 8 consecutive elements
__device__ __forceinline__ void fwht8_inlane(float v[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

// Full 32-point rotation of a block spread over a quad (lane p = lane & 3 holds
// block elements 8p .. 8p+7): stages 8 and 16 pair lane p with p^1 and p^2.
__device__ __forceinline__ void fwht32_quad(float v[8], uint32_t p) {
  fwht8_inlane(v);
  const bool up1 = (p & 1u) != 0, up2 = (p & 2u) != 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float o = dpp_xor1f(v[i]);
    v[i] = up1 ? (o - v[i]) : (v[i] + o);
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float o = dpp_xor2f(v[i]);
    v[i] = up2 ? (o - v[i]) : (v[i] + o);
  }
  const float c = __uint_as_float(kHadamardScaleBits);
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = v[i] * c;
}

// Full 32-point rotation of a column held in one lane (32 registers).
__device__ __forceinline__ void fwht32_inlane(float v[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; i++) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  const float c = __uint_as_float(kHadamardScaleBits);
#pragma unroll
  for (int i = 0; i < 32; i++) v[i] = v[i] * c;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// NVFP4 tensor scale from the tensor-amax partials.
// s_t = RN(amax / 2688), 1 for an all-zero tensor, kept >= 2^-117 so that
// s_b * s_t (s_b >= 2^-9) stays a normal binary32 number.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float nv_tensor_scale_from_amax_bits(uint32_t amax_bits) {
  float amax = __uint_as_float(amax_bits);
  if (!(amax > 0.0f)) return 1.0f;
  float st = __fdiv_rn(amax, 2688.0f);
  return st < 0x1p-117f ? 0x1p-117f : st;
}

// Every workgroup of the quantize pass reduces the (few hundred) partial
// maxima itself; workgroup 0 publishes s_t.  Runs before any other work.
__device__ float load_tensor_scale(const uint32_t* partials, int nparts, float* ts_out) {
  __shared__ float s_ts;
  if (threadIdx.x < 64) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += 64) m = max(m, partials[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    if (threadIdx.x == 0) {
      float st = nv_tensor_scale_from_amax_bits(m);
      s_ts = st;
      if (blockIdx.x == 0 && blockIdx.y == 0) ts_out[0] = st;
    }
  }
  __syncthreads();
  return s_ts;
}

// Per NVFP4 block: scale byte and the reciprocal used on the elements.
// den = RN(6 s_t), r = RN(amax / den), s_b = smallest E4M3 >= r,
// inv = RN(1 / RN(s_b * s_t)) (0 when s_b = 0).
__device__ __forceinline__ void nv_block_scale(float amax, float st, uint32_t& byte, float& inv) {
  float den = 6.0f * st;
  float r = __fdiv_rn(amax, den);
  byte = e4m3_round_up_byte(r);
  float d = e4m3_value(byte) * st;
  inv = byte ? __fdiv_rn(1.0f, d) : 0.0f;
}

// ---------------------------------------------------------------------------
// Tensor amax pass (NVFP4): largest finite |y| over the tensor, y the input
// or its block rotation.  Each workgroup writes one partial (binary32 bits;
// non-negative floats order like unsigned integers).
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ void __launch_bounds__(256) amax_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                   int64_t ldx, uint32_t* __restrict__ partials) {
  uint32_t m = 0;
  const int64_t cpr = (C + 7) / 8;                 // 8-element chunks per row (last may be partial)
  const int64_t total = R * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t i = t / cpr, q = t - i * cpr;
    const uint16_t* src = x + i * ldx + q * 8;
    uint32_t w[4];
    if (VEC) {
      u32v4 v = __builtin_nontemporal_load((const u32v4*)src);
      w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    } else {
      const int n = (C - q * 8) < 8 ? (int)(C - q * 8) : 8;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        uint32_t lo = (2 * j < n) ? src[2 * j] : 0u, hi = (2 * j + 1 < n) ? src[2 * j + 1] : 0u;
        w[j] = lo | (hi << 16);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
      if (lo < 0x7F80u) m = max(m, lo << 16);
      if (hi < 0x7F80u) m = max(m, hi << 16);
    }
  }
  __shared__ uint32_t red[4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int k = 1; k < (int)(blockDim.x >> 6); k++) r = max(r, red[k]);
    partials[blockIdx.x] = r;
  }
}

// Tensor amax with the rotation applied (NVFP4 + Hadamard), contraction along
// the rows' own axis (axis 1) or along columns (axis 0): one lane per
// 32-element contraction block, loaded element by element.
template <bool AXIS1>
__global__ void __launch_bounds__(256) amax_rot_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                       int64_t ldx, uint32_t* __restrict__ partials) {
  uint32_t m = 0;
  const int64_t rows = AXIS1 ? R : C, K = AXIS1 ? C : R;
  const int64_t bpr = K / 32;
  const int64_t total = rows * bpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t i = t / bpr, b = t - i * bpr;
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; j++) {
      const int64_t k = b * 32 + j;
      uint16_t h = AXIS1 ? x[i * ldx + k] : x[k * ldx + i];
      v[j] = __uint_as_float((uint32_t)h << 16);
    }
    fwht32_inlane(v);
#pragma unroll
    for (int j = 0; j < 32; j++) {
      uint32_t a = __float_as_uint(v[j]) & 0x7FFFFFFFu;
      if (a < 0x7F800000u) m = max(m, a);
    }
  }
  __shared__ uint32_t red[4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int k = 1; k < (int)(blockDim.x >> 6); k++) r = max(r, red[k]);
    partials[blockIdx.x] = r;
  }
}

// ---------------------------------------------------------------------------
// Row quantizer (axis = 1).  Lane = 8 consecutive elements of one row; the
// row's chunks are numbered t = i * (C/8) + q, so a Philox block (8
// elements of the output stream, counter = output index / 8) is exactly the
// lane's chunk: one Philox call per lane.
// ---------------------------------------------------------------------------
struct RowArgs {
  const uint16_t* x;
  int64_t R, C, ldx;
  uint8_t* codes;
  uint8_t* scales;
  uint64_t seed;
  const uint32_t* partials;
  int nparts;
  float* ts_out;
};

template <int FMT, int RND, bool HAD, bool VEC>
__global__ void __launch_bounds__(256) quant_rows_kernel(RowArgs a) {
  constexpr int LPB = (FMT == FMT_MX) ? 4 : 2;   // lanes per scale block
  float st = 1.0f;
  if (FMT == FMT_NV) st = load_tensor_scale(a.partials, a.nparts, a.ts_out);

  const int64_t cpr = a.C / 8;
  const int64_t total = a.R * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
  const uint32_t p = threadIdx.x & 3u;           // position in the quad

  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t i = t / cpr, q = t - i * cpr;
    const uint16_t* src = a.x + i * a.ldx + q * 8;
    uint32_t w[4];
    if (VEC) {
      u32v4 v = __builtin_nontemporal_load((const u32v4*)src);
      w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    } else {
#pragma unroll
      for (int j = 0; j < 4; j++) w[j] = (uint32_t)src[2 * j] | ((uint32_t)src[2 * j + 1] << 16);
    }

    float y[8];
    uint32_t amax_bits;   // binary32 pattern of the lane's largest |y|
    bool nonfinite;
    if (HAD) {
#pragma unroll
      for (int j = 0; j < 4; j++) { y[2 * j] = bf16lo(w[j]); y[2 * j + 1] = bf16hi(w[j]); }
      fwht32_quad(y, p);
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; j++) m = max(m, __float_as_uint(y[j]) & 0x7FFFFFFFu);
      amax_bits = m;
    } else {
      uint32_t m = pk_max_u16(pk_max_u16(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu),
                              pk_max_u16(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu));
      amax_bits = max(m & 0xFFFFu, m >> 16) << 16;
    }
    // block reduction across the lanes of the block
    amax_bits = max(amax_bits, dpp_xor1(amax_bits));
    if (LPB == 4) amax_bits = max(amax_bits, dpp_xor2(amax_bits));
    nonfinite = amax_bits >= 0x7F800000u;

    uint32_t byte, packed = 0;
    if (FMT == FMT_MX) {
      byte = nonfinite ? 0xFFu : mx_scale_byte_from_f32bits(amax_bits);
      if (!nonfinite) {
        if (RND == RND_RTN) {
          const float sc = e8m0_as_cvt_scale(byte);
          if (HAD) {
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[0], y[1], sc, 0);
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[2], y[3], sc, 1);
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[4], y[5], sc, 2);
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[6], y[7], sc, 3);
          } else {
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2, w[0]), sc, 0);
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2, w[1]), sc, 1);
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2, w[2]), sc, 2);
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2, w[3]), sc, 3);
          }
        } else {
          if (!HAD) {
#pragma unroll
            for (int j = 0; j < 4; j++) { y[2 * j] = bf16lo(w[j]); y[2 * j + 1] = bf16hi(w[j]); }
          }
          const float inv = mx_inv_scale(byte);
          const uint64_t g = (uint64_t)t;        // output index / 8
          u32x4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), 1u, 0u, k0, k1);
          const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
          for (int j = 0; j < 8; j++) {
            uint32_t rnd = (rw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            packed |= sr_code(y[j] * inv, rnd) << (4 * j);
          }
        }
      }
    } else {
      if (!HAD) {
#pragma unroll
        for (int j = 0; j < 4; j++) { y[2 * j] = bf16lo(w[j]); y[2 * j + 1] = bf16hi(w[j]); }
      }
      float inv = 0.0f;
      if (nonfinite) {
        byte = 0x7Fu;
      } else {
        nv_block_scale(__uint_as_float(amax_bits), st, byte, inv);
      }
      if (!nonfinite) {
        float xs[8];
#pragma unroll
        for (int j = 0; j < 8; j++) xs[j] = byte ? y[j] * inv : __builtin_copysignf(0.0f, y[j]);
        if (RND == RND_RTN) {
          packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, xs[0], xs[1], 1.0f, 0);
          packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, xs[2], xs[3], 1.0f, 1);
          packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, xs[4], xs[5], 1.0f, 2);
          packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, xs[6], xs[7], 1.0f, 3);
        } else {
          const uint64_t g = (uint64_t)t;
          u32x4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), 1u, 0u, k0, k1);
          const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
          for (int j = 0; j < 8; j++) {
            uint32_t rnd = (rw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            packed |= sr_code(xs[j], rnd) << (4 * j);
          }
        }
      }
    }
    // codes: 4 bytes per lane; scales: one byte per block, from its first lane
    *(uint32_t*)(a.codes + i * (a.C / 2) + q * 4) = packed;
    if ((q & (LPB - 1)) == 0) a.scales[i * (a.C / (8 * LPB)) + q / LPB] = (uint8_t)byte;
  }
}

// ---------------------------------------------------------------------------
// Transposing quantizer (axis = 0).  Output row c (input column c), contraction
// index r.  A lane holds columns 2l, 2l+1 of a 32-row slab as 32 packed
// bf16 pairs; a wave covers 128 columns.  Grid: x over 128-column groups,
// y over 32-row slabs.
// ---------------------------------------------------------------------------
struct ColArgs {
  const uint16_t* x;
  int64_t R, C, ldx;
  uint8_t* codes;
  uint8_t* scales;
  uint64_t seed;
  const uint32_t* partials;
  int nparts;
  float* ts_out;
};

template <int FMT, int RND, bool HAD, bool VEC>
__global__ void __launch_bounds__(256) quant_cols_kernel(ColArgs a) {
  float st = 1.0f;
  if (FMT == FMT_NV) st = load_tensor_scale(a.partials, a.nparts, a.ts_out);
  const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
  const int64_t R = a.R, C = a.C;

  const int64_t slab = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);   // 32-row slab
  const int64_t r0 = slab * 32;
  if (r0 >= R) return;
  const int nrows = (R - r0) >= 32 ? 32 : (int)(R - r0);             // 32, or 16 (NVFP4 tail)
  const int64_t c0 = ((int64_t)blockIdx.x * 64 + (threadIdx.x & 63)) * 2;
  if (c0 >= C) return;
  const bool two = (c0 + 1) < C;

  uint32_t w[32];
#pragma unroll
  for (int j = 0; j < 32; j++) {
    if (j < nrows) {
      const uint16_t* src = a.x + (r0 + j) * a.ldx + c0;
      if (VEC && two) w[j] = __builtin_nontemporal_load((const uint32_t*)src);
      else w[j] = (uint32_t)src[0] | (two ? ((uint32_t)src[1] << 16) : 0u);
    } else {
      w[j] = 0;
    }
  }

  const int ncols = two ? 2 : 1;
  for (int h = 0; h < ncols; h++) {
    const int64_t c = c0 + h;
    float y[32];
    uint32_t bits[32];
#pragma unroll
    for (int j = 0; j < 32; j++) {
      bits[j] = h ? (w[j] & 0xFFFF0000u) : (w[j] << 16);
      y[j] = __uint_as_float(bits[j]);
    }
    if (HAD) fwht32_inlane(y);

    constexpr int BS = (FMT == FMT_MX) ? 32 : 16;
    uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 32 / BS; b++) {
      if (b * BS >= nrows) break;
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < BS; j++) m = max(m, __float_as_uint(y[b * BS + j]) & 0x7FFFFFFFu);
      const bool nonfinite = m >= 0x7F800000u;
      uint32_t byte;
      float mul = 0.0f, cvt_sc = 1.0f;
      if (FMT == FMT_MX) {
        byte = nonfinite ? 0xFFu : mx_scale_byte_from_f32bits(m);
        mul = mx_inv_scale(byte);
        cvt_sc = e8m0_as_cvt_scale(byte);
      } else if (nonfinite) {
        byte = 0x7Fu;
      } else {
        nv_block_scale(__uint_as_float(m), st, byte, mul);
      }
      if (!nonfinite) {
        const int64_t kbase = r0 + b * BS;     // contraction index of the block's first element
#pragma unroll
        for (int j2 = 0; j2 < BS / 8; j2++) {
          // 8 elements = one 32-bit word of codes and one Philox block
          uint32_t word = 0;
          const int e0 = b * BS + j2 * 8;
          if (RND == RND_RTN) {
            if (FMT == FMT_MX) {
              word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[e0 + 0], y[e0 + 1], cvt_sc, 0);
              word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[e0 + 2], y[e0 + 3], cvt_sc, 1);
              word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[e0 + 4], y[e0 + 5], cvt_sc, 2);
              word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[e0 + 6], y[e0 + 7], cvt_sc, 3);
            } else {
              float xs[8];
#pragma unroll
              for (int j = 0; j < 8; j++) xs[j] = byte ? y[e0 + j] * mul : __builtin_copysignf(0.0f, y[e0 + j]);
              word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, xs[0], xs[1], 1.0f, 0);
              word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, xs[2], xs[3], 1.0f, 1);
              word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, xs[4], xs[5], 1.0f, 2);
              word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, xs[6], xs[7], 1.0f, 3);
            }
          } else {
            const uint64_t g = (uint64_t)((c * R + kbase + j2 * 8) >> 3);
            u32x4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), 0u, 0u, k0, k1);
            const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int j = 0; j < 8; j++) {
              float xs;
              if (FMT == FMT_MX) xs = y[e0 + j] * mul;
              else xs = byte ? y[e0 + j] * mul : __builtin_copysignf(0.0f, y[e0 + j]);
              uint32_t rnd = (rw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
              word |= sr_code(xs, rnd) << (4 * j);
            }
          }
          out[e0 / 8] = word;
        }
      }
      a.scales[c * (R / BS) + (r0 / BS) + b] = (uint8_t)byte;
    }
    // 16-byte stores when the output rows are 16-byte aligned (R % 32 == 0),
    // else 8-byte stores (NVFP4 with R % 32 == 16); codes is 16-byte aligned
    uint8_t* dst = a.codes + c * (R / 2) + r0 / 2;
    if (nrows == 32 && (R % 32) == 0) {
      *(uint4*)dst = make_uint4(out[0], out[1], out[2], out[3]);
    } else {
      *(uint2*)dst = make_uint2(out[0], out[1]);
      if (nrows == 32) *(uint2*)(dst + 8) = make_uint2(out[2], out[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called from the C ABI after argument checks).
// ---------------------------------------------------------------------------
static int grid_for(int64_t work_items, int per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  const int64_t cap = 256 * 64;     // enough resident waves; larger work loops
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

int amax_partials_count(int64_t R, int64_t C) {
  int64_t work = R * ((C + 7) / 8);
  int64_t g = (work + 255) / 256;
  return (int)(g > kAmaxPartials ? kAmaxPartials : (g < 1 ? 1 : g));
}

template <int FMT, int RND, bool HAD>
static void launch_rows(const RowArgs& a, bool vec, hipStream_t s) {
  int grid = grid_for(a.R * (a.C / 8), 256);
  if (vec) hipLaunchKernelGGL((quant_rows_kernel<FMT, RND, HAD, true>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((quant_rows_kernel<FMT, RND, HAD, false>), dim3(grid), dim3(256), 0, s, a);
}

template <int FMT, int RND, bool HAD>
static void launch_cols(const ColArgs& a, bool vec, hipStream_t s) {
  dim3 grid((unsigned)((a.C + 127) / 128), (unsigned)((a.R + 127) / 128));
  if (vec) hipLaunchKernelGGL((quant_cols_kernel<FMT, RND, HAD, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((quant_cols_kernel<FMT, RND, HAD, false>), grid, dim3(256), 0, s, a);
}

template <int FMT, int RND>
static void dispatch_had(bool had, int axis, const RowArgs& ra, const ColArgs& ca, bool vec, hipStream_t s) {
  if (axis == 1) {
    if (had) launch_rows<FMT, RND, true>(ra, vec, s);
    else launch_rows<FMT, RND, false>(ra, vec, s);
  } else {
    if (had) launch_cols<FMT, RND, true>(ca, vec, s);
    else launch_cols<FMT, RND, false>(ca, vec, s);
  }
}

hipError_t launch_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int rounding,
                           int hadamard, int axis, uint64_t seed, uint8_t* codes, uint8_t* scales,
                           float* tensor_scale, uint32_t* partials, hipStream_t stream) {
  int nparts = 0;
  if (fmt == FMT_NV) {
    if (hadamard) {
      int64_t blocks = (axis == 1 ? R * (C / 32) : C * (R / 32));
      nparts = (int)((blocks + 255) / 256);
      if (nparts > kAmaxPartials) nparts = kAmaxPartials;
      if (nparts < 1) nparts = 1;
      if (axis == 1) hipLaunchKernelGGL((amax_rot_kernel<true>), dim3(nparts), dim3(256), 0, stream, x, R, C, ldx, partials);
      else hipLaunchKernelGGL((amax_rot_kernel<false>), dim3(nparts), dim3(256), 0, stream, x, R, C, ldx, partials);
    } else {
      // the unrotated amax does not depend on the axis: scan the rows of [R, C]
      nparts = amax_partials_count(R, C);
      const bool v16 = (((uintptr_t)x & 15u) == 0) && (ldx % 8 == 0) && (C % 8 == 0);
      if (v16) hipLaunchKernelGGL((amax_kernel<true>), dim3(nparts), dim3(256), 0, stream, x, R, C, ldx, partials);
      else hipLaunchKernelGGL((amax_kernel<false>), dim3(nparts), dim3(256), 0, stream, x, R, C, ldx, partials);
    }
  }
  const bool vec = (((uintptr_t)x & 15u) == 0) && (ldx % 8 == 0);
  RowArgs ra{x, R, C, ldx, codes, scales, seed, partials, nparts, tensor_scale};
  ColArgs ca{x, R, C, ldx, codes, scales, seed, partials, nparts, tensor_scale};
  const bool vec_cols = (((uintptr_t)x & 3u) == 0) && (ldx % 2 == 0);
  const bool v = (axis == 1) ? vec : vec_cols;
  if (fmt == FMT_MX) {
    if (rounding == RND_RTN) dispatch_had<FMT_MX, RND_RTN>(hadamard, axis, ra, ca, v, stream);
    else dispatch_had<FMT_MX, RND_SR>(hadamard, axis, ra, ca, v, stream);
  } else {
    if (rounding == RND_RTN) dispatch_had<FMT_NV, RND_RTN>(hadamard, axis, ra, ca, v, stream);
    else dispatch_had<FMT_NV, RND_SR>(hadamard, axis, ra, ca, v, stream);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize: value = E2M1(code) * scale (NVFP4: RN(RN(E2M1 * s_b) * s_t)).
// Lane = 8 elements (one 32-bit word of codes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  // magnitude table {0, .5, 1, 1.5, 2, 3, 4, 6} in binary32 bit patterns
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float mag = e == 0 ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return (c & 8u) ? -mag : mag;
}

template <int FMT>
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ ts, int64_t rows, int64_t K,
                                                      float* __restrict__ y, int64_t ldy) {
  constexpr int BS = (FMT == FMT_MX) ? 32 : 16;
  const int64_t cpr = K / 8;
  const int64_t total = rows * cpr;
  const float st = (FMT == FMT_NV) ? ts[0] : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t i = t / cpr, q = t - i * cpr;
    const uint32_t word = *(const uint32_t*)(codes + i * (K / 2) + q * 4);
    const uint32_t sb = scales[i * (K / BS) + (q * 8) / BS];
    float* dst = y + i * ldy + q * 8;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint32_t c = (word >> (4 * j)) & 0xFu;
      float v;
      if (FMT == FMT_MX) v = e2m1_value(c) * e8m0_value(sb);
      else v = (e2m1_value(c) * e4m3_value(sb)) * st;
      dst[j] = v;
    }
  }
}

hipError_t launch_dequantize(int fmt, int64_t rows, int64_t K, const uint8_t* codes, const uint8_t* scales,
                             const float* ts, float* y, int64_t ldy, hipStream_t stream) {
  int grid = grid_for(rows * (K / 8), 256);
  if (fmt == FMT_MX)
    hipLaunchKernelGGL((dequant_kernel<FMT_MX>), dim3(grid), dim3(256), 0, stream, codes, scales, ts, rows, K, y, ldy);
  else
    hipLaunchKernelGGL((dequant_kernel<FMT_NV>), dim3(grid), dim3(256), 0, stream, codes, scales, ts, rows, K, y, ldy);
  return hipGetLastError();
}

}  // namespace mxfp4
