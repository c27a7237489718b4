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
// FP4 conversions: v_cvt_scalef32_pk_fp4_* for round-to-nearest (x / 2^e to
// nearest-even with saturation) and v_cvt_scalef32_sr_pk_fp4_f32 for
// stochastic rounding (sr_encode8 in fp4_device.h), fed by Philox4x32-10.
//
// axis = 1 (rows, quant_rows_kernel): each lane owns 8 consecutive elements
//   of one row, so a 32-block spans a quad of 4 lanes (16-block: 2 lanes).
// axis = 0 (transposed, quant_cols_tile_kernel): a workgroup stages a
//   256-row x 64-column tile in LDS, each lane then owns one column (so a
//   contraction block sits in one lane's registers), and the codes and scale
//   bytes go back through LDS so that the stores write whole row segments;
//   inputs that are not 16-byte aligned take quant_cols_kernel (a lane owns
//   two adjacent columns and 32 consecutive rows).
// STATS instantiations of the row and tiled kernels also add the signal and
// quantization-noise sums of the operand (mxfp4_quantize_noise).
#include "fp4_device.h"
#include "mse_device.h"
#include "mxfp4_internal.h"

namespace mxfp4 {

// ---------------------------------------------------------------------------
// Hadamard helpers (the butterfly order and the scale constant are given with
// fwht32_inlane in fp4_device.h).
// ---------------------------------------------------------------------------
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

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// NVFP4 tensor scale.
// s_t = RN(amax / 2688), 1 for an all-zero tensor, kept >= 2^-117 so that
// s_b * s_t (s_b >= 2^-9) stays a normal binary32 number.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float nv_tensor_scale_from_amax_bits(uint32_t amax_bits) {
  float amax = __uint_as_float(amax_bits);
  if (!(amax > 0.0f)) return 1.0f;
  float st = __fdiv_rn(amax, 2688.0f);
  return st < 0x1p-117f ? 0x1p-117f : st;
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
// Encoding of 8 consecutive contraction elements of one block into a 32-bit
// word of codes (element j in bits 4j+3..4j), given the block's scale byte.
//   MXFP4 RTN: the hardware FP4 conversion of y / 2^e (nearest-even,
//              saturating); bf16 inputs go in directly as packed pairs.
//   NVFP4:     x' = RN(y * inv) (+-0 for a zero scale), then RTN (conversion
//              with unit scale) or SR.
//   SR:        16 bits per element from the lane's Philox block rw, rounded
//              by the hardware stochastic FP4 conversion (sr_encode8).
// ---------------------------------------------------------------------------
template <int FMT, int RND, bool BF16IN>
__device__ __forceinline__ uint32_t encode8(const float y[8], const uint32_t w[4], uint32_t byte, float mul,
                                            const uint32_t rw[4]) {
  uint32_t packed = 0;
  if (FMT == FMT_MX && RND == RND_RTN) {
    const float sc = e8m0_as_cvt_scale(byte);
    if (BF16IN) {
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2, w[0]), sc, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2, w[1]), sc, 1);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2, w[2]), sc, 2);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2, w[3]), sc, 3);
    } else {
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[0], y[1], sc, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[2], y[3], sc, 1);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[4], y[5], sc, 2);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[6], y[7], sc, 3);
    }
    return packed;
  }
  float xs[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    if (FMT == FMT_MX) xs[j] = y[j] * mul;                      // exact: mul is a power of two
    else xs[j] = byte ? y[j] * mul : __builtin_copysignf(0.0f, y[j]);
  }
  if (RND == RND_RTN) {
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, xs[0], xs[1], 1.0f, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, xs[2], xs[3], 1.0f, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, xs[4], xs[5], 1.0f, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, xs[6], xs[7], 1.0f, 3);
  } else {
    packed = sr_encode8(xs, rw);
  }
  return packed;
}

// Scale byte and element multiplier of a block from its absmax bit pattern.
template <int FMT>
__device__ __forceinline__ void block_scale(uint32_t amax_bits, float st, uint32_t& byte, float& mul, bool& nonfinite) {
  nonfinite = amax_bits >= 0x7F800000u;
  if (FMT == FMT_MX) {
    byte = nonfinite ? 0xFFu : mx_scale_byte_from_f32bits(amax_bits);
    mul = mx_inv_scale(byte);
  } else if (nonfinite) {
    byte = 0x7Fu;
    mul = 0.0f;
  } else {
    nv_block_scale(__uint_as_float(amax_bits), st, byte, mul);
  }
}

// MXFP4 with a fixed grid scale alpha: the exponent is chosen for
// RN(alpha * absmax) (an overflowed product takes e = 127); a block holding a
// non-finite element keeps the NaN scale byte.  alpha = 1 gives block_scale.
__device__ __forceinline__ void grid_block_scale(uint32_t amax_bits, float alpha, uint32_t& byte, float& mul,
                                                 bool& nonfinite) {
  nonfinite = amax_bits >= 0x7F800000u;
  if (nonfinite) {
    byte = 0xFFu;
  } else {
    const uint32_t sb = __float_as_uint(alpha * __uint_as_float(amax_bits));
    byte = sb >= 0x7F800000u ? 254u : mx_scale_byte_from_f32bits(sb);
  }
  mul = mx_inv_scale(byte);
}

// ---------------------------------------------------------------------------
// Tensor amax pass (NVFP4): largest finite |y| over the tensor, y the input
// or its block rotation.  Each workgroup writes one partial (binary32 bits;
// non-negative floats order like unsigned integers); a one-workgroup
// finalize reduces them into s_t.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t block_max_u32(uint32_t m) {
  __shared__ uint32_t red[16];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = red[0];
  for (int k = 1; k < (int)(blockDim.x >> 6); k++) r = max(r, red[k]);
  return r;
}

__device__ __forceinline__ uint32_t finite_abs_max16(uint32_t w, uint32_t m) {
  const uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
  if (lo < 0x7F80u) m = max(m, lo << 16);
  if (hi < 0x7F80u) m = max(m, hi << 16);
  return m;
}

// Exact grid: a workgroup scans kAmaxChunksPerWG consecutive 16-byte chunks
// (eight per thread, all loads issued before the reductions) and writes one
// partial.  The rows may be padded: a chunk's row comes from a fast division.
template <bool VEC>
__global__ void __launch_bounds__(256) amax_kernel(const uint16_t* __restrict__ x, int64_t C, int64_t ldx,
                                                   FastDiv cpr, uint32_t total, uint32_t* __restrict__ partials) {
  constexpr int U = kAmaxChunksPerWG / 256;
  uint32_t m = 0;
  const uint32_t base = blockIdx.x * (uint32_t)kAmaxChunksPerWG + threadIdx.x;
  uint32_t w[U][4];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t t = base + u * 256u;
    w[u][0] = w[u][1] = w[u][2] = w[u][3] = 0;
    if (t < total) {
      const uint32_t i = fastdiv(t, cpr), q = t - i * cpr.d;
      const uint16_t* src = x + (int64_t)i * ldx + (int64_t)q * 8;
      if (VEC) {
        u32v4 v = __builtin_nontemporal_load((const u32v4*)src);
        w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2]; w[u][3] = v[3];
      } else {
        const int n = (C - (int64_t)q * 8) < 8 ? (int)(C - (int64_t)q * 8) : 8;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const uint32_t lo = (2 * j < n) ? src[2 * j] : 0u, hi = (2 * j + 1 < n) ? src[2 * j + 1] : 0u;
          w[u][j] = lo | (hi << 16);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; u++)
#pragma unroll
    for (int j = 0; j < 4; j++) m = finite_abs_max16(w[u][j], m);
  const uint32_t r = block_max_u32(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = r;
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
  const uint32_t r = block_max_u32(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = r;
}

__global__ void __launch_bounds__(1024) amax_finalize_kernel(const uint32_t* __restrict__ partials, int64_t nparts,
                                                             float* __restrict__ ts_out) {
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < nparts; i += blockDim.x) m = max(m, partials[i]);
  const uint32_t r = block_max_u32(m);
  if (threadIdx.x == 0) ts_out[0] = nv_tensor_scale_from_amax_bits(r);
}

// ---------------------------------------------------------------------------
// Row quantizer (axis = 1).  Lane = 8 consecutive elements of one row, chunk
// t = i * (C/8) + q; a 32-block is a quad of lanes (16-block: a pair).  The
// codes of chunk t are bytes 4t..4t+3 and its block's scale byte is t / (lanes
// per block), whatever the row length.  A Philox block (8 elements of the
// output stream, counter = output index / 8) is exactly one chunk.  Each
// thread keeps four 16-byte loads in flight.
// ---------------------------------------------------------------------------
struct RowArgs {
  const uint16_t* x;      // first element of the launch's slice
  int64_t ldx;
  FastDiv cpr;            // chunks per row
  uint32_t total;         // chunks in the slice (< 2^31)
  uint64_t tbase;         // global index of the slice's first chunk (Philox counter)
  uint8_t* codes;         // codes and scales of the slice's first chunk
  uint8_t* scales;
  uint64_t seed;
  const float* st;        // NVFP4 tensor scale (device), written by the finalize kernel
  double* parts;          // STATS: 3 binary64 sums per workgroup of the launch
  float alpha;            // GRID: the fixed grid scale
};

// LOAD bit 0: element loads (the input is not 16-byte aligned), else 16-byte
// loads.  LOAD bit 1: rows are padded (ldx > C), so a chunk's row comes from a
// division; else the slice is contiguous.
// STATS: also the signal and noise sums of the operand (noise_accum8; blocks
// with a NaN scale byte counted as left out), one triple per workgroup.
// GRID: MXFP4 round-to-nearest with the fixed grid scale a.alpha.
template <int FMT, int RND, bool HAD, int LOAD, bool STATS = false, bool GRID = false>
__global__ void __launch_bounds__(256) quant_rows_kernel(RowArgs a) {
  constexpr int LPB = (FMT == FMT_MX) ? 4 : 2;   // lanes per scale block
  constexpr int U = kRowChunksPerWG / 256;
  const float st = (FMT == FMT_NV) ? a.st[0] : 1.0f;
  const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
  const uint32_t p = threadIdx.x & 3u;           // position in the quad
  const uint32_t base = blockIdx.x * (uint32_t)kRowChunksPerWG + threadIdx.x;
  double s0 = 0.0, s1 = 0.0, left = 0.0;
  uint32_t w[U][4];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t t = base + u * 256u;
    w[u][0] = w[u][1] = w[u][2] = w[u][3] = 0;
    if (t < a.total) {
      const uint16_t* src;
      if (LOAD & 2) {
        const uint32_t i = fastdiv(t, a.cpr), q = t - i * a.cpr.d;
        src = a.x + (int64_t)i * a.ldx + (int64_t)q * 8;
      } else {
        src = a.x + (uint64_t)t * 8;
      }
      if (LOAD & 1) {
#pragma unroll
        for (int j = 0; j < 4; j++) w[u][j] = (uint32_t)src[2 * j] | ((uint32_t)src[2 * j + 1] << 16);
      } else {
        u32v4 v = __builtin_nontemporal_load((const u32v4*)src);
        w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2]; w[u][3] = v[3];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t t = base + u * 256u;
    if (t >= a.total) break;     // whole blocks leave together: total is a multiple of the lanes per block
    float y[8];
#pragma unroll
    for (int j = 0; j < 4; j++) { y[2 * j] = bf16lo(w[u][j]); y[2 * j + 1] = bf16hi(w[u][j]); }
    uint32_t amax_bits;
    if (HAD) {
      fwht32_quad(y, p);
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; j++) m = max(m, __float_as_uint(y[j]) & 0x7FFFFFFFu);
      amax_bits = m;
    } else {
      const uint32_t m = pk_max_u16(pk_max_u16(w[u][0] & 0x7FFF7FFFu, w[u][1] & 0x7FFF7FFFu),
                                    pk_max_u16(w[u][2] & 0x7FFF7FFFu, w[u][3] & 0x7FFF7FFFu));
      amax_bits = max(m & 0xFFFFu, m >> 16) << 16;
    }
    amax_bits = max(amax_bits, dpp_xor1(amax_bits));
    if (LPB == 4) amax_bits = max(amax_bits, dpp_xor2(amax_bits));
    uint32_t byte;
    float mul;
    bool nonfinite;
    if constexpr (GRID) grid_block_scale(amax_bits, a.alpha, byte, mul, nonfinite);
    else block_scale<FMT>(amax_bits, st, byte, mul, nonfinite);
    uint32_t rw[4] = {0, 0, 0, 0};
    if (RND == RND_SR && !nonfinite) {
      const uint64_t g = a.tbase + t;      // = output index / 8
      const u32x4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), 1u, 0u, k0, k1);
      rw[0] = r.x; rw[1] = r.y; rw[2] = r.z; rw[3] = r.w;
    }
    const uint32_t packed = nonfinite ? 0u : encode8<FMT, RND, !HAD>(y, w[u], byte, mul, rw);
    // outputs are not re-read by this kernel: stream them past the caches
    __builtin_nontemporal_store(packed, (uint32_t*)(a.codes + (uint64_t)t * 4));
    if ((p & (LPB - 1)) == 0) __builtin_nontemporal_store((uint8_t)byte, a.scales + t / LPB);
    if constexpr (STATS) {
      if (nonfinite) left += 8.0;
      else noise_accum8(y, packed, FMT == FMT_MX ? (double)e8m0_value(byte) : (double)e4m3_value(byte) * (double)st,
                        s0, s1);
    }
  }
  if constexpr (STATS) block_sum3(s0, s1, left, a.parts + 3 * (int64_t)blockIdx.x);
}

// ---------------------------------------------------------------------------
// Transposing quantizer (axis = 0), output row c = input column c, contraction
// index r.  Main kernel: a workgroup stages a 256-row x 64-column bf16 tile in
// LDS with 16-byte coalesced loads (8 rows x 128 B per wave instruction);
// wave w then owns rows 64w..64w+63 and lane l column l, so every contraction
// block of a column is in one lane's registers and the four waves write 128
// contiguous bytes of each output row.  Needs C % 8 == 0 and 16-byte aligned
// rows; the small kernel after it covers the rest.
// ---------------------------------------------------------------------------
struct ColArgs {
  const uint16_t* x;
  int64_t R, C, ldx;
  int64_t r_off;          // first input row of the launch (grid.y covers at most 65535 tiles)
  uint8_t* codes;
  uint8_t* scales;
  uint64_t seed;
  const float* st;
  double* parts;          // STATS (tile kernel): 3 binary64 sums per workgroup of the launch
  float alpha;            // GRID (tile kernel): the fixed grid scale
};

// GRID: MXFP4 with the fixed grid scale a.alpha.  MSE: MXFP4 with the
// MSE-fitted block scale (mse_block of mse_device.h on the lane's block).
template <int FMT, int RND, bool HAD, bool STATS = false, bool GRID = false, bool MSE = false>
__global__ void __launch_bounds__(256) quant_cols_tile_kernel(ColArgs a) {
  constexpr int BS = (FMT == FMT_MX) ? 32 : 16;
  __shared__ __attribute__((aligned(16))) uint16_t tile[256 * 64];   // 32 KB
  const float st = (FMT == FMT_NV) ? a.st[0] : 1.0f;
  const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
  const int64_t R = a.R, C = a.C;
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = a.r_off + (int64_t)blockIdx.y * 256;
  const int tid = threadIdx.x;

  // stage: thread loads 8 x 16 B (rows tid/8 + 32j, columns c0 + 8 (tid % 8)
  // ..).  Addresses are clamped into the tensor and the out-of-range chunks
  // zeroed afterwards, so all eight loads are issued back to back.
  {
    const int cc = (tid & 7) * 8;
    const bool col_ok = c0 + cc < C;
    const int64_t cl = col_ok ? c0 + cc : C - 8;
    u32v4 v[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int64_t row = r0 + (tid >> 3) + 32 * j;
      const int64_t rl = row < R ? row : R - 1;
      v[j] = __builtin_nontemporal_load((const u32v4*)(a.x + rl * a.ldx + cl));
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int row = (tid >> 3) + 32 * j;
      const bool ok = col_ok && (r0 + row < R);
      *(u32v4*)(tile + row * 64 + cc) = ok ? v[j] : (u32v4){0, 0, 0, 0};
    }
  }
  __syncthreads();

  const int w = tid >> 6, l = tid & 63;
  const int64_t c = c0 + l;
  const int64_t rw0 = r0 + 64 * w;                  // first contraction index of this wave
  const bool active = rw0 < R && c < C;
  double s0 = 0.0, s1 = 0.0, left = 0.0;
  // two halves of 32 rows (one MXFP4 block, two NVFP4 blocks); R is a
  // multiple of the block, so a half is whole, half-filled (NVFP4) or empty
  uint32_t out[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  uint32_t sbyte[2][32 / BS] = {};
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int64_t rh = rw0 + 32 * h;
    if (!active || rh >= R) break;
    float y[32];
#pragma unroll
    for (int j = 0; j < 32; j++) y[j] = __uint_as_float((uint32_t)tile[(64 * w + 32 * h + j) * 64 + l] << 16);
    if (HAD) fwht32_inlane(y);
    if constexpr (MSE) {             // MXFP4: the half is one block, the lane holds it
      sbyte[h][0] = mse_block<FMT_MX, 32>(y, 1.0f, out[h]);
      continue;
    }
#pragma unroll
    for (int b = 0; b < 32 / BS; b++) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < BS; j++) m = max(m, __float_as_uint(y[b * BS + j]) & 0x7FFFFFFFu);
      uint32_t byte;
      float mul;
      bool nonfinite;
      if constexpr (GRID) grid_block_scale(m, a.alpha, byte, mul, nonfinite);
      else block_scale<FMT>(m, st, byte, mul, nonfinite);
#pragma unroll
      for (int j2 = 0; j2 < BS / 8; j2++) {
        const int e0 = b * BS + j2 * 8;
        uint32_t rw[4] = {0, 0, 0, 0};
        if (RND == RND_SR && !nonfinite) {
          const uint64_t g = (uint64_t)((c * R + rh + e0) >> 3);
          const u32x4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), 0u, 0u, k0, k1);
          rw[0] = r.x; rw[1] = r.y; rw[2] = r.z; rw[3] = r.w;
        }
        const uint32_t dummy[4] = {0, 0, 0, 0};
        out[h][e0 / 8] = nonfinite ? 0u : encode8<FMT, RND, false>(y + e0, dummy, byte, mul, rw);
        // (rows past R are zeros with zero codes: they add nothing)
        if constexpr (STATS) {
          if (nonfinite) left += 8.0;
          else noise_accum8(y + e0, out[h][e0 / 8],
                            FMT == FMT_MX ? (double)e8m0_value(byte) : (double)e4m3_value(byte) * (double)st, s0, s1);
        }
      }
      sbyte[h][b] = byte;
    }
  }
  // The workgroup's codes form 64 output rows (columns c0..c0+63) of 128
  // contiguous bytes (contraction rows r0..r0+255), its scales 64 rows of
  // 256 / BS bytes.  Written straight from the lanes, every store of a wave
  // would touch 64 different lines; staged through LDS (the tile buffer, once
  // every wave has read it; code rows padded to 144 bytes and scale rows to
  // 20 so the lanes' accesses spread over the banks), each wave store of codes
  // writes eight whole 128-byte row segments and consecutive lanes write
  // consecutive scale bytes.
  constexpr int NSB = 256 / BS;                     // scale bytes per output row
  uint8_t* const stage = (uint8_t*)tile;
  uint8_t* const stage_s = stage + 64 * 144;
  __syncthreads();
  if (active) {
    *(u32v4*)(stage + l * 144 + 32 * w) = (u32v4){out[0][0], out[0][1], out[0][2], out[0][3]};
#pragma unroll
    for (int b = 0; b < 32 / BS; b++) stage_s[l * 20 + (64 * w) / BS + b] = (uint8_t)sbyte[0][b];
    if (rw0 + 32 < R) {
      *(u32v4*)(stage + l * 144 + 32 * w + 16) = (u32v4){out[1][0], out[1][1], out[1][2], out[1][3]};
#pragma unroll
      for (int b = 0; b < 32 / BS; b++) stage_s[l * 20 + (64 * w + 32) / BS + b] = (uint8_t)sbyte[1][b];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NSB / 4; i++) {
    const int q = tid + 256 * i;
    const int row = q / NSB, col = q % NSB;
    const int64_t cc = c0 + row, rb = r0 / BS + col;  // output row, block index
    if (cc < C && rb * BS < R) a.scales[cc * (R / BS) + rb] = stage_s[row * 20 + col];
  }
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int q = tid + 256 * i;
    const int row = q >> 3, ch = q & 7;
    const int64_t cc = c0 + row, rr = r0 + 32 * ch;    // output row, first contraction index
    if (cc >= C || rr >= R) continue;
    const u32v4 v = *(const u32v4*)(stage + row * 144 + 16 * ch);
    uint8_t* dst = a.codes + cc * (R / 2) + rr / 2;
    if ((R - rr) >= 32 && (R % 32) == 0) {
      __builtin_nontemporal_store(v, (u32v4*)dst);
    } else {
      *(uint2*)dst = make_uint2(v[0], v[1]);
      if ((R - rr) >= 32) *(uint2*)(dst + 8) = make_uint2(v[2], v[3]);
    }
  }
  if constexpr (STATS) block_sum3(s0, s1, left, a.parts + 3 * ((int64_t)blockIdx.y * gridDim.x + blockIdx.x));
}

// Small transposing kernel for ragged or unaligned inputs: a lane holds
// columns 2l, 2l+1 of a 32-row slab (32 loads of one 32-bit pair each).
template <int FMT, int RND, bool HAD, bool VEC>
__global__ void __launch_bounds__(256) quant_cols_kernel(ColArgs a) {
  const float st = (FMT == FMT_NV) ? a.st[0] : 1.0f;
  const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
  const int64_t R = a.R, C = a.C;
  constexpr int BS = (FMT == FMT_MX) ? 32 : 16;

  const int64_t slab = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);   // 32-row slab
  const int64_t r0 = a.r_off + slab * 32;
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
#pragma unroll
    for (int j = 0; j < 32; j++) y[j] = __uint_as_float(h ? (w[j] & 0xFFFF0000u) : (w[j] << 16));
    if (HAD) fwht32_inlane(y);
    uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 32 / BS; b++) {
      if (b * BS >= nrows) break;
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < BS; j++) m = max(m, __float_as_uint(y[b * BS + j]) & 0x7FFFFFFFu);
      uint32_t byte;
      float mul;
      bool nonfinite;
      block_scale<FMT>(m, st, byte, mul, nonfinite);
#pragma unroll
      for (int j2 = 0; j2 < BS / 8; j2++) {
        const int e0 = b * BS + j2 * 8;
        uint32_t rw[4] = {0, 0, 0, 0};
        if (RND == RND_SR && !nonfinite) {
          const uint64_t g = (uint64_t)((c * R + r0 + e0) >> 3);
          const u32x4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), 0u, 0u, k0, k1);
          rw[0] = r.x; rw[1] = r.y; rw[2] = r.z; rw[3] = r.w;
        }
        const uint32_t dummy[4] = {0, 0, 0, 0};
        out[e0 / 8] = nonfinite ? 0u : encode8<FMT, RND, false>(y + e0, dummy, byte, mul, rw);
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
static int grid_for(int64_t work_items, int per_block, int64_t cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

// Each launcher returns the number of workgroups it launched (the STATS
// partial triples it wrote); with launch = false it only counts them.
template <int FMT, int RND, bool HAD, bool STATS, bool GRID = false>
static int64_t launch_rows(const RowArgs& a, int load, bool launch, hipStream_t s) {
  const int grid = (int)(((uint64_t)a.total + kRowChunksPerWG - 1) / kRowChunksPerWG);
  if (!launch) return grid;
  switch (load) {
    case 0: hipLaunchKernelGGL((quant_rows_kernel<FMT, RND, HAD, 0, STATS, GRID>), dim3(grid), dim3(256), 0, s, a); break;
    case 1: hipLaunchKernelGGL((quant_rows_kernel<FMT, RND, HAD, 1, STATS, GRID>), dim3(grid), dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((quant_rows_kernel<FMT, RND, HAD, 2, STATS, GRID>), dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((quant_rows_kernel<FMT, RND, HAD, 3, STATS, GRID>), dim3(grid), dim3(256), 0, s, a); break;
  }
  return grid;
}

// STATS only with the tiled kernel (the caller sends the other inputs
// through quantize, then the separate noise pass).
// GRID and MSE only with the tiled kernel (the caller checks).
template <int FMT, int RND, bool HAD, bool STATS, bool GRID = false, bool MSE = false>
static int64_t launch_cols(ColArgs a, bool tiled, bool vec, bool launch, hipStream_t s) {
  // grid.y is limited to 65535: larger inputs go in slabs of rows
  const int64_t rows_per = tiled ? 256 : 128;
  const int64_t slab = 65535 * rows_per;
  int64_t n = 0;
  for (int64_t r = 0; r < a.R; r += slab) {
    a.r_off = r;
    const int64_t nr = (a.R - r) < slab ? (a.R - r) : slab;
    const int64_t cols_per = tiled ? 64 : 128;
    dim3 grid((unsigned)((a.C + cols_per - 1) / cols_per), (unsigned)((nr + rows_per - 1) / rows_per));
    if (launch) {
      if (tiled) hipLaunchKernelGGL((quant_cols_tile_kernel<FMT, RND, HAD, STATS, GRID, MSE>), grid, dim3(256), 0, s, a);
      else if constexpr (!GRID && !MSE) {
        if (vec) hipLaunchKernelGGL((quant_cols_kernel<FMT, RND, HAD, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((quant_cols_kernel<FMT, RND, HAD, false>), grid, dim3(256), 0, s, a);
      }
    }
    const int64_t wgs = (int64_t)grid.x * grid.y;
    n += wgs;
    if (STATS && a.parts) a.parts += 3 * wgs;   // (null when only counting)
  }
  return n;
}

// Chunk ranges of one launch stay below 2^31 so the kernels index in 32 bits.
constexpr uint64_t kSliceChunks = (uint64_t)1 << 30;

template <int FMT, int RND, bool HAD, bool STATS, bool GRID = false>
static int64_t launch_rows_sliced(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, bool aligned16,
                                  uint64_t seed, uint8_t* codes, uint8_t* scales, const float* st, double* parts,
                                  bool launch, hipStream_t s, float alpha = 1.0f) {
  constexpr int LPB = (FMT == FMT_MX) ? 4 : 2;
  const uint64_t cpr = (uint64_t)C / 8;
  RowArgs a{};
  a.ldx = ldx;
  a.seed = seed;
  a.st = st;
  a.parts = parts;
  a.alpha = alpha;
  int64_t n = 0;
  auto go = [&](int load) {
    const int64_t g = launch_rows<FMT, RND, HAD, STATS, GRID>(a, load, launch, s);
    n += g;
    if (STATS && a.parts) a.parts += 3 * g;   // (null when only counting)
  };
  const int elem = aligned16 ? 0 : 1;
  auto packed_range = [&](const uint16_t* xr, uint64_t t0, uint64_t m_all) {
    // a contiguous range of m_all chunks starting at global chunk t0
    for (uint64_t off = 0; off < m_all; off += kSliceChunks) {
      const uint64_t m = (m_all - off) < kSliceChunks ? (m_all - off) : kSliceChunks;
      a.x = xr + off * 8;
      a.cpr = make_fastdiv(1);
      a.total = (uint32_t)m;
      a.tbase = t0 + off;
      a.codes = codes + (t0 + off) * 4;
      a.scales = scales + (t0 + off) / LPB;
      go(elem);
    }
  };
  if (ldx == C || R == 1) {
    packed_range(x, 0, (uint64_t)R * cpr);
  } else if (cpr < kSliceChunks) {
    const int64_t rows_per = (int64_t)(kSliceChunks / cpr);
    for (int64_t r = 0; r < R; r += rows_per) {
      const int64_t nr = (R - r) < rows_per ? (R - r) : rows_per;
      a.x = x + r * ldx;
      a.cpr = make_fastdiv((uint32_t)cpr);
      a.total = (uint32_t)((uint64_t)nr * cpr);
      a.tbase = (uint64_t)r * cpr;
      a.codes = codes + a.tbase * 4;
      a.scales = scales + a.tbase / LPB;
      go(2 | elem);
    }
  } else {
    for (int64_t r = 0; r < R; r++) packed_range(x + r * ldx, (uint64_t)r * cpr, cpr);
  }
  return n;
}

template <int FMT, int RND, bool HAD, bool STATS>
static int64_t launch_one(int axis, const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint64_t seed,
                          uint8_t* codes, uint8_t* scales, const float* st, double* parts, hipStream_t s) {
  const bool aligned16 = (((uintptr_t)x & 15u) == 0) && (ldx % 8 == 0);
  if (axis == 1)
    return launch_rows_sliced<FMT, RND, HAD, STATS>(x, R, C, ldx, aligned16, seed, codes, scales, st, parts, true, s);
  ColArgs ca{x, R, C, ldx, 0, codes, scales, seed, st, parts, 1.0f};
  const bool tiled = aligned16 && (C % 8 == 0);
  const bool vec = (((uintptr_t)x & 3u) == 0) && (ldx % 2 == 0);
  return launch_cols<FMT, RND, HAD, STATS>(ca, tiled, vec, true, s);
}

template <int FMT, int RND, bool STATS = false>
static int64_t launch_had(bool had, int axis, const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint64_t seed,
                          uint8_t* codes, uint8_t* scales, const float* st, hipStream_t s, double* parts = nullptr) {
  if (had) return launch_one<FMT, RND, true, STATS>(axis, x, R, C, ldx, seed, codes, scales, st, parts, s);
  return launch_one<FMT, RND, false, STATS>(axis, x, R, C, ldx, seed, codes, scales, st, parts, s);
}

// Tensor amax of an NVFP4 input into s_t (device): partial maxima, then the
// one-workgroup finalize.
void launch_tensor_scale(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                                float* tensor_scale, uint32_t* partials, hipStream_t s) {
  int64_t nparts = 0;
  if (hadamard) {
    const int64_t blocks = (axis == 1 ? R * (C / 32) : C * (R / 32));
    nparts = grid_for(blocks, 256, kAmaxRotPartials);
    if (axis == 1) hipLaunchKernelGGL((amax_rot_kernel<true>), dim3((unsigned)nparts), dim3(256), 0, s, x, R, C, ldx, partials);
    else hipLaunchKernelGGL((amax_rot_kernel<false>), dim3((unsigned)nparts), dim3(256), 0, s, x, R, C, ldx, partials);
  } else {
    // the unrotated amax does not depend on the axis: scan the rows of [R, C]
    // in ranges of whole rows below 2^31 chunks (a row of more chunks than
    // that is scanned alone, as a contiguous range); each range writes its
    // own run of partials
    const uint64_t cpr = ((uint64_t)C + 7) / 8;
    const bool vec = (((uintptr_t)x & 15u) == 0) && (ldx % 8 == 0) && (C % 8 == 0);
    auto scan = [&](const uint16_t* xr, int64_t nr, int64_t c, uint64_t per_row) {
      const uint32_t total = (uint32_t)((uint64_t)nr * per_row);
      const unsigned grid = (unsigned)((total + kAmaxChunksPerWG - 1) / kAmaxChunksPerWG);
      const FastDiv f = make_fastdiv((uint32_t)per_row);
      if (vec) hipLaunchKernelGGL((amax_kernel<true>), dim3(grid), dim3(256), 0, s, xr, c, ldx, f, total, partials + nparts);
      else hipLaunchKernelGGL((amax_kernel<false>), dim3(grid), dim3(256), 0, s, xr, c, ldx, f, total, partials + nparts);
      nparts += grid;
    };
    if (cpr < kSliceChunks) {
      const int64_t rows_per = (int64_t)(kSliceChunks / cpr);
      for (int64_t r = 0; r < R; r += rows_per) scan(x + r * ldx, (R - r) < rows_per ? (R - r) : rows_per, C, cpr);
    } else {
      for (int64_t r = 0; r < R; r++)
        for (uint64_t off = 0; off < cpr; off += kSliceChunks) {
          const uint64_t m = (cpr - off) < kSliceChunks ? (cpr - off) : kSliceChunks;
          const int64_t c = (int64_t)(m * 8) < (C - (int64_t)off * 8) ? (int64_t)(m * 8) : (C - (int64_t)off * 8);
          scan(x + r * ldx + off * 8, 1, c, m);
        }
    }
  }
  hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(1024), 0, s, partials, nparts, tensor_scale);
}

// MXFP4 with a fixed grid scale through the row and tiled transposing
// quantizers (the block kernel of mse.hip covers the rest); false when the
// input takes neither.
template <bool HAD>
static bool launch_grid_fast_t(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int axis, float alpha,
                               uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const bool aligned16 = (((uintptr_t)x & 15u) == 0) && (ldx % 8 == 0);
  if (axis == 1) {
    launch_rows_sliced<FMT_MX, RND_RTN, HAD, false, true>(x, R, C, ldx, aligned16, 0, codes, scales, nullptr,
                                                          nullptr, true, s, alpha);
    return true;
  }
  if (!(aligned16 && C % 8 == 0)) return false;
  ColArgs ca{x, R, C, ldx, 0, codes, scales, 0, nullptr, nullptr, alpha};
  launch_cols<FMT_MX, RND_RTN, HAD, false, true>(ca, true, true, true, s);
  return true;
}

bool launch_quantize_grid_fast(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                               float alpha, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (hadamard) return launch_grid_fast_t<true>(x, R, C, ldx, axis, alpha, codes, scales, s);
  return launch_grid_fast_t<false>(x, R, C, ldx, axis, alpha, codes, scales, s);
}

// MXFP4 with MSE-fitted block scales, transposed (axis 0), through the tiled
// transposing quantizer: the block kernel of mse.hip reads a column block
// element by element, the tile kernel stages it through LDS with full-line
// loads (same block step, same bits).  Along rows the block kernel already
// reads whole lines and is bound by its binary64 arithmetic: a quad-of-lanes
// version in the row quantizer measured the same 44 us on a config-3 weight.
// False when the input is not the tiled kernel's.
template <bool HAD>
static bool launch_mse_fast_t(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int axis, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const bool aligned16 = (((uintptr_t)x & 15u) == 0) && (ldx % 8 == 0);
  if (axis == 1 || !(aligned16 && C % 8 == 0)) return false;
  ColArgs ca{x, R, C, ldx, 0, codes, scales, 0, nullptr, nullptr, 1.0f};
  launch_cols<FMT_MX, RND_RTN, HAD, false, false, true>(ca, true, true, true, s);
  return true;
}

bool launch_quantize_mse_mx_fast(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (hadamard) return launch_mse_fast_t<true>(x, R, C, ldx, axis, codes, scales, s);
  return launch_mse_fast_t<false>(x, R, C, ldx, axis, codes, scales, s);
}

// ---------------------------------------------------------------------------
// Q-EMA weight quantizer ("Oscillation-Reduced MXFP4 Training for Vision
// Transformers", abstract, names Q-EMA without giving its rule; the reading
// here: the forward pass quantizes an exponential moving average of the latent
// weights).  One pass: m <- RN(RN(beta m) + RN(c w)) with c = RN(1 - beta) in
// binary32 (no fused multiply-add), the new m stored back, then MXFP4
// round-to-nearest of the new m along its rows (block Hadamard first with HAD).
// Lane = 8 consecutive elements of a row: a 16-byte load of w, two of m and
// two 16-byte stores of the new m; a 32-block is a quad of lanes, as in the
// row quantizer.  HBM bytes per element: 2 (w) + 4 + 4 (m in, out) + 0.5 + 1/32.
// ---------------------------------------------------------------------------
struct QemaArgs {
  const uint16_t* w;
  int64_t ldw;
  float* m;
  int64_t lde;
  FastDiv cpr;            // chunks (8 elements) per row
  uint32_t total;         // chunks in the tensor (< 2^31)
  float beta, c;
  uint8_t* codes;
  uint8_t* scales;
};

template <bool HAD, bool PADDED>
__global__ void __launch_bounds__(256) qema_kernel(QemaArgs a) {
  constexpr int U = 2;
  const uint32_t p = threadIdx.x & 3u;
  const uint32_t base = blockIdx.x * (uint32_t)(256 * U) + threadIdx.x;
  uint32_t wv[U][4];
  f32x4 mv[U][2];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t t = base + u * 256u;
    if (t >= a.total) continue;
    const uint16_t* ws;
    float* ms;
    if (PADDED) {
      const uint32_t i = fastdiv(t, a.cpr), q = t - i * a.cpr.d;
      ws = a.w + (int64_t)i * a.ldw + (int64_t)q * 8;
      ms = a.m + (int64_t)i * a.lde + (int64_t)q * 8;
    } else {
      ws = a.w + (uint64_t)t * 8;
      ms = a.m + (uint64_t)t * 8;
    }
    const u32v4 v = __builtin_nontemporal_load((const u32v4*)ws);
    wv[u][0] = v[0]; wv[u][1] = v[1]; wv[u][2] = v[2]; wv[u][3] = v[3];
    mv[u][0] = __builtin_nontemporal_load((const f32x4*)ms);
    mv[u][1] = __builtin_nontemporal_load((const f32x4*)(ms + 4));
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t t = base + u * 256u;
    if (t >= a.total) break;     // whole blocks leave together (total is a multiple of 4)
    float y[8];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float w0 = bf16lo(wv[u][j]), w1 = bf16hi(wv[u][j]);
      const float m0 = mv[u][j >> 1][2 * (j & 1)], m1 = mv[u][j >> 1][2 * (j & 1) + 1];
      y[2 * j] = a.beta * m0 + a.c * w0;          // built without FP contraction: three roundings
      y[2 * j + 1] = a.beta * m1 + a.c * w1;
    }
    float* ms;
    if (PADDED) {
      const uint32_t i = fastdiv(t, a.cpr), q = t - i * a.cpr.d;
      ms = a.m + (int64_t)i * a.lde + (int64_t)q * 8;
    } else {
      ms = a.m + (uint64_t)t * 8;
    }
    __builtin_nontemporal_store((f32x4){y[0], y[1], y[2], y[3]}, (f32x4*)ms);
    __builtin_nontemporal_store((f32x4){y[4], y[5], y[6], y[7]}, (f32x4*)(ms + 4));
    if (HAD) fwht32_quad(y, p);
    uint32_t am = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) am = max(am, __float_as_uint(y[j]) & 0x7FFFFFFFu);
    am = max(am, dpp_xor1(am));
    am = max(am, dpp_xor2(am));
    uint32_t packed = 0, byte = 0xFFu;
    if (am < 0x7F800000u) {
      byte = mx_scale_byte_from_f32bits(am);
      const float sc = e8m0_as_cvt_scale(byte);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[0], y[1], sc, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[2], y[3], sc, 1);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[4], y[5], sc, 2);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[6], y[7], sc, 3);
    }
    __builtin_nontemporal_store(packed, (uint32_t*)(a.codes + (uint64_t)t * 4));
    if (p == 0) __builtin_nontemporal_store((uint8_t)byte, a.scales + t / 4);
  }
}

hipError_t launch_qema(const uint16_t* w, int64_t R, int64_t C, int64_t ldw, float* m, int64_t lde, float beta,
                       int hadamard, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  QemaArgs a;
  a.w = w;
  a.ldw = ldw;
  a.m = m;
  a.lde = lde;
  a.cpr = make_fastdiv((uint32_t)(C / 8));
  a.total = (uint32_t)(R * (C / 8));
  a.beta = beta;
  a.c = 1.0f - beta;
  a.codes = codes;
  a.scales = scales;
  const bool padded = ldw != C || lde != C;
  const unsigned grid = (unsigned)((a.total + 511) / 512);
  if (hadamard) {
    if (padded) hipLaunchKernelGGL((qema_kernel<true, true>), dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((qema_kernel<true, false>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (padded) hipLaunchKernelGGL((qema_kernel<false, true>), dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((qema_kernel<false, false>), dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

size_t quantize_workspace_bytes(int fmt, int64_t R, int64_t C) {
  if (fmt != FMT_NV) return 0;
  // partials written by launch_tensor_scale's unrotated scan, range by range
  const uint64_t cpr = ((uint64_t)C + 7) / 8;
  const uint64_t per = kAmaxChunksPerWG;
  uint64_t n = 0;
  if (R > 0 && cpr > 0) {
    if (cpr < kSliceChunks) {
      const uint64_t rows_per = kSliceChunks / cpr, full = (uint64_t)R / rows_per, rem = (uint64_t)R % rows_per;
      n = full * ((rows_per * cpr + per - 1) / per) + (rem ? (rem * cpr + per - 1) / per : 0);
    } else {
      const uint64_t m_full = cpr / kSliceChunks, m_rem = cpr % kSliceChunks;
      n = (uint64_t)R * (m_full * ((kSliceChunks + per - 1) / per) + (m_rem ? (m_rem + per - 1) / per : 0));
    }
  }
  if (n < (uint64_t)kAmaxRotPartials) n = kAmaxRotPartials;
  return (size_t)n * sizeof(uint32_t);
}

hipError_t launch_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int rounding,
                           int hadamard, int axis, uint64_t seed, uint8_t* codes, uint8_t* scales,
                           float* tensor_scale, uint32_t* partials, hipStream_t stream) {
  if (fmt == FMT_NV) launch_tensor_scale(x, R, C, ldx, hadamard, axis, tensor_scale, partials, stream);
  if (fmt == FMT_MX) {
    if (rounding == RND_RTN) launch_had<FMT_MX, RND_RTN>(hadamard, axis, x, R, C, ldx, seed, codes, scales, tensor_scale, stream);
    else launch_had<FMT_MX, RND_SR>(hadamard, axis, x, R, C, ldx, seed, codes, scales, tensor_scale, stream);
  } else {
    if (rounding == RND_RTN) launch_had<FMT_NV, RND_RTN>(hadamard, axis, x, R, C, ldx, seed, codes, scales, tensor_scale, stream);
    else launch_had<FMT_NV, RND_SR>(hadamard, axis, x, R, C, ldx, seed, codes, scales, tensor_scale, stream);
  }
  return hipGetLastError();
}

// Quantize with the signal / noise sums (mxfp4_quantize_noise).  The row and
// the tiled transposing kernels add the sums as they encode; inputs that take
// the small transposing kernel are quantized, then summed by the separate
// noise pass (the same sums).
int64_t quantize_noise_parts(int fmt, int hadamard, int64_t R, int64_t C, int axis) {
  if (R == 0 || C == 0) return 1;
  int64_t n;
  if (axis == 1) {
    // the launch plan depends on whether the rows are packed: count both
    const int64_t a = launch_rows_sliced<FMT_MX, RND_RTN, false, true>(nullptr, R, C, C, true, 0, nullptr, nullptr,
                                                                      nullptr, nullptr, false, nullptr);
    const int64_t b = launch_rows_sliced<FMT_MX, RND_RTN, false, true>(nullptr, R, C, C + 8, true, 0, nullptr,
                                                                      nullptr, nullptr, nullptr, false, nullptr);
    n = a > b ? a : b;
  } else {
    ColArgs ca{nullptr, R, C, C, 0, nullptr, nullptr, 0, nullptr, nullptr, 1.0f};
    const int64_t a = launch_cols<FMT_MX, RND_RTN, false, true>(ca, true, true, false, nullptr);
    const int64_t b = (int64_t)(noise_workspace_bytes(fmt, hadamard, C, R) / (3 * sizeof(double)));
    n = a > b ? a : b;
  }
  return n < 1 ? 1 : n;
}

hipError_t launch_quantize_noise(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int rounding,
                                 int hadamard, int axis, uint64_t seed, uint8_t* codes, uint8_t* scales,
                                 float* tensor_scale, uint32_t* amax_partials, double* stats, double* parts,
                                 hipStream_t stream) {
  const bool aligned16 = (((uintptr_t)x & 15u) == 0) && (ldx % 8 == 0);
  if (axis == 0 && !(aligned16 && C % 8 == 0)) {
    hipError_t e = launch_quantize(x, R, C, ldx, fmt, rounding, hadamard, axis, seed, codes, scales, tensor_scale,
                                   amax_partials, stream);
    if (e != hipSuccess) return e;
    return launch_noise(x, ldx, axis, fmt, hadamard, C, R, codes, scales, tensor_scale, stats, parts, stream);
  }
  if (fmt == FMT_NV) launch_tensor_scale(x, R, C, ldx, hadamard, axis, tensor_scale, amax_partials, stream);
  int64_t n;
  if (fmt == FMT_MX) {
    if (rounding == RND_RTN)
      n = launch_had<FMT_MX, RND_RTN, true>(hadamard, axis, x, R, C, ldx, seed, codes, scales, tensor_scale, stream, parts);
    else
      n = launch_had<FMT_MX, RND_SR, true>(hadamard, axis, x, R, C, ldx, seed, codes, scales, tensor_scale, stream, parts);
  } else {
    if (rounding == RND_RTN)
      n = launch_had<FMT_NV, RND_RTN, true>(hadamard, axis, x, R, C, ldx, seed, codes, scales, tensor_scale, stream, parts);
    else
      n = launch_had<FMT_NV, RND_SR, true>(hadamard, axis, x, R, C, ldx, seed, codes, scales, tensor_scale, stream, parts);
  }
  launch_noise_finalize(parts, n, stats, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize: value = E2M1(code) * scale (NVFP4: RN(RN(E2M1 * s_b) * s_t)).
// Lane = 8 elements (one 32-bit word of codes).
// ---------------------------------------------------------------------------
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
  int grid = grid_for(rows * (K / 8), 256, 256 * 64);
  if (fmt == FMT_MX)
    hipLaunchKernelGGL((dequant_kernel<FMT_MX>), dim3(grid), dim3(256), 0, stream, codes, scales, ts, rows, K, y, ldy);
  else
    hipLaunchKernelGGL((dequant_kernel<FMT_NV>), dim3(grid), dim3(256), 0, stream, codes, scales, ts, rows, K, y, ldy);
  return hipGetLastError();
}

}  // namespace mxfp4
