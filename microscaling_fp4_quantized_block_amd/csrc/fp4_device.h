// fp4_device.h -- device helpers shared by the libmxfp4 kernels (gfx950).
//
// Formats (web pages on microscaling FP4, cited by title and section):
//   E2M1 elements and the NVFP4 block of 16 with an E4M3 scale:
//     "FP4 All the Way: Fully Quantized Training of LLMs", abstract.
//   MXFP4's power-of-two (E8M0) shared scale per group:
//     "Bridging the Gap Between Promise and Performance for Microscaling FP4
//     Quantization", abstract; "Oscillation-Reduced MXFP4 Training for Vision
//     Transformers", abstract (per-group scaling).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int FMT_MX = 0;
constexpr int FMT_NV = 1;
constexpr int RND_RTN = 0;
constexpr int RND_SR = 1;

// ---------------------------------------------------------------------------
// Cross-lane helpers (DPP within a quad of 4 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  // quad_perm [1,0,3,2]
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
  // quad_perm [2,3,0,1]
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
}
__device__ __forceinline__ float dpp_xor1f(float v) {
  return __uint_as_float(dpp_xor1(__float_as_uint(v)));
}
__device__ __forceinline__ float dpp_xor2f(float v) {
  return __uint_as_float(dpp_xor2(__float_as_uint(v)));
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// ---------------------------------------------------------------------------
// Division of a 32-bit index by a divisor fixed for the launch
// (Granlund & Montgomery: q = (umulhi(n, m) + n) >> s, the sum in 64 bits).
struct FastDiv {
  uint32_t d, m, s;
};
static FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) s++;
  const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}
__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
  const uint32_t hi = __umulhi(n, f.m);
  return (uint32_t)(((uint64_t)hi + n) >> f.s);
}

// ---------------------------------------------------------------------------
// MXFP4 shared scale: the smallest e with 6 * 2^e >= amax, clamped to
// [-127, 127]; returned as the E8M0 byte e + 127.  `abits` is the IEEE
// binary32 pattern of amax >= 0 (finite).  For a normal amax = (1 + f) 2^E:
// e = E - 2 when f <= 1/2, else E - 1; zero and subnormal amax give -127.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t mx_scale_byte_from_f32bits(uint32_t abits) {
  int ef = (int)(abits >> 23);                    // biased exponent (sign is 0)
  int inc = (abits & 0x7FFFFFu) > 0x400000u ? 1 : 0;
  int b = ef - 2 + inc;                           // (E - 2 + inc) + 127
  if (ef == 0) b = 0;
  return (uint32_t)(b < 0 ? 0 : b);
}

// The binary32 number whose exponent field is the E8M0 byte: the scale
// operand format of the gfx950 FP4 conversion instructions (only the
// exponent bits are used; byte 0 stands for 2^-127).
__device__ __forceinline__ float e8m0_as_cvt_scale(uint32_t byte) {
  return __uint_as_float(byte << 23);
}

// Exact binary32 value 2^(127 - byte) = 1 / 2^(byte - 127), byte in [0, 254].
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) {
  int ef = 254 - (int)byte;                       // exponent field of 2^(127-byte)
  // byte 254 -> 2^-127 is subnormal: 0x00400000
  return ef > 0 ? __uint_as_float((uint32_t)ef << 23) : __uint_as_float(0x00400000u);
}

// Exact binary32 value of an E8M0 byte (0xFF -> NaN); 2^-127 is subnormal.
__device__ __forceinline__ float e8m0_value(uint32_t byte) {
  if (byte == 0xFFu) return __uint_as_float(0x7FC00000u);
  return byte > 0 ? __uint_as_float(byte << 23) : __uint_as_float(0x00400000u);
}

// ---------------------------------------------------------------------------
// Block Hadamard rotation ("Bridging the Gap Between Promise and Performance
// for Microscaling FP4 Quantization", abstract: block-wise Hadamard
// transforms).  Butterfly h: (x[i], x[i+h]) -> (x[i] + x[i+h], x[i] - x[i+h])
// for i & h == 0, strides 1, 2, 4, 8, 16 in that order, then multiply by
// RN_f32(1/sqrt(32)) = 0x3E3504F3.  Every evaluation of this butterfly tree in
// IEEE binary32 gives the same bits, whatever the data layout.
// ---------------------------------------------------------------------------
constexpr uint32_t kHadamardScaleBits = 0x3E3504F3u;

// Full 32-point rotation of a block held in one lane (32 registers).
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

// MXFP4 round-to-nearest of one 32-element block held in one lane: the E8M0
// byte from the block absmax (an integer max over |binary32 bits|), then the
// hardware FP4 conversion of y / 2^e (nearest-even, saturating); element j
// lands in bits 4 (j % 8) .. +3 of codes[j / 8].  A block holding a NaN or an
// infinity gets byte 0xFF and all-zero codes.
__device__ __forceinline__ uint32_t mx_rtn_block32(const float y[32], uint32_t codes[4]) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 32; j++) m = max(m, __float_as_uint(y[j]) & 0x7FFFFFFFu);
  if (m >= 0x7F800000u) {
    codes[0] = codes[1] = codes[2] = codes[3] = 0u;
    return 0xFFu;
  }
  const uint32_t byte = mx_scale_byte_from_f32bits(m);
  const float sc = e8m0_as_cvt_scale(byte);
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint32_t packed = 0;
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[8 * q + 0], y[8 * q + 1], sc, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[8 * q + 2], y[8 * q + 3], sc, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[8 * q + 4], y[8 * q + 5], sc, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[8 * q + 6], y[8 * q + 7], sc, 3);
    codes[q] = packed;
  }
  return byte;
}

// E2M1 code -> value (OCP layout: bit 3 sign, bits 2:1 exponent with bias 1,
// bit 0 mantissa; exponent 0 is subnormal), exact in binary32.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  // magnitude table {0, .5, 1, 1.5, 2, 3, 4, 6} in binary32 bit patterns
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float mag = e == 0 ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return (c & 8u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// E4M3 (bias 7, no infinities, 0x7F NaN).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_value(uint32_t byte) {
  byte &= 0x7Fu;
  if (byte == 0x7Fu) return __uint_as_float(0x7FC00000u);
  if (byte < 8u) return (float)byte * 0x1p-9f;    // subnormal m * 2^-9 (exact)
  return __uint_as_float((((byte >> 3) + 120u) << 23) | ((byte & 7u) << 20));
}

// Smallest non-negative E4M3 value >= r (r >= 0, finite), saturating at 448.
//   r < 2^-6 : subnormal range, byte = ceil(r * 2^9) (8 means 2^-6, which is
//              also the byte of the smallest normal);
//   else     : r = (1 + f) 2^E, byte = ((E + 7) << 3) + ceil(8 f), where a
//              mantissa of 8 carries into the exponent.
__device__ __forceinline__ uint32_t e4m3_round_up_byte(float r) {
  if (!(r > 0.0f)) return 0u;
  if (r > 448.0f) return 0x7Eu;
  uint32_t b;
  if (r < 0x1p-6f) {
    b = (uint32_t)__builtin_ceilf(r * 512.0f);
  } else {
    uint32_t bits = __float_as_uint(r);
    int E = (int)(bits >> 23) - 127;
    uint32_t m = ((bits & 0x7FFFFFu) + 0xFFFFFu) >> 20;
    b = (uint32_t)((E + 7) << 3) + m;
  }
  return b > 0x7Eu ? 0x7Eu : b;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  The key schedule is
// uniform across a wavefront, so key words live in scalar registers.
// ---------------------------------------------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; r++) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input XOR in one v_bitop3 (truth table 0x96)
    uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// ---------------------------------------------------------------------------
// Stochastic rounding of 8 scaled elements xs[j] to 4-bit codes, element j
// drawing the 16-bit value r_j = bits 16(j&1)..+15 of rw[j/2].
//
// Definition: a = min(|xs|, 6) lies between E2M1 neighbours lo <= a < hi;
// with t = floor(2^16 (a - lo) / (hi - lo)) the code rounds up iff r_j < t,
// and carries the input's sign bit (also for a zero result).
//
// gfx950's v_cvt_scalef32_sr_pk_fp4_f32 rounds the element in its first slot
// up iff (a - lo) / (hi - lo) + rnd * 2^-32 >= 1, saturating at 6 and keeping
// the sign bit (measured on every 16-bit draw at each threshold and one ulp
// either side in every binade, plus zeros, denormals and saturation).  With
// rnd = (65535 - r) * 2^16 that is frac + (65535 - r) / 2^16 >= 1, i.e.
// floor(2^16 frac) >= r + 1: exactly the definition.  The second slot draws
// from rnd shifted left by one, so two independent 16-bit draws cannot share
// one call; each element gets its own call with 0 in the second slot (code 0
// in the byte's high nibble).  Only byte 0 of the result is defined with
// sel = 0 (the compiler does not carry the old value into the other bytes),
// so the byte-0 codes are gathered with v_perm_b32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t sr_encode8(const float xs[8], const uint32_t rw[4]) {
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const uint32_t w = rw[j >> 1];
    // (65535 - r) << 16 for r in the low or the high half of w
    const uint32_t rnd = (j & 1) ? (~w & 0xFFFF0000u) : ((w << 16) ^ 0xFFFF0000u);
    c[j] = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (f32x2){xs[j], 0.0f}, rnd, 1.0f, 0);
  }
  // v_perm_b32 selector bytes: 0..3 pick bytes of the second operand, 4..7 of
  // the first, 0x0C gives zero
  const uint32_t even = __builtin_amdgcn_perm(c[2], c[0], 0x0C0C0400u) | __builtin_amdgcn_perm(c[6], c[4], 0x04000C0Cu);
  const uint32_t odd = __builtin_amdgcn_perm(c[3], c[1], 0x0C0C0400u) | __builtin_amdgcn_perm(c[7], c[5], 0x04000C0Cu);
  return even | (odd << 4);
}

// ---------------------------------------------------------------------------
// Signal and quantization-noise sums (binary64): for 8 elements y and their
// codes (one 32-bit word), Q(y) = E2M1(code) * sc exactly,
//   s0 += y^2, s1 += (Q(y) - y)^2,
// squares accumulated with fused multiply-adds (y * y is exact, so the
// same as a multiply and an add).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void noise_accum8(const float y[8], uint32_t codes, double sc, double& s0, double& s1) {
  float g[8];
  const f32x2 g0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const f32x2 g1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const f32x2 g2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const f32x2 g3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  g[0] = g0[0]; g[1] = g0[1]; g[2] = g1[0]; g[3] = g1[1];
  g[4] = g2[0]; g[5] = g2[1]; g[6] = g3[0]; g[7] = g3[1];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const double yv = (double)y[j];
    const double d = (double)g[j] * sc - yv;
    s0 = __builtin_fma(yv, yv, s0);
    s1 = __builtin_fma(d, d, s1);
  }
}

// Sum of three per-thread values over a 256-thread workgroup (butterflies
// within each wave, then the four waves in a fixed order) into out[0..2] by
// thread 0.  Every thread of the workgroup must call it.
__device__ __forceinline__ void block_sum3(double& a, double& b, double& c, double* out) {
  __shared__ double red[3][4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
    c += __shfl_xor(c, off, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][w] = a; red[1][w] = b; red[2][w] = c; }
  __syncthreads();
  if (threadIdx.x == 0) {
    out[0] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    out[1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    out[2] = (red[2][0] + red[2][1]) + (red[2][2] + red[2][3]);
  }
}

}  // namespace mxfp4
