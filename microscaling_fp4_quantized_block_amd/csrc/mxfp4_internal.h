// mxfp4_internal.h -- launchers shared between the C ABI and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

// Work per workgroup of the quantizer kernels, in 16-byte (8-element) chunks:
// the row quantizer and the NVFP4 tensor-amax scan use an exact grid.
constexpr int kRowChunksPerWG = 512;
constexpr int kAmaxChunksPerWG = 2048;
// Workgroups (and partial maxima) of the rotated tensor-amax pass.
constexpr int kAmaxRotPartials = 1024;

// Workspace of mxfp4_quantize: one 32-bit partial maximum per workgroup of
// the NVFP4 tensor-amax pass (0 bytes for MXFP4).
size_t quantize_workspace_bytes(int fmt, int64_t R, int64_t C);

hipError_t launch_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int rounding,
                           int hadamard, int axis, uint64_t seed, uint8_t* codes, uint8_t* scales,
                           float* tensor_scale, uint32_t* partials, hipStream_t stream);

hipError_t launch_dequantize(int fmt, int64_t rows, int64_t K, const uint8_t* codes, const uint8_t* scales,
                             const float* ts, float* y, int64_t ldy, hipStream_t stream);

// GEMM planning: how many K-splits a launch uses (1 = none).  The workspace
// holds splits * M * N floats when splits > 1.
struct GemmPlan {
  int splits;
  int64_t k_tiles;     // contraction tiles of the kernel's K step
  int narrow_tm;       // MXFP4 with M <= 128: rows per narrow tile / 32 (1, 2 or 4); 0 = wide tiles
  int waves8;          // MXFP4 wide tiles with at most four stages: the 8-wave kernel
  int decode;          // MXFP4 with few rows against a long weight: gemm_mx_decode_kernel with this many 16-row A tiles
};
// MXFP4 with at most MXFP4_DECODE_MAX_M activation rows takes the decode
// kernel against weights of at least MXFP4_DECODE_MIN_N rows, or when a
// workgroup's operand bytes stay within MXFP4_DECODE_WG_BYTES
#ifndef MXFP4_DECODE_MIN_N
#define MXFP4_DECODE_MIN_N 2048
#endif
#ifndef MXFP4_DECODE_MAX_M
#define MXFP4_DECODE_MAX_M 128
#endif
#ifndef MXFP4_DECODE_WG_BYTES
#define MXFP4_DECODE_WG_BYTES (512 * 1024)
#endif
// and from this many, two 16-row weight tiles per workgroup
#ifndef MXFP4_DECODE_TN2_MIN_N
#define MXFP4_DECODE_TN2_MIN_N 8192
#endif
GemmPlan plan_gemm(int fmt, int64_t M, int64_t N, int64_t K);

// C: fp32, or bf16 (round to nearest even from the fp32 result) when c_bf16.
hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* C, int64_t ldc,
                          int c_bf16, float* workspace, const GemmPlan& plan, hipStream_t stream);

// MXFP4 GEMM whose epilogue quantizes C for the next layer: codes/scales of
// Q_MX,RTN(bf16(A B^T)) along rows (block Hadamard first when hadamard); plans
// without a K split only (splits == 1), N % 32 == 0.
hipError_t launch_gemm_mx_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                                   const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, uint8_t* q_codes,
                                   uint8_t* q_scales, int hadamard, const GemmPlan& plan, hipStream_t stream);

// Fused activation quantization + MXFP4 GEMM (narrow plans with 32-row tiles,
// M <= 32, whose splits hold at most 16 stages): A = Q_MX,RTN(x [M, K] bf16,
// row stride ldx, block Hadamard when hadamard), C = A * B^T.
bool fused_plan_ok(const GemmPlan& plan);
hipError_t launch_gemm_mx_fused(const uint16_t* x, int64_t ldx, int hadamard, const uint8_t* b_codes,
                                const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* C, int64_t ldc,
                                float* workspace, const GemmPlan& plan, hipStream_t stream);

hipError_t launch_gemm_nv(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                          const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts, int64_t M,
                          int64_t N, int64_t K, void* C, int64_t ldc, int c_bf16, float* workspace,
                          const GemmPlan& plan, hipStream_t stream);

// NVFP4 tensor scale of an input (amax pass + finalize) into tensor_scale;
// partials: quantize_workspace_bytes(FMT_NV, R, C) bytes.
void launch_tensor_scale(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                         float* tensor_scale, uint32_t* partials, hipStream_t s);

// MXFP4 round-to-nearest with a fixed grid scale through the row / tiled
// transposing quantizers; false (nothing launched) when the input takes
// neither (an unaligned transposed input).
bool launch_quantize_grid_fast(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                               float alpha, uint8_t* codes, uint8_t* scales, hipStream_t s);

// MXFP4 round-to-nearest with MSE-fitted block scales, transposed (axis 0),
// through the tiled transposing quantizer; false (nothing launched) when the
// input is not that kernel's (axis 1, or unaligned).
bool launch_quantize_mse_mx_fast(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s);

// Round-to-nearest quantization with MSE-fitted scales (mse.hip).
size_t quantize_mse_workspace_bytes(int fmt, int hadamard, int64_t R, int64_t C, int axis);
hipError_t launch_quantize_mse(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int hadamard,
                               int axis, int iters, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                               void* workspace, hipStream_t stream);

// MXFP4 round-to-nearest with a fixed grid scale alpha (mse.hip): each block's
// exponent chosen for RN(alpha * absmax).  K % 32 == 0.
hipError_t launch_quantize_grid(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                                float alpha, uint8_t* codes, uint8_t* scales, hipStream_t stream);

// Signal and quantization-noise sums of a quantized operand (noise.hip):
// workspace = 3 doubles per workgroup of the pass.
size_t noise_workspace_bytes(int fmt, int hadamard, int64_t rows, int64_t K);
// Fixed-order sum of nparts partial triples into stats[0..2].
void launch_noise_finalize(const double* partials, int64_t nparts, double* stats, hipStream_t s);
// Quantize with the signal / noise sums: quantize_noise_parts is the largest
// number of partial triples (doubles x 3) any launch plan of the call writes.
int64_t quantize_noise_parts(int fmt, int hadamard, int64_t R, int64_t C, int axis);
hipError_t launch_quantize_noise(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int rounding,
                                 int hadamard, int axis, uint64_t seed, uint8_t* codes, uint8_t* scales,
                                 float* tensor_scale, uint32_t* amax_partials, double* stats, double* parts,
                                 hipStream_t stream);
hipError_t launch_noise(const uint16_t* x, int64_t ldx, int axis, int fmt, int hadamard, int64_t rows, int64_t K,
                        const uint8_t* codes, const uint8_t* scales, const float* ts, double* stats,
                        double* partials, hipStream_t stream);

// Q-EMA weight quantizer (quantize.hip): ema <- RN(RN(beta ema) + RN((1 - beta) w)),
// then MXFP4 round-to-nearest of the new ema along its rows.  Needs C % 32 == 0,
// R * C / 8 < 2^31, w and ema rows 16-byte aligned.
hipError_t launch_qema(const uint16_t* w, int64_t R, int64_t C, int64_t ldw, float* m, int64_t lde, float beta,
                       int hadamard, uint8_t* codes, uint8_t* scales, hipStream_t stream);

// The static device scratch of mxfp4_quantize_noalloc (noalloc.hip): its size,
// and the current device's address of it (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);

}  // namespace mxfp4
