// mxfp4_abi.cpp -- the C ABI of libmxfp4: argument checks, sizes, dispatch.
//
// Every entry point validates its arguments before anything is launched and
// reports problems as an mxfp4_status; nothing is allocated, freed or
// synchronized here.  The operations themselves are described in mxfp4.h.
#include "mxfp4.h"

#include <hip/hip_runtime.h>

#include "mxfp4_internal.h"

namespace {

int block_of(int fmt) { return fmt == MXFP4_FMT_MX ? 32 : 16; }
bool fmt_ok(int fmt) { return fmt == MXFP4_FMT_MX || fmt == MXFP4_FMT_NV; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Largest element count the kernels index (R * C and rows * k): the 64-bit
// index math is exact well beyond any tensor that fits in device memory.
constexpr int64_t kMaxElems = (int64_t)1 << 40;

// Longest GEMM contraction: a 256-row tile of operand codes (256 * K/2 bytes)
// stays within the 2^31-byte range of a buffer resource.
constexpr int64_t kMaxGemmK = (int64_t)1 << 24;

}  // namespace

extern "C" {

const char* mxfp4_status_string(int status) {
  switch (status) {
    case MXFP4_OK: return "MXFP4_OK";
    case MXFP4_ERR_INVALID_ARG: return "MXFP4_ERR_INVALID_ARG: null pointer, bad enum, negative size or leading dimension too small";
    case MXFP4_ERR_UNSUPPORTED_SHAPE: return "MXFP4_ERR_UNSUPPORTED_SHAPE: contraction length is not a multiple of the required block";
    case MXFP4_ERR_FORMAT_MISMATCH: return "MXFP4_ERR_FORMAT_MISMATCH: GEMM operands differ in format, contraction length or rotation";
    case MXFP4_ERR_WORKSPACE: return "MXFP4_ERR_WORKSPACE: workspace missing or too small";
    case MXFP4_ERR_HIP: return "MXFP4_ERR_HIP: a HIP kernel launch failed";
    default: return "unknown mxfp4_status";
  }
}

mxfp4_status mxfp4_qema_quantize(const uint16_t* w, int64_t R, int64_t C, int64_t ldw, float* ema, int64_t lde,
                                 float beta, int hadamard, mxfp4_tensor* out, hipStream_t stream) {
  if (!out || (hadamard != 0 && hadamard != 1) || !(beta >= 0.0f && beta <= 1.0f)) return MXFP4_ERR_INVALID_ARG;
  if (R < 0 || C < 0 || ldw < C || lde < C || ldw < 1 || lde < 1) return MXFP4_ERR_INVALID_ARG;
  if (C % 32 != 0) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (R > 0 && C / 8 > (((int64_t)1 << 31) - 1) / R) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (out->fmt != MXFP4_FMT_MX || out->rows != R || out->k != C || out->hadamard != hadamard)
    return MXFP4_ERR_INVALID_ARG;
  if (R == 0 || C == 0) return MXFP4_OK;
  if (!w || !ema || !out->codes || !out->scales) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(w, 16) || ldw % 8 != 0 || !aligned(ema, 16) || lde % 4 != 0 || !aligned(out->codes, 16))
    return MXFP4_ERR_INVALID_ARG;
  hipError_t e = mxfp4::launch_qema(w, R, C, ldw, ema, lde, beta, hadamard, out->codes, out->scales, stream);
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

mxfp4_status mxfp4_quantize_grid(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                                 float alpha, mxfp4_tensor* out, hipStream_t stream) {
  if (!out || (hadamard != 0 && hadamard != 1) || (axis != 0 && axis != 1)) return MXFP4_ERR_INVALID_ARG;
  if (!(alpha > 0.0f) || !(alpha <= 65536.0f)) return MXFP4_ERR_INVALID_ARG;
  if (R < 0 || C < 0 || ldx < C || ldx < 1) return MXFP4_ERR_INVALID_ARG;
  const int64_t rows = axis == 1 ? R : C, k = axis == 1 ? C : R;
  if (k % 32 != 0) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (R > 0 && C > kMaxElems / R) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (out->fmt != MXFP4_FMT_MX || out->rows != rows || out->k != k || out->hadamard != hadamard)
    return MXFP4_ERR_INVALID_ARG;
  if (rows == 0 || k == 0) return MXFP4_OK;
  if (!x || !out->codes || !out->scales || !aligned(out->codes, 16)) return MXFP4_ERR_INVALID_ARG;
  hipError_t e = mxfp4::launch_quantize_grid(x, R, C, ldx, hadamard, axis, alpha, out->codes, out->scales, stream);
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

mxfp4_status mxfp4_noise_ratio(const double* stats, double* ratio, int* below_threshold) {
  if (!stats || !ratio || !below_threshold) return MXFP4_ERR_INVALID_ARG;
  const double signal = stats[0], noise = stats[1];
  if (!(signal >= 0.0) || !(noise >= 0.0)) return MXFP4_ERR_INVALID_ARG;   // also rejects NaN
  *ratio = noise == 0.0 ? __builtin_inf() : __builtin_sqrt(signal / noise);
  *below_threshold = *ratio < __builtin_sqrt(3.0) ? 1 : 0;
  return MXFP4_OK;
}

mxfp4_status mxfp4_tensor_bytes(int fmt, int64_t rows, int64_t k, size_t* codes_bytes, size_t* scales_bytes) {
  if (!fmt_ok(fmt) || rows < 0 || k < 0 || !codes_bytes || !scales_bytes) return MXFP4_ERR_INVALID_ARG;
  if (k % block_of(fmt) != 0) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  *codes_bytes = (size_t)rows * (size_t)(k / 2);
  *scales_bytes = (size_t)rows * (size_t)(k / block_of(fmt));
  return MXFP4_OK;
}

mxfp4_status mxfp4_quantize_workspace_bytes(int fmt, int64_t R, int64_t C, int axis, size_t* bytes) {
  if (!fmt_ok(fmt) || R < 0 || C < 0 || (axis != 0 && axis != 1) || !bytes) return MXFP4_ERR_INVALID_ARG;
  *bytes = mxfp4::quantize_workspace_bytes(fmt, R, C);
  return MXFP4_OK;
}

}  // extern "C"

namespace {

// Argument checks of mxfp4_quantize (and its no-allocation variant); OK with
// *empty set when there is nothing to do.
mxfp4_status check_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int rounding,
                            int hadamard, int axis, const mxfp4_tensor* out, bool* empty) {
  *empty = false;
  if (!fmt_ok(fmt) || (rounding != MXFP4_RTN && rounding != MXFP4_SR) || (hadamard != 0 && hadamard != 1) ||
      (axis != 0 && axis != 1) || !out)
    return MXFP4_ERR_INVALID_ARG;
  if (R < 0 || C < 0 || ldx < C || ldx < 1) return MXFP4_ERR_INVALID_ARG;
  const int64_t rows = axis == 1 ? R : C, k = axis == 1 ? C : R;
  if (k % block_of(fmt) != 0 || (hadamard && k % 32 != 0)) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (R > 0 && C > kMaxElems / R) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (out->fmt != fmt || out->rows != rows || out->k != k || out->hadamard != hadamard)
    return MXFP4_ERR_INVALID_ARG;
  if (rows == 0 || k == 0) {
    *empty = true;
    return MXFP4_OK;
  }
  if (!x || !out->codes || !out->scales) return MXFP4_ERR_INVALID_ARG;
  // the kernels store codes as aligned 32-bit (rows) or 8/16-byte (transposed) words
  if (!aligned(out->codes, 16)) return MXFP4_ERR_INVALID_ARG;
  if (fmt == MXFP4_FMT_NV && !out->tensor_scale) return MXFP4_ERR_INVALID_ARG;
  return MXFP4_OK;
}

}  // namespace

extern "C" {

mxfp4_status mxfp4_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int rounding,
                            int hadamard, int axis, uint64_t seed, mxfp4_tensor* out, void* workspace,
                            size_t ws_bytes, hipStream_t stream) {
  bool empty;
  const mxfp4_status st = check_quantize(x, R, C, ldx, fmt, rounding, hadamard, axis, out, &empty);
  if (st != MXFP4_OK || empty) return st;
  uint32_t* partials = nullptr;
  if (fmt == MXFP4_FMT_NV) {
    if (!workspace || ws_bytes < mxfp4::quantize_workspace_bytes(fmt, R, C) || !aligned(workspace, 4))
      return MXFP4_ERR_WORKSPACE;
    partials = (uint32_t*)workspace;
  }
  hipError_t e = mxfp4::launch_quantize(x, R, C, ldx, fmt, rounding, hadamard, axis, seed, out->codes,
                                        out->scales, out->tensor_scale, partials, stream);
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

mxfp4_status mxfp4_quantize_noalloc(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int rounding,
                                    int hadamard, int axis, uint64_t seed, mxfp4_tensor* out, hipStream_t stream) {
  bool empty;
  const mxfp4_status st = check_quantize(x, R, C, ldx, fmt, rounding, hadamard, axis, out, &empty);
  if (st != MXFP4_OK || empty) return st;
  uint32_t* partials = nullptr;
  if (fmt == MXFP4_FMT_NV) {
    if (mxfp4::quantize_workspace_bytes(fmt, R, C) > mxfp4::noalloc_scratch_bytes()) return MXFP4_ERR_WORKSPACE;
    void* p = nullptr;
    if (mxfp4::noalloc_scratch(&p) != hipSuccess) return MXFP4_ERR_HIP;
    partials = (uint32_t*)p;
  }
  hipError_t e = mxfp4::launch_quantize(x, R, C, ldx, fmt, rounding, hadamard, axis, seed, out->codes,
                                        out->scales, out->tensor_scale, partials, stream);
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

// Workspace of mxfp4_quantize_noise: the quantizer's (NVFP4 amax partials),
// padded to 16 bytes, then the partial sums.
static size_t quantize_noise_ws(int fmt, int hadamard, int64_t R, int64_t C, int axis, size_t* amax_bytes) {
  const size_t q = (mxfp4::quantize_workspace_bytes(fmt, R, C) + 15) & ~(size_t)15;
  *amax_bytes = q;
  return q + (size_t)mxfp4::quantize_noise_parts(fmt, hadamard, R, C, axis) * 3 * sizeof(double);
}

mxfp4_status mxfp4_quantize_noise_workspace_bytes(int fmt, int hadamard, int64_t R, int64_t C, int axis,
                                                  size_t* bytes) {
  if (!fmt_ok(fmt) || (hadamard != 0 && hadamard != 1) || R < 0 || C < 0 || (axis != 0 && axis != 1) || !bytes)
    return MXFP4_ERR_INVALID_ARG;
  const int64_t k = axis == 1 ? C : R;
  if (k % block_of(fmt) != 0 || (hadamard && k % 32 != 0)) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (R > 0 && C > kMaxElems / R) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  size_t a;
  *bytes = quantize_noise_ws(fmt, hadamard, R, C, axis, &a);
  return MXFP4_OK;
}

mxfp4_status mxfp4_quantize_noise(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int rounding,
                                  int hadamard, int axis, uint64_t seed, mxfp4_tensor* out, double* stats,
                                  void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!fmt_ok(fmt) || (rounding != MXFP4_RTN && rounding != MXFP4_SR) || (hadamard != 0 && hadamard != 1) ||
      (axis != 0 && axis != 1) || !out || !stats)
    return MXFP4_ERR_INVALID_ARG;
  if (R < 0 || C < 0 || ldx < C || ldx < 1) return MXFP4_ERR_INVALID_ARG;
  const int64_t rows = axis == 1 ? R : C, k = axis == 1 ? C : R;
  if (k % block_of(fmt) != 0 || (hadamard && k % 32 != 0)) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (R > 0 && C > kMaxElems / R) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (out->fmt != fmt || out->rows != rows || out->k != k || out->hadamard != hadamard)
    return MXFP4_ERR_INVALID_ARG;
  if (!aligned(stats, 8)) return MXFP4_ERR_INVALID_ARG;
  if (rows > 0 && k > 0) {
    if (!x || !out->codes || !out->scales || !aligned(x, 2) || !aligned(out->codes, 16)) return MXFP4_ERR_INVALID_ARG;
    if (fmt == MXFP4_FMT_NV && !out->tensor_scale) return MXFP4_ERR_INVALID_ARG;
  }
  size_t amax_bytes;
  const size_t need = quantize_noise_ws(fmt, hadamard, R, C, axis, &amax_bytes);
  if (!workspace || ws_bytes < need || !aligned(workspace, 16)) return MXFP4_ERR_WORKSPACE;
  hipError_t e;
  if (rows == 0 || k == 0) {
    // nothing to quantize: the finalize over no partials writes zero sums
    mxfp4::launch_noise_finalize(nullptr, 0, stats, stream);
    e = hipGetLastError();
  } else {
    e = mxfp4::launch_quantize_noise(x, R, C, ldx, fmt, rounding, hadamard, axis, seed, out->codes, out->scales,
                                     out->tensor_scale, (uint32_t*)workspace, stats,
                                     (double*)((uint8_t*)workspace + amax_bytes), stream);
  }
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

mxfp4_status mxfp4_dequantize(const mxfp4_tensor* q, float* y, int64_t ldy, hipStream_t stream) {
  if (!q || !fmt_ok(q->fmt) || q->rows < 0 || q->k < 0) return MXFP4_ERR_INVALID_ARG;
  if (q->k % block_of(q->fmt) != 0) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (ldy < q->k) return MXFP4_ERR_INVALID_ARG;
  if (q->rows == 0 || q->k == 0) return MXFP4_OK;
  if (!y || !q->codes || !q->scales || (q->fmt == MXFP4_FMT_NV && !q->tensor_scale)) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(q->codes, 4)) return MXFP4_ERR_INVALID_ARG;
  hipError_t e = mxfp4::launch_dequantize(q->fmt, q->rows, q->k, q->codes, q->scales, q->tensor_scale, y, ldy,
                                          stream);
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

static mxfp4_status check_gemm_operands(const mxfp4_tensor* A, const mxfp4_tensor* B) {
  if (!A || !B || !fmt_ok(A->fmt) || !fmt_ok(B->fmt) || A->rows < 0 || B->rows < 0 || A->k < 0 || B->k < 0)
    return MXFP4_ERR_INVALID_ARG;
  if (A->fmt != B->fmt || A->k != B->k || A->hadamard != B->hadamard) return MXFP4_ERR_FORMAT_MISMATCH;
  // the kernels' contraction step is 128 (one 64-byte chunk of codes per row)
  if (A->k % 128 != 0) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  // a tile's operand rows are addressed through 32-bit buffer offsets
  if (A->k > kMaxGemmK) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  return MXFP4_OK;
}

mxfp4_status mxfp4_gemm_workspace_bytes(const mxfp4_tensor* A, const mxfp4_tensor* B, size_t* bytes) {
  if (!bytes) return MXFP4_ERR_INVALID_ARG;
  mxfp4_status s = check_gemm_operands(A, B);
  if (s != MXFP4_OK) return s;
  mxfp4::GemmPlan pl = mxfp4::plan_gemm(A->fmt, A->rows, B->rows, A->k);
  *bytes = pl.splits > 1 ? (size_t)pl.splits * (size_t)A->rows * (size_t)B->rows * sizeof(float) : 0;
  return MXFP4_OK;
}

// C: fp32, or bf16 bit patterns when c_bf16.
static mxfp4_status gemm_impl(const mxfp4_tensor* A, const mxfp4_tensor* B, void* C, int64_t ldc, int c_bf16,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  mxfp4_status s = check_gemm_operands(A, B);
  if (s != MXFP4_OK) return s;
  const int64_t M = A->rows, N = B->rows, K = A->k;
  if (ldc < N || ldc < 1) return MXFP4_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return MXFP4_OK;
  if (!C || !A->codes || !A->scales || !B->codes || !B->scales) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(C, c_bf16 ? 2 : 4)) return MXFP4_ERR_INVALID_ARG;
  if (A->fmt == MXFP4_FMT_NV && (!A->tensor_scale || !B->tensor_scale)) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(A->codes, 16) || !aligned(B->codes, 16) || !aligned(A->scales, 4) || !aligned(B->scales, 4))
    return MXFP4_ERR_INVALID_ARG;
  mxfp4::GemmPlan pl = mxfp4::plan_gemm(A->fmt, M, N, K);
  if (pl.splits > 1) {
    const size_t need = (size_t)pl.splits * (size_t)M * (size_t)N * sizeof(float);
    if (!workspace || ws_bytes < need || !aligned(workspace, 4)) return MXFP4_ERR_WORKSPACE;
  }
  hipError_t e;
  if (A->fmt == MXFP4_FMT_MX)
    e = mxfp4::launch_gemm_mx(A->codes, A->scales, B->codes, B->scales, M, N, K, C, ldc, c_bf16,
                              (float*)workspace, pl, stream);
  else
    e = mxfp4::launch_gemm_nv(A->codes, A->scales, A->tensor_scale, B->codes, B->scales, B->tensor_scale, M, N, K,
                              C, ldc, c_bf16, (float*)workspace, pl, stream);
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

mxfp4_status mxfp4_gemm(const mxfp4_tensor* A, const mxfp4_tensor* B, float* C, int64_t ldc, void* workspace,
                        size_t ws_bytes, hipStream_t stream) {
  return gemm_impl(A, B, C, ldc, 0, workspace, ws_bytes, stream);
}

mxfp4_status mxfp4_gemm_bf16(const mxfp4_tensor* A, const mxfp4_tensor* B, uint16_t* C, int64_t ldc,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
  return gemm_impl(A, B, C, ldc, 1, workspace, ws_bytes, stream);
}

// GEMM with the output quantized for the next layer.  Fused into the GEMM's
// epilogue for MXFP4 operands when the plan has no K split; otherwise the bf16
// C goes through the workspace (mxfp4_gemm_bf16, then mxfp4_quantize).
static mxfp4_status check_gemm_quantize(const mxfp4_tensor* A, const mxfp4_tensor* B, int hadamard,
                                        const mxfp4_tensor* out) {
  mxfp4_status s = check_gemm_operands(A, B);
  if (s != MXFP4_OK) return s;
  if (!out || (hadamard != 0 && hadamard != 1)) return MXFP4_ERR_INVALID_ARG;
  if (B->rows % 32 != 0) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (out->fmt != MXFP4_FMT_MX || out->rows != A->rows || out->k != B->rows || out->hadamard != hadamard)
    return MXFP4_ERR_INVALID_ARG;
  if (A->rows > 0 && B->rows > kMaxElems / A->rows) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  return MXFP4_OK;
}

static size_t align16_bytes(size_t n) { return (n + 15) & ~(size_t)15; }

static size_t gemm_quantize_ws(const mxfp4_tensor* A, const mxfp4_tensor* B, bool* fused) {
  const mxfp4::GemmPlan pl = mxfp4::plan_gemm(A->fmt, A->rows, B->rows, A->k);
  *fused = A->fmt == MXFP4_FMT_MX && pl.splits == 1 && !pl.decode;
  if (*fused) return 0;
  const size_t gemm_ws = pl.splits > 1 ? (size_t)pl.splits * (size_t)A->rows * (size_t)B->rows * sizeof(float) : 0;
  return align16_bytes((size_t)A->rows * (size_t)B->rows * 2) + gemm_ws;
}

mxfp4_status mxfp4_gemm_quantize_workspace_bytes(const mxfp4_tensor* A, const mxfp4_tensor* B, int hadamard,
                                                 const mxfp4_tensor* out, size_t* bytes) {
  if (!bytes) return MXFP4_ERR_INVALID_ARG;
  mxfp4_status s = check_gemm_quantize(A, B, hadamard, out);
  if (s != MXFP4_OK) return s;
  bool fused;
  *bytes = gemm_quantize_ws(A, B, &fused);
  return MXFP4_OK;
}

mxfp4_status mxfp4_gemm_quantize(const mxfp4_tensor* A, const mxfp4_tensor* B, int hadamard, mxfp4_tensor* out,
                                 void* workspace, size_t ws_bytes, hipStream_t stream) {
  mxfp4_status s = check_gemm_quantize(A, B, hadamard, out);
  if (s != MXFP4_OK) return s;
  const int64_t M = A->rows, N = B->rows, K = A->k;
  if (M == 0 || N == 0) return MXFP4_OK;
  if (!A->codes || !A->scales || !B->codes || !B->scales || !out->codes || !out->scales) return MXFP4_ERR_INVALID_ARG;
  if (A->fmt == MXFP4_FMT_NV && (!A->tensor_scale || !B->tensor_scale)) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(A->codes, 16) || !aligned(B->codes, 16) || !aligned(A->scales, 4) || !aligned(B->scales, 4) ||
      !aligned(out->codes, 16))
    return MXFP4_ERR_INVALID_ARG;
  bool fused;
  const size_t need = gemm_quantize_ws(A, B, &fused);
  if (need && (!workspace || ws_bytes < need || !aligned(workspace, 16))) return MXFP4_ERR_WORKSPACE;
  if (fused) {
    const mxfp4::GemmPlan pl = mxfp4::plan_gemm(A->fmt, M, N, K);
    hipError_t e = mxfp4::launch_gemm_mx_quantize(A->codes, A->scales, B->codes, B->scales, M, N, K, out->codes,
                                                  out->scales, hadamard, pl, stream);
    return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
  }
  uint16_t* cb = (uint16_t*)workspace;
  uint8_t* gws = (uint8_t*)workspace + align16_bytes((size_t)M * (size_t)N * 2);
  s = gemm_impl(A, B, cb, N, 1, gws, ws_bytes - align16_bytes((size_t)M * (size_t)N * 2), stream);
  if (s != MXFP4_OK) return s;
  return mxfp4_quantize(cb, M, N, N, MXFP4_FMT_MX, MXFP4_RTN, hadamard, 1, 0, out, nullptr, 0, stream);
}

// Online activation quantization + GEMM: fused into the narrow GEMM when the
// plan allows, else quantize into the workspace, then the GEMM.
static mxfp4_status check_quantize_gemm(int64_t M, int64_t K, int hadamard, const mxfp4_tensor* B) {
  if (!B || M < 0 || K < 0 || B->rows < 0 || B->k < 0 || (hadamard != 0 && hadamard != 1) || !fmt_ok(B->fmt))
    return MXFP4_ERR_INVALID_ARG;
  if (B->fmt != MXFP4_FMT_MX || B->k != K || B->hadamard != hadamard) return MXFP4_ERR_FORMAT_MISMATCH;
  if (K % 128 != 0 || K > kMaxGemmK) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (M > 0 && K > kMaxElems / M) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  return MXFP4_OK;
}

static size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

static size_t quantize_gemm_ws(int64_t M, int64_t N, int64_t K, bool* fused) {
  const mxfp4::GemmPlan pl = mxfp4::plan_gemm(MXFP4_FMT_MX, M, N, K);
  const size_t gemm_ws = pl.splits > 1 ? (size_t)pl.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
  *fused = mxfp4::fused_plan_ok(pl);
  if (*fused) return gemm_ws;
  return align16((size_t)M * (size_t)(K / 2)) + align16((size_t)M * (size_t)(K / 32)) + gemm_ws;
}

mxfp4_status mxfp4_quantize_gemm_workspace_bytes(int64_t M, int64_t K, int hadamard, const mxfp4_tensor* B,
                                                 size_t* bytes) {
  if (!bytes) return MXFP4_ERR_INVALID_ARG;
  mxfp4_status s = check_quantize_gemm(M, K, hadamard, B);
  if (s != MXFP4_OK) return s;
  bool fused;
  *bytes = (M == 0 || B->rows == 0) ? 0 : quantize_gemm_ws(M, B->rows, K, &fused);
  return MXFP4_OK;
}

mxfp4_status mxfp4_quantize_gemm(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int hadamard,
                                 const mxfp4_tensor* B, float* C, int64_t ldc, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
  mxfp4_status s = check_quantize_gemm(M, K, hadamard, B);
  if (s != MXFP4_OK) return s;
  const int64_t N = B->rows;
  if (ldx < K || ldx < 1 || ldc < N || ldc < 1) return MXFP4_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return MXFP4_OK;
  if (!x || !C || !B->codes || !B->scales) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(x, 2) || !aligned(B->codes, 16) || !aligned(B->scales, 4)) return MXFP4_ERR_INVALID_ARG;
  bool fused;
  const size_t need = quantize_gemm_ws(M, N, K, &fused);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 16))) return MXFP4_ERR_WORKSPACE;
  const mxfp4::GemmPlan pl = mxfp4::plan_gemm(MXFP4_FMT_MX, M, N, K);
  hipError_t e;
  if (fused) {
    e = mxfp4::launch_gemm_mx_fused(x, ldx, hadamard, B->codes, B->scales, M, N, K, C, ldc, (float*)workspace, pl,
                                    stream);
  } else {
    uint8_t* a_codes = (uint8_t*)workspace;
    uint8_t* a_scales = a_codes + align16((size_t)M * (size_t)(K / 2));
    float* gemm_ws = (float*)(a_scales + align16((size_t)M * (size_t)(K / 32)));
    e = mxfp4::launch_quantize(x, M, K, ldx, MXFP4_FMT_MX, MXFP4_RTN, hadamard, 1, 0, a_codes, a_scales, nullptr,
                               nullptr, stream);
    if (e == hipSuccess)
      e = mxfp4::launch_gemm_mx(a_codes, a_scales, B->codes, B->scales, M, N, K, C, ldc, 0, gemm_ws, pl, stream);
  }
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

static mxfp4_status check_noise_operand(const mxfp4_tensor* q) {
  if (!q || !fmt_ok(q->fmt) || q->rows < 0 || q->k < 0 || (q->hadamard != 0 && q->hadamard != 1))
    return MXFP4_ERR_INVALID_ARG;
  if (q->k % block_of(q->fmt) != 0 || (q->hadamard && q->k % 32 != 0)) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (q->rows > 0 && q->k > kMaxElems / q->rows) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  return MXFP4_OK;
}

mxfp4_status mxfp4_quantization_noise_workspace_bytes(const mxfp4_tensor* q, size_t* bytes) {
  if (!bytes) return MXFP4_ERR_INVALID_ARG;
  mxfp4_status s = check_noise_operand(q);
  if (s != MXFP4_OK) return s;
  *bytes = mxfp4::noise_workspace_bytes(q->fmt, q->hadamard, q->rows, q->k);
  return MXFP4_OK;
}

mxfp4_status mxfp4_quantization_noise(const uint16_t* x, int64_t ldx, int axis, const mxfp4_tensor* q,
                                      double* stats, void* workspace, size_t ws_bytes, hipStream_t stream) {
  mxfp4_status s = check_noise_operand(q);
  if (s != MXFP4_OK) return s;
  if (axis != 0 && axis != 1) return MXFP4_ERR_INVALID_ARG;
  const int64_t C = axis == 1 ? q->k : q->rows;   // columns of the input x [R, C]
  if (ldx < C || ldx < 1 || !stats) return MXFP4_ERR_INVALID_ARG;
  if (q->rows > 0 && q->k > 0) {
    if (!x || !q->codes || !q->scales || (q->fmt == MXFP4_FMT_NV && !q->tensor_scale)) return MXFP4_ERR_INVALID_ARG;
    if (!aligned(x, 2) || !aligned(q->codes, 8)) return MXFP4_ERR_INVALID_ARG;
  }
  if (!aligned(stats, 8)) return MXFP4_ERR_INVALID_ARG;
  const size_t need = mxfp4::noise_workspace_bytes(q->fmt, q->hadamard, q->rows, q->k);
  if (!workspace || ws_bytes < need || !aligned(workspace, 8)) return MXFP4_ERR_WORKSPACE;
  hipError_t e = mxfp4::launch_noise(x, ldx, axis, q->fmt, q->hadamard, q->rows, q->k, q->codes, q->scales,
                                     q->tensor_scale, stats, (double*)workspace, stream);
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

mxfp4_status mxfp4_quantize_mse_workspace_bytes(int fmt, int hadamard, int64_t R, int64_t C, int axis,
                                                size_t* bytes) {
  if (!fmt_ok(fmt) || (hadamard != 0 && hadamard != 1) || R < 0 || C < 0 || (axis != 0 && axis != 1) || !bytes)
    return MXFP4_ERR_INVALID_ARG;
  const int64_t k = axis == 1 ? C : R;
  if (k % block_of(fmt) != 0 || (hadamard && k % 32 != 0)) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (R > 0 && C > kMaxElems / R) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  *bytes = mxfp4::quantize_mse_workspace_bytes(fmt, hadamard, R, C, axis);
  return MXFP4_OK;
}

mxfp4_status mxfp4_quantize_mse(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int fmt, int hadamard,
                                int axis, int iters, mxfp4_tensor* out, void* workspace, size_t ws_bytes,
                                hipStream_t stream) {
  if (!fmt_ok(fmt) || (hadamard != 0 && hadamard != 1) || (axis != 0 && axis != 1) || !out || iters < 0 ||
      iters > 64)
    return MXFP4_ERR_INVALID_ARG;
  if (R < 0 || C < 0 || ldx < C || ldx < 1) return MXFP4_ERR_INVALID_ARG;
  const int64_t rows = axis == 1 ? R : C, k = axis == 1 ? C : R;
  if (k % block_of(fmt) != 0 || (hadamard && k % 32 != 0)) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (R > 0 && C > kMaxElems / R) return MXFP4_ERR_UNSUPPORTED_SHAPE;
  if (out->fmt != fmt || out->rows != rows || out->k != k || out->hadamard != hadamard) return MXFP4_ERR_INVALID_ARG;
  if (rows == 0 || k == 0) return MXFP4_OK;
  if (!x || !out->codes || !out->scales || !aligned(x, 2) || !aligned(out->codes, 16)) return MXFP4_ERR_INVALID_ARG;
  if (fmt == MXFP4_FMT_NV) {
    if (!out->tensor_scale) return MXFP4_ERR_INVALID_ARG;
    const size_t need = mxfp4::quantize_mse_workspace_bytes(fmt, hadamard, R, C, axis);
    if (!workspace || ws_bytes < need || !aligned(workspace, 16)) return MXFP4_ERR_WORKSPACE;
  }
  hipError_t e = mxfp4::launch_quantize_mse(x, R, C, ldx, fmt, hadamard, axis, iters, out->codes, out->scales,
                                            out->tensor_scale, workspace, stream);
  return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP;
}

}  // extern "C"
