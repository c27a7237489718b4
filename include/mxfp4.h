/*
 * mxfp4.h -- C ABI of libmxfp4: microscaling FP4 quantization and the
 * block-scaled FP4 GEMM on AMD Instinct MI355X (gfx950).
 *
 * What the library computes, and where the method comes from (web pages on
 * microscaling FP4, cited by title and section):
 *   - "FP4 All the Way: Fully Quantized Training of LLMs", abstract:
 *     E2M1 elements; NVFP4 = blocks of 16 E2M1 values sharing an E4M3
 *     scale; round-to-nearest on the forward pass and stochastic rounding on
 *     the backward and update passes; weights, activations and gradients
 *     are all quantized, so all three GEMMs of a linear layer run in FP4.
 *   - "Oscillation-Reduced MXFP4 Training for Vision Transformers", abstract:
 *     the MX format quantizes per group with one shared scale per group.
 *   - "Bridging the Gap Between Promise and Performance for Microscaling FP4
 *     Quantization", abstract (and the digest of it, step 3): MXFP4 scales
 *     are powers of two; block-wise (block-diagonal) Hadamard rotations are
 *     fused into the weights offline and applied online to activations;
 *     FP4 GEMM kernels consume the packed operands.
 *
 * Conventions shared by every entry point
 *   - Formats: MXFP4 = blocks of 32 E2M1 codes + one E8M0 byte (2^(b-127));
 *     NVFP4 = blocks of 16 E2M1 codes + one E4M3 byte, plus one FP32 tensor
 *     scale.
 *   - A quantized matrix is contraction-major: [rows, k], row-major.
 *     codes: rows * k/2 bytes, element k of a row in bits 4*(k&1)+3..4*(k&1)
 *     of byte k/2 (even k in the low nibble).  scales: rows * k/bs bytes,
 *     row-major.  NVFP4 tensor_scale: one float.
 *   - Memory: every pointer argument marked "device" is device memory owned
 *     by the caller; the library never allocates, frees or synchronizes, and
 *     keeps no state between calls (all entry points are reentrant).
 *   - Streams: work is enqueued on the caller's stream and is asynchronous;
 *     a fault during execution surfaces at the caller's next synchronization.
 *   - Errors: every entry point returns an mxfp4_status.  Arguments are
 *     checked before anything is launched; a rejected call has no effect.
 *     MXFP4_ERR_HIP reports a failed kernel launch (hipGetLastError).
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXFP4_OK = 0,
    MXFP4_ERR_INVALID_ARG = -1,       /* null pointer, bad enum, negative size, ld too small */
    MXFP4_ERR_UNSUPPORTED_SHAPE = -2, /* contraction length not a multiple of the needed block */
    MXFP4_ERR_FORMAT_MISMATCH = -3,   /* GEMM operands differ in fmt, k or hadamard */
    MXFP4_ERR_WORKSPACE = -4,         /* workspace missing or smaller than required */
    MXFP4_ERR_HIP = -5                /* a HIP launch failed */
} mxfp4_status;

typedef enum { MXFP4_FMT_MX = 0, MXFP4_FMT_NV = 1 } mxfp4_fmt;
typedef enum { MXFP4_RTN = 0, MXFP4_SR = 1 } mxfp4_rounding;

/* A contraction-major quantized matrix [rows, k] (layout above). */
typedef struct {
    int32_t fmt;          /* mxfp4_fmt */
    int32_t hadamard;     /* 1 if the rows were rotated by the 32x32 block Hadamard */
    int64_t rows;
    int64_t k;            /* contraction length */
    uint8_t *codes;       /* device, rows * k/2 bytes */
    uint8_t *scales;      /* device, rows * k/bs bytes */
    float *tensor_scale;  /* device, 1 float for NVFP4; ignored (may be NULL) for MXFP4 */
} mxfp4_tensor;

/* Byte sizes of the codes and scales of a [rows, k] quantized matrix.
 * Fails with UNSUPPORTED_SHAPE if k is not a multiple of the block size
 * (32 for MXFP4, 16 for NVFP4). */
mxfp4_status mxfp4_tensor_bytes(int fmt, int64_t rows, int64_t k,
                                size_t *codes_bytes, size_t *scales_bytes);

/* Workspace needed by mxfp4_quantize for an [R, C] input (0 for MXFP4;
 * NVFP4 needs room for the per-workgroup partial maxima of the tensor-amax
 * pass).  The workspace holds no state between calls. */
mxfp4_status mxfp4_quantize_workspace_bytes(int fmt, int64_t R, int64_t C, int axis,
                                            size_t *bytes);

/* Quantize a bf16 matrix X [R, C] (device, row-major, leading dimension
 * ldx >= C, elements given as raw bf16 bit patterns).
 *
 * Steps (sources as in the file header):
 *   1. (hadamard = 1) rotate each aligned block of 32 along the contraction
 *      axis by the normalised Sylvester Hadamard matrix H/sqrt(32), in FP32
 *      -- "block-wise Hadamard transforms" of the MR-GPTQ paper's abstract;
 *   2. (NVFP4) tensor scale s_t = max|y| / (6 * 448) over the whole tensor;
 *   3. per block absmax and shared scale: MXFP4 E8M0 2^e with e the smallest
 *      integer such that 6 * 2^e >= absmax; NVFP4 E4M3 = the smallest E4M3
 *      value >= absmax / (6 * s_t);
 *   4. scaled element rounded to E2M1: round-to-nearest-even (rounding =
 *      MXFP4_RTN, forward pass) or stochastic rounding with 16 bits of a
 *      Philox4x32-10 stream keyed by seed (rounding = MXFP4_SR, backward and
 *      update passes) -- "FP4 All the Way", abstract;
 *   5. nibble-pack codes and write the scale bytes contiguously.
 *
 * axis = 1: contraction along C; out is [R, C] (rows = R, k = C).
 * axis = 0: contraction along R; out is the transpose [C, R] (rows = C,
 *           k = R).  This is how the backward GEMMs get each operand
 *           quantized along its own contraction axis.
 * out: caller-filled descriptor; out->rows, out->k and out->fmt must match the
 *      call, and out->hadamard is compared with hadamard; codes/scales (and
 *      tensor_scale for NVFP4) must be non-NULL device buffers of the sizes
 *      mxfp4_tensor_bytes reports; codes must be 16-byte aligned.
 * k must be a multiple of the block size, and of 32 when hadamard = 1.
 * Blocks holding a NaN or infinity get the format's NaN scale byte (0xFF for
 * E8M0, 0x7F for E4M3) and all-zero codes.
 * workspace: device, at least mxfp4_quantize_workspace_bytes (may be NULL
 * when that is 0). */
mxfp4_status mxfp4_quantize(const uint16_t *x, int64_t R, int64_t C, int64_t ldx,
                            int fmt, int rounding, int hadamard, int axis, uint64_t seed,
                            mxfp4_tensor *out, void *workspace, size_t ws_bytes,
                            hipStream_t stream);

/* mxfp4_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and the same output bits, with no workspace argument.
 * The NVFP4 tensor-amax partials go to a static device array inside the
 * library instead: 1 MiB per device (262144 partials, one per 16 Ki input
 * elements), held by each device the library runs on until the process
 * ends.  Inputs whose partials would not fit (mxfp4_quantize_workspace_bytes
 * above 1 MiB, i.e. NVFP4 tensors of more than about 4.29e9 elements) are
 * rejected with MXFP4_ERR_WORKSPACE before anything is launched.  Calls on
 * one device share that array: calls that overlap on one device (other
 * streams, other host threads) race on it and must be serialized by the
 * caller.  The call allocates and frees nothing; the first call on a device
 * looks the array's address up (MXFP4_ERR_HIP if that fails).  MXFP4 needs no
 * scratch. */
mxfp4_status mxfp4_quantize_noalloc(const uint16_t *x, int64_t R, int64_t C, int64_t ldx,
                                    int fmt, int rounding, int hadamard, int axis, uint64_t seed,
                                    mxfp4_tensor *out, hipStream_t stream);

/* Dequantize q into y [q->rows, q->k] FP32 (device, leading dimension ldy >=
 * q->k): value = E2M1(code) * scale (NVFP4: * tensor_scale).  A rotated
 * tensor stays in the rotated domain. */
mxfp4_status mxfp4_dequantize(const mxfp4_tensor *q, float *y, int64_t ldy,
                              hipStream_t stream);

/* Workspace needed by mxfp4_gemm for these operands (split-K partial sums
 * for long contractions; 0 otherwise). */
mxfp4_status mxfp4_gemm_workspace_bytes(const mxfp4_tensor *A, const mxfp4_tensor *B,
                                        size_t *bytes);

/* C[M, N] = A * B^T, FP32, over the dequantized operands: A is [M, k], B is
 * [N, k], both quantized along k (the three GEMMs of a linear layer -- XW^T,
 * dY.W and dY^T.X -- are all this call on operands quantized with the axis
 * that puts their contraction last).  MXFP4 runs on the CDNA4 block-scaled
 * FP4 matrix cores; NVFP4 dequantizes exactly to fp16 in registers (an
 * E2M1 x E4M3 product has at most 6 significant bits) for the fp16 matrix
 * cores and applies both tensor scales in the epilogue.
 * C: device, row-major, ldc >= N, 4-byte aligned.  k must be a multiple of 128 and at most
 * 2^24 (UNSUPPORTED_SHAPE otherwise); fmt, k and hadamard of A and B must agree
 * (FORMAT_MISMATCH).  A->codes and B->codes must be 16-byte aligned and the
 * scales 4-byte aligned (INVALID_ARG otherwise).
 * MXFP4 with at most 128 rows of A (decode and small batches) against at
 * least 2048 rows of B, or with few operand bytes per 16 rows of B, streams
 * B once through a kernel of its own, with the contraction split inside each
 * workgroup: no workspace.
 * workspace: device, 4-byte aligned (WORKSPACE otherwise), at least
 *    mxfp4_gemm_workspace_bytes (NULL if 0); with 16-byte alignment, a
 *    16-byte aligned C and N and ldc multiples of 4, the split-K reduction
 *    reads four outputs at a time (same results either way). */
mxfp4_status mxfp4_gemm(const mxfp4_tensor *A, const mxfp4_tensor *B, float *C, int64_t ldc,
                        void *workspace, size_t ws_bytes, hipStream_t stream);

/* mxfp4_gemm with a bf16 C: each element is the FP32 value mxfp4_gemm writes
 * for the same operands, rounded to the nearest bf16 (ties to even; NaN stays
 * NaN, overflow rounds to infinity).  Half the output bytes, for layers whose
 * consumer takes bf16 (the output epilogue named next to the activation
 * prologue in "Bridging the Gap Between Promise and Performance for
 * Microscaling FP4 Quantization", abstract: the quantization costs are fused
 * into the GEMM kernels).  C: device, bf16 bit patterns, row-major, ldc >= N,
 * 2-byte aligned (INVALID_ARG otherwise).  Operands, workspace (the same
 * mxfp4_gemm_workspace_bytes: split-K partial sums stay FP32) and errors as
 * for mxfp4_gemm. */
mxfp4_status mxfp4_gemm_bf16(const mxfp4_tensor *A, const mxfp4_tensor *B, uint16_t *C, int64_t ldc,
                             void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace needed by mxfp4_gemm_quantize for these operands and output: 0
 * when the quantization is fused into the GEMM's epilogue (MXFP4 operands and
 * no K split), else room for the bf16 C (M * N * 2 bytes, padded to 16) and
 * the GEMM's own workspace.  Argument errors as for mxfp4_gemm_quantize. */
mxfp4_status mxfp4_gemm_quantize_workspace_bytes(const mxfp4_tensor *A, const mxfp4_tensor *B, int hadamard,
                                                 const mxfp4_tensor *out, size_t *bytes);

/* GEMM whose output is quantized for the next layer: the output epilogue of
 * the fused pipeline of "Bridging the Gap Between Promise and Performance for
 * Microscaling FP4 Quantization", abstract (quantization costs fused into the
 * FP4 GEMM kernels; the next layer's activations rotated and quantized on the
 * fly).  out = mxfp4_quantize(C, MXFP4, RTN, hadamard, axis 1) of the bf16 C
 * that mxfp4_gemm_bf16 writes for the same operands -- bit for bit: C = A B^T
 * in FP32, rounded to nearest-even bf16, then each aligned block of 32 along
 * a row of C (block Hadamard first when hadamard = 1) gets its E8M0 byte and
 * round-to-nearest codes.  The next layer's GEMM contracts over C's columns,
 * so out is already in its contraction-major layout.  For MXFP4 operands
 * without a K split, the GEMM kernel's epilogue encodes C in registers and
 * writes only codes and scales (0.53 bytes per output instead of 4);
 * otherwise (NVFP4 operands, split contractions, decode shapes) the bf16 C
 * goes through the workspace.  Operands as for mxfp4_gemm; N = B->rows must be a multiple of
 * 32 (UNSUPPORTED_SHAPE).  out: MXFP4 descriptor [A->rows, B->rows] with
 * out->hadamard == hadamard, codes 16-byte aligned (INVALID_ARG otherwise).
 * workspace: device, 16-byte aligned, at least
 * mxfp4_gemm_quantize_workspace_bytes (NULL if that is 0). */
mxfp4_status mxfp4_gemm_quantize(const mxfp4_tensor *A, const mxfp4_tensor *B, int hadamard, mxfp4_tensor *out,
                                 void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace needed by mxfp4_quantize_gemm for activations [M, K] against B:
 * the split-K partial sums when the quantization is fused into the GEMM,
 * else room for the quantized activations (codes, then scales, each padded
 * to 16 bytes) followed by the GEMM's own workspace.  Argument errors as for
 * mxfp4_quantize_gemm. */
mxfp4_status mxfp4_quantize_gemm_workspace_bytes(int64_t M, int64_t K, int hadamard, const mxfp4_tensor *B,
                                                 size_t *bytes);

/* Forward pass of an MXFP4 linear layer with online activation quantization
 * ("Bridging the Gap Between Promise and Performance for Microscaling FP4
 * Quantization", abstract: block-wise Hadamard rotations fused into the
 * weights offline and computed on the fly for the activations, in front of
 * FP4 GEMM kernels):
 *   C[M, N] = Q(x) * B^T,  Q = mxfp4_quantize(x, MXFP4, RTN, hadamard, axis 1),
 * bit for bit the result of mxfp4_quantize followed by mxfp4_gemm on the same
 * input.  Where the GEMM takes the narrow kernel with up to 32 activation
 * rows (long contractions against short weights), each GEMM workgroup
 * quantizes the activation rows of its own contraction range in LDS, so the
 * activations never go through memory as codes and the call is one GEMM
 * launch (plus the split-K reduction); otherwise x is quantized into the
 * workspace first: the decode kernel's shapes, where that kernel after a
 * quantizer pass is faster than the fused one, more rows, whose repeated
 * quantization in every column-tile workgroup would cost more than one
 * quantizer pass, and the rare plans whose contraction split is too long for
 * LDS.
 * x: device, bf16 bit patterns [M, K], row-major, leading dimension ldx >= K.
 * B: the pre-quantized weights [N, K] (MXFP4, B->k == K and B->hadamard ==
 *    hadamard, else FORMAT_MISMATCH); B->codes 16-byte and B->scales 4-byte
 *    aligned (INVALID_ARG otherwise).  K must be a multiple of 128 and at
 *    most 2^24 (UNSUPPORTED_SHAPE).
 * C: device, FP32, row-major, ldc >= N.
 * workspace: device, 16-byte aligned, at least
 *    mxfp4_quantize_gemm_workspace_bytes (NULL if that is 0). */
mxfp4_status mxfp4_quantize_gemm(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int hadamard,
                                 const mxfp4_tensor *B, float *C, int64_t ldc,
                                 void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace needed by mxfp4_quantize_mse (0 for MXFP4; NVFP4: the tensor
 * amax partials, then 16 bytes per unit of 32 contraction elements and per
 * operand row for the tensor-scale sums).  Errors as for mxfp4_quantize_mse. */
mxfp4_status mxfp4_quantize_mse_workspace_bytes(int fmt, int hadamard, int64_t R, int64_t C, int axis,
                                                size_t *bytes);

/* Round-to-nearest quantization with scales fitted for mean squared error
 * (the digest of the MR-GPTQ paper, step 1: the grid is fitted for MSE by
 * optimizing the block scales and the tensor scale in turn).  As read here:
 *   block step:  each block keeps, among the scales at and below its absmax
 *                scale, the one whose round-to-nearest encoding (exactly
 *                mxfp4_quantize(RTN)'s for that scale) has the smallest sum
 *                of (y - Q(y))^2 over its elements, a tie keeping the larger
 *                scale.  Only MXFP4 exponents e0, e0 - 1 and NVFP4 bytes
 *                b0 .. b0 - 5 (b0 the absmax scale) can ever win, and those
 *                are the ones tried; each error is summed in binary64, so
 *                blocks whose candidates tie to within that sum's rounding
 *                may take either;
 *   tensor step: NVFP4 only, the least-squares tensor scale for the block
 *                step's bytes and codes, sum(y p) / sum(p^2) with p = E4M3 x
 *                E2M1 in binary64 in a fixed order, rounded to binary32;
 *   schedule:    block step with the absmax tensor scale, then iters times
 *                (tensor step, block step); iters in [0, 64], ignored for MXFP4.
 * The output is an ordinary quantized tensor (mxfp4_gemm and
 * mxfp4_dequantize take it as is); arguments and layout as mxfp4_quantize
 * (RTN); the same input gives the same bits.  workspace: device, 16-byte
 * aligned, at least mxfp4_quantize_mse_workspace_bytes (NULL if that is 0). */
mxfp4_status mxfp4_quantize_mse(const uint16_t *x, int64_t R, int64_t C, int64_t ldx, int fmt, int hadamard,
                                int axis, int iters, mxfp4_tensor *out, void *workspace, size_t ws_bytes,
                                hipStream_t stream);

/* MXFP4 round-to-nearest with a fixed grid scale: the digest of the MR-GPTQ
 * paper, step 1, says that for MXFP4 with Hadamard rotations one fixed scale of
 * the quantization grid serves every model, without giving it; here it is the
 * argument alpha.  Each block's E8M0 exponent is the smallest e with
 * 6 * 2^e >= RN(alpha * absmax) (binary32 product; an overflowed product takes
 * e = 127), then the elements are rounded to nearest for that scale exactly as
 * mxfp4_quantize(MXFP4, RTN) rounds them (saturating at +-6).  alpha = 1 is
 * mxfp4_quantize's absmax rule; alpha < 1 lets block maxima saturate for a
 * finer grid.  alpha in (0, 65536] (INVALID_ARG otherwise); the block Hadamard
 * is applied first when hadamard = 1 (the setting the page names, not a
 * requirement).  Arguments and layout as mxfp4_quantize with fmt = MXFP4;
 * k % 32 == 0; codes 16-byte aligned.  No workspace. */
mxfp4_status mxfp4_quantize_grid(const uint16_t *x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                                 float alpha, mxfp4_tensor *out, hipStream_t stream);

/* Workspace needed by mxfp4_quantization_noise for the quantized operand q
 * (three doubles per workgroup of the pass; never 0). */
mxfp4_status mxfp4_quantization_noise_workspace_bytes(const mxfp4_tensor *q, size_t *bytes);

/* The two norms of the sqrt(3) threshold of "FP4 All the Way", abstract
 * (quantized training loses effectiveness once the gradient norm falls below
 * about sqrt(3) times the quantization noise), for a tensor q that
 * mxfp4_quantize made from x with this axis:
 *   stats[0] = sum y^2            (the signal),
 *   stats[1] = sum (Q(y) - y)^2   (the quantization noise),
 *   stats[2] = number of elements left out,
 * over the elements y of the quantized operand (the contraction rows of x,
 * rotated when q->hadamard), Q(y) the exactly dequantized value (E2M1 x
 * scale, NVFP4 x tensor scale), in binary64; blocks with a NaN scale byte
 * are left out.  The ratio sqrt(stats[0] / stats[1]) is the one the page
 * compares with sqrt(3).  The sums come from per-workgroup partials added in
 * a fixed order: the same inputs give the same bits.
 * x: device bf16 [R, C] with (R, C) = (q->rows, q->k) for axis 1 and
 *    (q->k, q->rows) for axis 0, leading dimension ldx >= C.
 * q->codes must be 8-byte aligned (INVALID_ARG otherwise).
 * stats: device, 3 doubles (8-byte aligned).
 * workspace: device, 8-byte aligned, at least
 *    mxfp4_quantization_noise_workspace_bytes. */
mxfp4_status mxfp4_quantization_noise(const uint16_t *x, int64_t ldx, int axis, const mxfp4_tensor *q,
                                      double *stats, void *workspace, size_t ws_bytes,
                                      hipStream_t stream);

/* Workspace needed by mxfp4_quantize_noise (the quantizer's, padded to 16
 * bytes, then three doubles per workgroup of the largest launch plan the call
 * can take).  Errors as for mxfp4_quantize. */
mxfp4_status mxfp4_quantize_noise_workspace_bytes(int fmt, int hadamard, int64_t R, int64_t C, int axis,
                                                  size_t *bytes);

/* mxfp4_quantize and the sums of mxfp4_quantization_noise of its output in
 * one pass: the sqrt(3) diagnostic of "FP4 All the Way", abstract, computed
 * while the (typically stochastically rounded) gradient is quantized, so the
 * input is read once.  out receives exactly what mxfp4_quantize writes for
 * the same arguments; stats[0..2] = sum y^2, sum (Q(y) - y)^2 and the number
 * of elements in blocks with a NaN scale byte, in binary64 as
 * mxfp4_quantization_noise defines them (the terms are the same; the sums
 * are added in another fixed order, so the last bits may differ from that
 * call's; the same inputs give the same bits).  Transposed inputs that are
 * not 16-byte aligned (or C % 8 != 0) are quantized, then summed by the
 * separate pass.
 * Arguments as for mxfp4_quantize, plus stats: device, 3 doubles, 8-byte
 * aligned; x must be 2-byte aligned.  workspace: device, 16-byte aligned, at
 * least mxfp4_quantize_noise_workspace_bytes (never 0). */
mxfp4_status mxfp4_quantize_noise(const uint16_t *x, int64_t R, int64_t C, int64_t ldx,
                                  int fmt, int rounding, int hadamard, int axis, uint64_t seed,
                                  mxfp4_tensor *out, double *stats, void *workspace, size_t ws_bytes,
                                  hipStream_t stream);

/* The sqrt(3) test of "FP4 All the Way", abstract (quantized training loses
 * effectiveness once the gradient norm falls below about sqrt(3) times the
 * quantization noise), on the sums of mxfp4_quantization_noise or
 * mxfp4_quantize_noise after the caller has copied them to the host:
 *   *ratio = sqrt(stats[0] / stats[1])   (+infinity when stats[1] = 0),
 *   *below_threshold = 1 if *ratio < sqrt(3), else 0.
 * stats: host, 3 doubles; ratio, below_threshold: host.  INVALID_ARG for a
 * null pointer or a negative or NaN sum.  Pure host arithmetic: no stream, no
 * device access. */
mxfp4_status mxfp4_noise_ratio(const double *stats, double *ratio, int *below_threshold);

/* Q-EMA weight quantization ("Oscillation-Reduced MXFP4 Training for Vision
 * Transformers", abstract, names Q-EMA among the methods that reduce weight
 * oscillation in MXFP4 training; the page gives no rule).  As read here: the
 * forward pass quantizes an exponential moving average of the latent weights
 * instead of the weights themselves, and this call fuses the average's update
 * with the quantization in one pass over memory:
 *   ema <- RN(RN(beta * ema) + RN(c * w)),  c = RN(1 - beta)   (binary32),
 *   out  = MXFP4 round-to-nearest of the new ema along its rows (the
 *          contraction axis of W in X W^T; block Hadamard first when
 *          hadamard = 1), exactly as mxfp4_quantize encodes an input with
 *          those values.
 * w:   device, bf16 latent weights [R, C], row-major, leading dimension
 *      ldw >= C, 16-byte aligned, ldw a multiple of 8.
 * ema: device, binary32 state [R, C] (read, then overwritten with the new
 *      average), leading dimension lde >= C, 16-byte aligned, lde a multiple
 *      of 4.  The caller initializes it (e.g. to the weights).
 * beta in [0, 1] (INVALID_ARG otherwise).  C % 32 == 0 and R * C / 8 < 2^31
 * (UNSUPPORTED_SHAPE otherwise).  out: an MXFP4 descriptor [R, C] with
 * out->hadamard == hadamard (INVALID_ARG otherwise), codes 16-byte aligned.
 * No workspace. */
mxfp4_status mxfp4_qema_quantize(const uint16_t *w, int64_t R, int64_t C, int64_t ldw, float *ema, int64_t lde,
                                 float beta, int hadamard, mxfp4_tensor *out, hipStream_t stream);

/* A static, human-readable description of a status code. */
const char *mxfp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
