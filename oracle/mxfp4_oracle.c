/*
 * mxfp4_oracle.c -- plain, slow CPU oracle for microscaling FP4 quantization
 * and the block-scaled FP4 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; it exists so tests (and the CPU baseline of the benchmark) can
 * check the HIP library against an independent, obviously correct definition.
 * It shares no source, header, table or constant generator with the HIP code.
 *
 * Sources of the method (web pages on microscaling FP4, cited by title and
 * section):
 *   [TJ]  "Oscillation-Reduced MXFP4 Training for Vision Transformers",
 *         abstract: MX = per-group quantization with one shared scale per group.
 *   [FQT] "FP4 All the Way: Fully Quantized Training of LLMs", abstract:
 *         E2M1 elements; NVFP4 = blocks of 16 E2M1 values sharing an E4M3 scale;
 *         round-to-nearest on the forward pass, stochastic rounding on the
 *         backward and update passes.
 *   [MRG] "Bridging the Gap Between Promise and Performance for Microscaling
 *         FP4 Quantization", abstract: MXFP4 scales are powers of two;
 *         block-wise Hadamard transforms, fused into the weights and computed
 *         online for activations.
 *   [DIG] the Russian-language digest of [MRG] (channel post), numbered
 *         steps 1 and 3: scales exist per block and per tensor; activations
 *         are rotated with block-diagonal Hadamard rotations.
 *
 * The pages fix formats and roles, not the arithmetic.  Every step the pages
 * leave open is taken with the plainest reading that the rest supports; each
 * such reading is marked READING below.  Floating-point steps that decide an
 * integer code are taken in IEEE binary32 (the kernel's precision); the
 * GEMM is evaluated in binary64 on the exactly dequantized operands.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math), so every float
 * operation below is one IEEE-754 binary32 round-to-nearest-even operation.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define FMT_MX 0
#define FMT_NV 1
#define RND_RTN 0
#define RND_SR 1

/* ------------------------------------------------------------------ */
/* Bit helpers                                                          */
/* ------------------------------------------------------------------ */
static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

/* bf16 -> fp32 is exact: a bf16 pattern is the top half of an fp32 pattern. */
static float bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* ------------------------------------------------------------------ */
/* E2M1 element [FQT abstract: "FP4 values (E2M1)"]                      */
/* READING: OCP bit layout -- bit 3 sign, bits 2:1 exponent (bias 1),   */
/* bit 0 mantissa; exponent 0 is subnormal (0 or 0.5).                  */
/* ------------------------------------------------------------------ */
double mxo_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* ------------------------------------------------------------------ */
/* E8M0 shared scale of MXFP4 [MRG abstract: power-of-two scale]        */
/* byte b encodes 2^(b-127); 0xFF is NaN.                               */
/* ------------------------------------------------------------------ */
double mxo_e8m0_value(int byte)
{
    if (byte == 0xFF) return NAN;
    return ldexp(1.0, byte - 127);
}

/* READING: the exponent e of a block is the smallest integer with
 * 6 * 2^e >= amax (so the block maximum lands inside the E2M1 range
 * [-6, 6] without clipping), clamped to the E8M0 range [-127, 127];
 * an all-zero block takes e = -127.  Written as the search it is. */
int mxo_mx_scale_exponent(float amax)
{
    if (!(amax > 0.0f)) return -127;
    for (int e = -127; e <= 127; e++)
        if (6.0 * ldexp(1.0, e) >= (double)amax) return e;
    return 127;
}

/* ------------------------------------------------------------------ */
/* E4M3 block scale of NVFP4 [FQT abstract: "shares a scale in E4M3"]  */
/* Bias 7, no infinities, S.1111.111 is NaN, exponent 0 is subnormal.   */
/* ------------------------------------------------------------------ */
double mxo_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);           /* m/8 * 2^-6 */
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* READING: the block scale is the smallest non-negative finite E4M3 value
 * that is >= r (round up, so the scaled block maximum stays within the
 * E2M1 range); r above 448 saturates to 448.  Brute force over the codes
 * in increasing order (0x00..0x7E are increasing for non-negative E4M3). */
int mxo_e4m3_round_up(float r)
{
    for (int b = 0x00; b <= 0x7E; b++)
        if (mxo_e4m3_value(b) >= (double)r) return b;
    return 0x7E;
}

/* ------------------------------------------------------------------ */
/* Round-to-nearest of a scaled element [FQT abstract: round-to-nearest */
/* on the forward pass].                                                */
/* READING: magnitude saturates at 6; the nearest of the 8 magnitudes   */
/* is chosen, ties going to the code with an even (zero) mantissa bit;  */
/* the sign bit is the sign bit of the input (so -0 and small negative  */
/* values give code 0x8).                                               */
/* xs must not be NaN (callers handle non-finite blocks).              */
/* ------------------------------------------------------------------ */
int mxo_rtn_code(double xs)
{
    int sign = signbit(xs) ? 8 : 0;
    double a = fabs(xs);
    if (a > 6.0) a = 6.0;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; c++) {
        double d = fabs(a - mxo_e2m1_value(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    return sign | best;
}

/* ------------------------------------------------------------------ */
/* Stochastic rounding [FQT abstract: stochastic rounding on backward   */
/* and update passes].                                                  */
/* READING: a = min(|xs|, 6).  A grid magnitude is kept as is.  Else    */
/* lo < a < hi are the neighbouring magnitudes, t = floor((a-lo)/(hi-lo)*2^16)
 * and the magnitude rounds up to hi iff rnd16 < t, so that the chance
 * of rounding up is t/2^16, within 2^-16 of (a-lo)/(hi-lo).  Sign as RTN. */
/* ------------------------------------------------------------------ */
int mxo_sr_code(double xs, uint32_t rnd16)
{
    int sign = signbit(xs) ? 8 : 0;
    double a = fabs(xs);
    if (a > 6.0) a = 6.0;
    for (int c = 0; c < 8; c++)
        if (a == mxo_e2m1_value(c)) return sign | c;
    int lo = 0;
    while (mxo_e2m1_value(lo + 1) < a) lo++;        /* grid[lo] < a < grid[lo+1] */
    double glo = mxo_e2m1_value(lo), ghi = mxo_e2m1_value(lo + 1);
    uint32_t t = (uint32_t)floor((a - glo) / (ghi - glo) * 65536.0);
    return sign | ((rnd16 < t) ? lo + 1 : lo);
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:  */
/* As Easy as 1, 2, 3", SC'11): 4x32-bit counter, 2x32-bit key, ten     */
/* rounds, each multiplying words 0 and 2 by the two Philox multipliers, */
/* the key bumped by the two Weyl constants between rounds.              */
/* ------------------------------------------------------------------ */
void mxo_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; round++) {
        uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += W0; k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* READING (random stream of stochastic rounding): element with output
 * logical index L = i*K + k (row i, contraction index k of the quantized,
 * contraction-major output) takes 16 bits of Philox4x32-10 with
 * key = (seed low, seed high) and counter = (g low, g high, axis, 0),
 * g = L / 8; element L uses 16-bit half (L & 1) of word (L & 7) / 2. */
uint32_t mxo_rnd16(uint64_t seed, uint64_t L, int axis)
{
    uint64_t g = L >> 3;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)axis, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    mxo_philox4x32_10(ctr, key, w);
    return (w[(L & 7) >> 1] >> (16 * (L & 1))) & 0xFFFFu;
}

/* ------------------------------------------------------------------ */
/* Block-wise Hadamard rotation [MRG abstract: block-wise Hadamard      */
/* transforms; DIG step 3: block-diagonal Hadamard rotations].          */
/* READING: blocks of 32 along the contraction axis, Sylvester order    */
/* H[i][j] = (-1)^popcount(i & j), normalised by 1/sqrt(32) so the      */
/* rotation is orthonormal.  Evaluated in binary32 as the fast          */
/* Walsh-Hadamard butterfly with strides 1, 2, 4, 8, 16 -- each pair     */
/* (x[i], x[i+h]), i & h == 0, becomes (x[i] + x[i+h], x[i] - x[i+h]) -- */
/* then every entry is multiplied by c = RN_f32(1/sqrt(32)).            */
/* ------------------------------------------------------------------ */
float mxo_hadamard_scale(void) { return (float)(1.0 / sqrt(32.0)); }

void mxo_fwht32(float x[32])
{
    for (int h = 1; h < 32; h <<= 1) {
        for (int i = 0; i < 32; i++) {
            if (i & h) continue;
            float a = x[i], b = x[i + h];
            x[i] = a + b;
            x[i + h] = a - b;
        }
    }
    const float c = mxo_hadamard_scale();
    for (int i = 0; i < 32; i++) x[i] = x[i] * c;
}

/* ------------------------------------------------------------------ */
/* Whole-tensor quantization                                            */
/* ------------------------------------------------------------------ */
/* Logical input X is [R, C] bf16, row-major with leading dimension ldx.
 * axis = 1: the output is [R, C] (contraction along C); axis = 0: the output
 * is [C, R], the transpose (contraction along R).  Output row i holds the
 * contraction vector v_i[k] = X[i][k] (axis 1) or X[k][i] (axis 0).
 * codes:  rows x K/2 bytes, code of k in bits 4*(k&1)+3 .. 4*(k&1).
 * scales: rows x K/bs bytes (E8M0 for MX, E4M3 for NV).
 * tensor_scale: one float (NV only).
 * Returns 0, or -1 on an invalid argument. */

/* Contraction row i of the operand: bf16 input x, or binary32 input xf when
 * x is NULL (used by the EMA quantizer below). */
static void load_row_any(const uint16_t *x, const float *xf, int64_t ldx, int axis,
                         int64_t i, int64_t K, int hadamard, float *v)
{
    for (int64_t k = 0; k < K; k++) {
        const int64_t at = axis == 1 ? i * ldx + k : k * ldx + i;
        v[k] = x ? bf16_to_f32(x[at]) : xf[at];
    }
    if (hadamard)
        for (int64_t k0 = 0; k0 < K; k0 += 32) mxo_fwht32(v + k0);
}

static void load_contraction_row(const uint16_t *x, int64_t ldx, int axis,
                                 int64_t i, int64_t K, int hadamard, float *v)
{
    load_row_any(x, NULL, ldx, axis, i, K, hadamard, v);
}

/* NVFP4 per-tensor scale.  READING: s_t = RN_f32(amax_t / (6 * 448)) so the
 * largest block scale lands on the largest E4M3 value; amax_t is the largest
 * finite |v| over the tensor (after the rotation, if any); s_t = 1 for an
 * all-zero tensor, and s_t is kept at or above 2^-117 so that the per-block
 * product s_b * s_t (s_b >= 2^-9) stays a normal binary32 number. */
float mxo_nv_tensor_scale(float amax_t)
{
    if (!(amax_t > 0.0f)) return 1.0f;
    float st = amax_t / 2688.0f;
    const float floor_st = ldexpf(1.0f, -117);
    return st < floor_st ? floor_st : st;
}

/* l0: stream index of the operand's element (0, 0); 0 for a whole tensor
 * (mxo_quantize), row0 * K for rows row0.. of a larger MXFP4 tensor
 * quantized along axis 1 (mxo_quantize_rows_at). */
static int quantize_impl(const uint16_t *x, const float *xf, int64_t R, int64_t C, int64_t ldx,
                         int fmt, int rounding, int hadamard, int axis, uint64_t seed,
                         uint64_t l0, uint8_t *codes, uint8_t *scales, float *tensor_scale)
{
    if ((!x && !xf) || !codes || !scales || R < 0 || C < 0 || ldx < C) return -1;
    if (fmt != FMT_MX && fmt != FMT_NV) return -1;
    if (rounding != RND_RTN && rounding != RND_SR) return -1;
    if (axis != 0 && axis != 1) return -1;
    if (fmt == FMT_NV && !tensor_scale) return -1;
    const int bs = (fmt == FMT_MX) ? 32 : 16;
    const int64_t rows = (axis == 1) ? R : C;
    const int64_t K = (axis == 1) ? C : R;
    if (K % bs != 0 || (hadamard && K % 32 != 0)) return -1;
    if (rows == 0 || K == 0) {
        if (fmt == FMT_NV) *tensor_scale = 1.0f;
        return 0;
    }

    /* NVFP4: the tensor scale needs the whole tensor's amax first. */
    float st = 1.0f;
    if (fmt == FMT_NV) {
        float amax_t = 0.0f;
        #pragma omp parallel
        {
            float *v = (float *)malloc(sizeof(float) * K);
            float local = 0.0f;
            #pragma omp for
            for (int64_t i = 0; i < rows; i++) {
                load_row_any(x, xf, ldx, axis, i, K, hadamard, v);
                for (int64_t k = 0; k < K; k++) {
                    float a = fabsf(v[k]);
                    if (isfinite(a) && a > local) local = a;
                }
            }
            #pragma omp critical
            if (local > amax_t) amax_t = local;
            free(v);
        }
        st = mxo_nv_tensor_scale(amax_t);
        *tensor_scale = st;
    }

    #pragma omp parallel
    {
        float *v = (float *)malloc(sizeof(float) * K);
        #pragma omp for
        for (int64_t i = 0; i < rows; i++) {
            load_row_any(x, xf, ldx, axis, i, K, hadamard, v);
            for (int64_t b = 0; b < K / bs; b++) {
                const float *blk = v + b * bs;
                /* block absmax; a non-finite entry makes the block NaN */
                float amax = 0.0f;
                int finite = 1;
                for (int j = 0; j < bs; j++) {
                    if (!isfinite(blk[j])) finite = 0;
                    else if (fabsf(blk[j]) > amax) amax = fabsf(blk[j]);
                }
                int scale_byte;
                double mx_step = 0.0;   /* MX: 2^-e */
                float nv_inv = 0.0f;    /* NV: RN(1 / RN(s_b * s_t)), 0 if s_b = 0 */
                if (!finite) {
                    scale_byte = (fmt == FMT_MX) ? 0xFF : 0x7F;
                } else if (fmt == FMT_MX) {
                    int e = mxo_mx_scale_exponent(amax);
                    scale_byte = e + 127;
                    mx_step = ldexp(1.0, -e);
                } else {
                    float den = 6.0f * st;
                    float r = amax / den;
                    scale_byte = mxo_e4m3_round_up(r);
                    if (scale_byte != 0) {
                        float sb = (float)mxo_e4m3_value(scale_byte);
                        float d = sb * st;
                        nv_inv = 1.0f / d;
                    }
                }
                scales[i * (K / bs) + b] = (uint8_t)scale_byte;
                for (int j = 0; j < bs; j++) {
                    int64_t k = b * bs + j;
                    int code;
                    if (!finite) {
                        code = 0;
                    } else {
                        double xs;
                        if (fmt == FMT_MX) {
                            xs = (double)blk[j] * mx_step;          /* exact */
                        } else if (scale_byte == 0) {
                            xs = copysign(0.0, (double)blk[j]);
                        } else {
                            float q = blk[j] * nv_inv;              /* one binary32 multiply */
                            xs = (double)q;
                        }
                        if (rounding == RND_RTN)
                            code = mxo_rtn_code(xs);
                        else
                            code = mxo_sr_code(xs, mxo_rnd16(seed, l0 + (uint64_t)(i * K + k), axis));
                    }
                    uint8_t *byte = &codes[i * (K / 2) + k / 2];
                    if ((k & 1) == 0) *byte = (uint8_t)((*byte & 0xF0) | code);
                    else *byte = (uint8_t)((*byte & 0x0F) | (code << 4));
                }
            }
        }
        free(v);
    }
    return 0;
}

int mxo_quantize(const uint16_t *x, int64_t R, int64_t C, int64_t ldx,
                 int fmt, int rounding, int hadamard, int axis, uint64_t seed,
                 uint8_t *codes, uint8_t *scales, float *tensor_scale)
{
    return quantize_impl(x, NULL, R, C, ldx, fmt, rounding, hadamard, axis, seed, 0, codes, scales, tensor_scale);
}

/* The same quantizer on a binary32 input (the values are used as they are;
 * for bf16-representable values it equals mxo_quantize bit for bit). */
int mxo_quantize_f32(const float *x, int64_t R, int64_t C, int64_t ldx,
                     int fmt, int rounding, int hadamard, int axis, uint64_t seed,
                     uint8_t *codes, uint8_t *scales, float *tensor_scale)
{
    if (!x) return -1;
    return quantize_impl(NULL, x, R, C, ldx, fmt, rounding, hadamard, axis, seed, 0, codes, scales, tensor_scale);
}

/* Rows row0 .. row0 + R - 1 of a larger tensor, MXFP4 along axis 1: every
 * block lies in one row, so only the stochastic-rounding stream index needs
 * the offset (NVFP4 would need the whole tensor's amax, and is refused). */
int mxo_quantize_rows_at(const uint16_t *x, int64_t R, int64_t C, int64_t ldx, int rounding, int hadamard,
                         uint64_t seed, int64_t row0, uint8_t *codes, uint8_t *scales)
{
    if (row0 < 0) return -1;
    return quantize_impl(x, NULL, R, C, ldx, FMT_MX, rounding, hadamard, 1, seed, (uint64_t)row0 * (uint64_t)C,
                         codes, scales, NULL);
}

/* ------------------------------------------------------------------ */
/* Dequantization: value = E2M1(code) * scale (NV: * tensor scale).     */
/* MX in binary32 is exact unless it leaves the binary32 range.  NV is  */
/* RN(RN(E2M1 * s_b) * s_t); the inner product is exact.                */
/* Rotated tensors stay in the rotated domain (READING).               */
/* ------------------------------------------------------------------ */
int mxo_dequantize(int fmt, int64_t rows, int64_t K, const uint8_t *codes,
                   const uint8_t *scales, const float *tensor_scale, float *y, int64_t ldy)
{
    if (fmt != FMT_MX && fmt != FMT_NV) return -1;
    const int bs = (fmt == FMT_MX) ? 32 : 16;
    if (K % bs != 0 || ldy < K) return -1;
    #pragma omp parallel for
    for (int64_t i = 0; i < rows; i++) {
        for (int64_t k = 0; k < K; k++) {
            int code = (codes[i * (K / 2) + k / 2] >> (4 * (k & 1))) & 0xF;
            int sbyte = scales[i * (K / bs) + k / bs];
            float v;
            if (fmt == FMT_MX) {
                v = (float)(mxo_e2m1_value(code) * mxo_e8m0_value(sbyte));
            } else {
                float g_sb = (float)(mxo_e2m1_value(code) * mxo_e4m3_value(sbyte));
                v = g_sb * tensor_scale[0];
            }
            y[i * ldy + k] = v;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Block-scaled GEMM, C = A * B^T over the contraction axis, evaluated  */
/* in binary64 on the exactly dequantized operands (E2M1 * scale, NV:   */
/* * tensor scale -- at most 30 significant bits, exact in binary64).   */
/* S = sum of |a*b|, the scale of the admissible error.                 */
/* Computes the sub-matrix rows ri[0..nr) x columns cj[0..nc).           */
/* ------------------------------------------------------------------ */
static double exact_operand(int fmt, const uint8_t *codes, const uint8_t *scales,
                            const float *ts, int64_t K, int64_t i, int64_t k)
{
    const int bs = (fmt == FMT_MX) ? 32 : 16;
    int code = (codes[i * (K / 2) + k / 2] >> (4 * (k & 1))) & 0xF;
    int sbyte = scales[i * (K / bs) + k / bs];
    if (fmt == FMT_MX) return mxo_e2m1_value(code) * mxo_e8m0_value(sbyte);
    return mxo_e2m1_value(code) * mxo_e4m3_value(sbyte) * (double)ts[0];
}

int mxo_gemm(int fmt, int64_t K,
             const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ts,
             const uint8_t *b_codes, const uint8_t *b_scales, const float *b_ts,
             const int64_t *ri, int64_t nr, const int64_t *cj, int64_t nc,
             double *Cout, double *Sout)
{
    if (fmt != FMT_MX && fmt != FMT_NV) return -1;
    const int bs = (fmt == FMT_MX) ? 32 : 16;
    if (K % bs != 0) return -1;
    if (nr == 0 || nc == 0) return 0;
    /* the selected rows of A, dequantized once */
    double *arows = (double *)malloc(sizeof(double) * (size_t)nr * (size_t)(K > 0 ? K : 1));
    if (!arows) return -1;
    #pragma omp parallel for
    for (int64_t p = 0; p < nr; p++)
        for (int64_t k = 0; k < K; k++)
            arows[p * K + k] = exact_operand(fmt, a_codes, a_scales, a_ts, K, ri[p], k);
    #pragma omp parallel
    {
        double *brow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        #pragma omp for
        for (int64_t q = 0; q < nc; q++) {
            for (int64_t k = 0; k < K; k++)
                brow[k] = exact_operand(fmt, b_codes, b_scales, b_ts, K, cj[q], k);
            for (int64_t p = 0; p < nr; p++) {
                const double *arow = arows + p * K;
                double c = 0.0, s = 0.0;
                for (int64_t k = 0; k < K; k++) {
                    double prod = arow[k] * brow[k];
                    c += prod;
                    s += fabs(prod);
                }
                Cout[p * nc + q] = c;
                Sout[p * nc + q] = s;
            }
        }
        free(brow);
    }
    free(arows);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Quantization noise against the signal, the quantities of the         */
/* threshold in [FQT] abstract (quantized training loses effectiveness  */
/* once the gradient norm falls below about sqrt(3) times the            */
/* quantization noise).  READING: the signal is the quantized operand   */
/* itself, y = the contraction rows of x (rotated when hadamard), and   */
/* the noise is Q(y) - y with Q(y) the exactly dequantized value        */
/* (E2M1 * scale, NV: * tensor scale, exact in binary64).  Blocks with  */
/* a non-finite element (NaN scale byte) are left out and counted.      */
/*   out[0] = sum y^2, out[1] = sum (Q(y) - y)^2   (binary64, row order) */
/*   out[2] = number of elements left out.                               */
/* ------------------------------------------------------------------ */
int mxo_noise_stats(const uint16_t *x, int64_t R, int64_t C, int64_t ldx,
                    int fmt, int hadamard, int axis,
                    const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                    double *out)
{
    if (!x || !codes || !scales || !out || R < 0 || C < 0 || ldx < C) return -1;
    if ((fmt != FMT_MX && fmt != FMT_NV) || (axis != 0 && axis != 1)) return -1;
    if (fmt == FMT_NV && !tensor_scale) return -1;
    const int bs = (fmt == FMT_MX) ? 32 : 16;
    const int64_t rows = (axis == 1) ? R : C;
    const int64_t K = (axis == 1) ? C : R;
    if (K % bs != 0 || (hadamard && K % 32 != 0)) return -1;
    out[0] = out[1] = out[2] = 0.0;
    if (rows == 0 || K == 0) return 0;
    double *row_s0 = (double *)calloc((size_t)rows, sizeof(double));
    double *row_s1 = (double *)calloc((size_t)rows, sizeof(double));
    double *row_n = (double *)calloc((size_t)rows, sizeof(double));
    #pragma omp parallel
    {
        float *v = (float *)malloc(sizeof(float) * K);
        #pragma omp for
        for (int64_t i = 0; i < rows; i++) {
            load_contraction_row(x, ldx, axis, i, K, hadamard, v);
            double s0 = 0.0, s1 = 0.0, n = 0.0;
            for (int64_t b = 0; b < K / bs; b++) {
                int sbyte = scales[i * (K / bs) + b];
                int nan_scale = (fmt == FMT_MX) ? (sbyte == 0xFF) : ((sbyte & 0x7F) == 0x7F);
                if (nan_scale) { n += bs; continue; }
                for (int j = 0; j < bs; j++) {
                    int64_t k = b * bs + j;
                    int code = (codes[i * (K / 2) + k / 2] >> (4 * (k & 1))) & 0xF;
                    double q = mxo_e2m1_value(code) * (fmt == FMT_MX ? mxo_e8m0_value(sbyte)
                                                                      : mxo_e4m3_value(sbyte) * (double)tensor_scale[0]);
                    double yk = (double)v[k];
                    double d = q - yk;
                    s0 += yk * yk;
                    s1 += d * d;
                }
            }
            row_s0[i] = s0;
            row_s1[i] = s1;
            row_n[i] = n;
        }
        free(v);
    }
    for (int64_t i = 0; i < rows; i++) {
        out[0] += row_s0[i];
        out[1] += row_s1[i];
        out[2] += row_n[i];
    }
    free(row_s0);
    free(row_s1);
    free(row_n);
    return 0;
}

/* ------------------------------------------------------------------ */
/* MSE-fitted scales [DIG step 1: the quantization grid is fitted for   */
/* mean squared error by optimizing, in turn, the scales of each block  */
/* and the scale of the tensor].  READINGS (the page gives the idea,    */
/* not the procedure):                                                  */
/*  - round-to-nearest only (a forward / weight quantizer);             */
/*  - block step: among every scale value at or below the block's       */
/*    absmax scale (MX: 2^e for e = e0, e0 - 1, ..., -127; NV: the E4M3  */
/*    bytes b0, b0 - 1, ..., 1 times the tensor scale), the block keeps  */
/*    the one whose round-to-nearest encoding -- exactly the absmax     */
/*    quantizer's encoding for that scale -- has the smallest squared   */
/*    error sum (y - Q(y))^2 over the block, Q(y) the exactly           */
/*    dequantized value; a tie keeps the larger scale.  Larger scales   */
/*    are not candidates: below the block maximum their grids hold no   */
/*    point the absmax grid lacks (MX: {0,1,2,3,4,6} 2^(e0+1) is a      */
/*    subset of the e0 grid), so they only coarsen it;                  */
/*  - the error of a candidate is exact up to a final rounding: each    */
/*    difference y - Q(y) is exact in binary64 (at most ~36 significant */
/*    bits), its square exact in binary128, and the block's squares are */
/*    added in binary128, elements in turn;                             */
/*  - the search walks the scales downwards and stops once the clipping */
/*    of the block maximum alone, (amax - 6 s)^2 for a grid top 6 s      */
/*    below amax, exceeds the best error found: that term only grows as */
/*    s falls, so no smaller scale can win (an exact cut, not a window);*/
/*  - tensor step (NV): with block bytes b and codes g fixed, the least */
/*    squares tensor scale sum(y p) / sum(p^2), p = E4M3(b) E2M1(g);    */
/*    each product is exact in binary64 and added in binary128, elements*/
/*    of a row in turn, then the rows in turn; blocks with a NaN scale  */
/*    are left out; the quotient is rounded once to binary32 and kept   */
/*    >= 2^-117; the scale is unchanged when sum(y p) <= 0;             */
/*  - schedule: block step with the absmax tensor scale, then `iters`   */
/*    times (tensor step, block step).  MX has no tensor step.          */
/* ------------------------------------------------------------------ */
typedef __float128 q128;

/* Codes of one block for MX exponent e (scale 2^e), or for NV byte b under
 * tensor scale st, encoded as the absmax quantizer encodes them; returns the
 * block's squared error in binary128. */
static q128 mx_candidate(const float *y, int bs, int e, int *codes)
{
    const double step = ldexp(1.0, -e), sc = ldexp(1.0, e);
    q128 E = 0;
    for (int j = 0; j < bs; j++) {
        codes[j] = mxo_rtn_code((double)y[j] * step);
        double d = (double)y[j] - mxo_e2m1_value(codes[j]) * sc;      /* exact */
        E += (q128)d * (q128)d;
    }
    return E;
}

static q128 nv_candidate(const float *y, int bs, int b, float st, int *codes)
{
    const float sb = (float)mxo_e4m3_value(b);
    const float d32 = sb * st;
    const float inv = 1.0f / d32;
    q128 E = 0;
    for (int j = 0; j < bs; j++) {
        float q = y[j] * inv;                                          /* one binary32 multiply */
        codes[j] = mxo_rtn_code((double)q);
        double d = (double)y[j] - mxo_e2m1_value(codes[j]) * (double)sb * (double)st;   /* exact */
        E += (q128)d * (q128)d;
    }
    return E;
}

/* Absmax of a block; 0 if it holds a non-finite value. */
static int block_amax(const float *y, int bs, float *amax)
{
    *amax = 0.0f;
    for (int j = 0; j < bs; j++) {
        if (!isfinite(y[j])) return 0;
        if (fabsf(y[j]) > *amax) *amax = fabsf(y[j]);
    }
    return 1;
}

/* The absmax scale of a finite block: MX exponent e0, NV byte b0. */
static int absmax_scale(int fmt, float amax, float st)
{
    if (fmt == FMT_MX) return mxo_mx_scale_exponent(amax);
    float den = 6.0f * st;
    float r = amax / den;
    return mxo_e4m3_round_up(r);
}

/* The block step for one finite block: scale byte, codes and the smallest
 * squared error (binary128). */
static void mse_block(int fmt, const float *y, float st, int *byte_out, int *codes, q128 *err_out)
{
    const int bs = (fmt == FMT_MX) ? 32 : 16;
    float amax;
    int cand[32];
    block_amax(y, bs, &amax);
    const int top = absmax_scale(fmt, amax, st);
    if (fmt == FMT_NV && top == 0) {
        /* the block's absmax maps to scale 0: every code is a signed zero */
        *byte_out = 0;
        q128 E = 0;
        for (int j = 0; j < bs; j++) {
            codes[j] = mxo_rtn_code(copysign(0.0, (double)y[j]));
            E += (q128)y[j] * (q128)y[j];
        }
        *err_out = E;
        return;
    }
    const int lowest = (fmt == FMT_MX) ? -127 : 1;
    q128 best = 0;
    int have = 0;
    for (int s = top; s >= lowest; s--) {
        const double grid_top = (fmt == FMT_MX) ? 6.0 * ldexp(1.0, s)
                                                : 6.0 * mxo_e4m3_value(s) * (double)st;
        if (have && grid_top < (double)amax) {
            const q128 clip = ((q128)amax - (q128)grid_top) * ((q128)amax - (q128)grid_top);
            if (clip > best) break;
        }
        q128 E = (fmt == FMT_MX) ? mx_candidate(y, bs, s, cand) : nv_candidate(y, bs, s, st, cand);
        if (!have || E < best) {
            have = 1;
            best = E;
            *byte_out = (fmt == FMT_MX) ? s + 127 : s;
            for (int j = 0; j < bs; j++) codes[j] = cand[j];
        }
    }
    *err_out = best;
}

/* The operand's contraction rows, rotated once: rows x K floats. */
static float *load_operand(const uint16_t *x, int64_t ldx, int hadamard, int axis, int64_t rows, int64_t K)
{
    float *Y = (float *)malloc(sizeof(float) * (size_t)rows * (size_t)K);
    if (!Y) return NULL;
    #pragma omp parallel for
    for (int64_t i = 0; i < rows; i++) load_contraction_row(x, ldx, axis, i, K, hadamard, Y + i * K);
    return Y;
}

/* Least-squares tensor scale for fixed bytes and codes (NV); st_prev when
 * sum(y p) <= 0. */
static float ls_tensor_scale(const float *Y, int64_t rows, int64_t K, const uint8_t *codes,
                             const uint8_t *scales, float st_prev)
{
    const int bs = 16;
    q128 *rn = (q128 *)malloc(sizeof(q128) * (size_t)rows);
    q128 *rd = (q128 *)malloc(sizeof(q128) * (size_t)rows);
    #pragma omp parallel for
    for (int64_t i = 0; i < rows; i++) {
        q128 sn = 0, sd = 0;
        for (int64_t k = 0; k < K; k++) {
            int sbyte = scales[i * (K / bs) + k / bs];
            if ((sbyte & 0x7F) == 0x7F) continue;
            int code = (codes[i * (K / 2) + k / 2] >> (4 * (k & 1))) & 0xF;
            double p = mxo_e2m1_value(code) * mxo_e4m3_value(sbyte);     /* exact */
            sn += (q128)((double)Y[i * K + k] * p);                      /* exact product */
            sd += (q128)(p * p);
        }
        rn[i] = sn;
        rd[i] = sd;
    }
    q128 num = 0, den = 0;
    for (int64_t i = 0; i < rows; i++) {
        num += rn[i];
        den += rd[i];
    }
    free(rn);
    free(rd);
    if (!(num > 0) || !(den > 0)) return st_prev;
    float s = (float)(num / den);
    const float floor_st = ldexpf(1.0f, -117);
    return s < floor_st ? floor_st : s;
}

static void put_code(uint8_t *codes, int64_t K, int64_t i, int64_t k, int c)
{
    uint8_t *cb = &codes[i * (K / 2) + k / 2];
    if ((k & 1) == 0) *cb = (uint8_t)((*cb & 0xF0) | c);
    else *cb = (uint8_t)((*cb & 0x0F) | (c << 4));
}

static int get_code(const uint8_t *codes, int64_t K, int64_t i, int64_t k)
{
    return (codes[i * (K / 2) + k / 2] >> (4 * (k & 1))) & 0xF;
}

static float tensor_absmax_scale(const float *Y, int64_t n)
{
    float amax_t = 0.0f;
    for (int64_t t = 0; t < n; t++) {
        float a = fabsf(Y[t]);
        if (isfinite(a) && a > amax_t) amax_t = a;
    }
    return mxo_nv_tensor_scale(amax_t);
}

int mxo_quantize_mse(const uint16_t *x, int64_t R, int64_t C, int64_t ldx,
                     int fmt, int hadamard, int axis, int iters,
                     uint8_t *codes, uint8_t *scales, float *tensor_scale)
{
    if (!x || !codes || !scales || R < 0 || C < 0 || ldx < C || iters < 0) return -1;
    if ((fmt != FMT_MX && fmt != FMT_NV) || (axis != 0 && axis != 1)) return -1;
    if (fmt == FMT_NV && !tensor_scale) return -1;
    const int bs = (fmt == FMT_MX) ? 32 : 16;
    const int64_t rows = (axis == 1) ? R : C;
    const int64_t K = (axis == 1) ? C : R;
    if (K % bs != 0 || (hadamard && K % 32 != 0)) return -1;
    if (rows == 0 || K == 0) {
        if (fmt == FMT_NV) *tensor_scale = 1.0f;
        return 0;
    }
    float *Y = load_operand(x, ldx, hadamard, axis, rows, K);
    if (!Y) return -1;
    float st = (fmt == FMT_NV) ? tensor_absmax_scale(Y, rows * K) : 1.0f;
    for (int round = 0; round <= iters; round++) {
        if (round > 0 && fmt == FMT_NV) st = ls_tensor_scale(Y, rows, K, codes, scales, st);
        if (round > 0 && fmt == FMT_MX) break;
        /* block step */
        #pragma omp parallel for
        for (int64_t i = 0; i < rows; i++) {
            int cs[32];
            for (int64_t b = 0; b < K / bs; b++) {
                const float *y = Y + i * K + b * bs;
                float amax;
                int byte = 0;
                if (!block_amax(y, bs, &amax)) {
                    byte = (fmt == FMT_MX) ? 0xFF : 0x7F;
                    for (int j = 0; j < bs; j++) cs[j] = 0;
                } else {
                    q128 E;
                    mse_block(fmt, y, st, &byte, cs, &E);
                }
                scales[i * (K / bs) + b] = (uint8_t)byte;
                for (int j = 0; j < bs; j++) put_code(codes, K, i, b * bs + j, cs[j]);
            }
        }
    }
    if (fmt == FMT_NV) *tensor_scale = st;
    free(Y);
    return 0;
}

/* Check a quantized tensor that claims to be the block step of the MSE
 * quantizer for x under tensor scale st (st ignored for MX).  A block passes
 * when (1) a non-finite block has the NaN byte and zero codes; otherwise
 * (2) its byte is a candidate (a scale at or below its absmax scale; NV:
 * byte 0 only when the absmax scale is byte 0), (3) its codes are the
 * round-to-nearest encoding for its byte, and (4) its squared error is at
 * most (1 + rel_tol) times the smallest over all candidates (several bytes
 * are correct when errors tie to within the rounding of a binary64 sum).
 * out[0] blocks, out[1] blocks failing (1)-(3), out[2] blocks failing (4),
 * out[3] blocks whose byte differs from the oracle's own choice (near ties),
 * out[4] the first failing block (row-major over [rows, K / bs]) or -1. */
int mxo_mse_check(const uint16_t *x, int64_t R, int64_t C, int64_t ldx, int fmt, int hadamard, int axis,
                  float st, const uint8_t *codes, const uint8_t *scales, double rel_tol, int64_t *out)
{
    if (!x || !codes || !scales || !out || R < 0 || C < 0 || ldx < C) return -1;
    if ((fmt != FMT_MX && fmt != FMT_NV) || (axis != 0 && axis != 1)) return -1;
    const int bs = (fmt == FMT_MX) ? 32 : 16;
    const int64_t rows = (axis == 1) ? R : C;
    const int64_t K = (axis == 1) ? C : R;
    if (K % bs != 0 || (hadamard && K % 32 != 0)) return -1;
    for (int t = 0; t < 4; t++) out[t] = 0;
    out[4] = -1;
    if (rows == 0 || K == 0) return 0;
    float *Y = load_operand(x, ldx, hadamard, axis, rows, K);
    if (!Y) return -1;
    const int64_t nb = K / bs;
    int64_t bad_enc = 0, bad_err = 0, differ = 0, first = -1;
    #pragma omp parallel for reduction(+:bad_enc, bad_err, differ)
    for (int64_t i = 0; i < rows; i++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *y = Y + i * K + b * bs;
            const int byte = scales[i * nb + b];
            int got[32], cand[32], best_codes[32];
            for (int j = 0; j < bs; j++) got[j] = get_code(codes, K, i, b * bs + j);
            int enc_ok = 1, err_ok = 1;
            float amax;
            if (!block_amax(y, bs, &amax)) {
                enc_ok = byte == ((fmt == FMT_MX) ? 0xFF : 0x7F);
                for (int j = 0; j < bs; j++) enc_ok = enc_ok && got[j] == 0;
            } else {
                int best_byte = 0;
                q128 Emin;
                mse_block(fmt, y, st, &best_byte, best_codes, &Emin);
                const int top = absmax_scale(fmt, amax, st);
                q128 E = 0;
                if (fmt == FMT_MX) {
                    const int e = byte - 127;
                    if (byte == 0xFF || e > top || e < -127) enc_ok = 0;
                    else E = mx_candidate(y, bs, e, cand);
                } else if (top == 0) {
                    enc_ok = byte == 0;
                    for (int j = 0; j < bs; j++) cand[j] = mxo_rtn_code(copysign(0.0, (double)y[j]));
                    E = Emin;
                } else {
                    if (byte < 1 || byte > top) enc_ok = 0;
                    else E = nv_candidate(y, bs, byte, st, cand);
                }
                if (enc_ok)
                    for (int j = 0; j < bs; j++) enc_ok = enc_ok && got[j] == cand[j];
                if (enc_ok) err_ok = E <= Emin * (q128)(1.0 + rel_tol);
                if (enc_ok && byte != best_byte) differ++;
            }
            if (!enc_ok) bad_enc++;
            else if (!err_ok) bad_err++;
            if (!enc_ok || !err_ok) {
                #pragma omp critical
                if (first < 0 || i * nb + b < first) first = i * nb + b;
            }
        }
    }
    out[1] = bad_enc;
    out[2] = bad_err;
    out[3] = differ;
    out[0] = rows * nb;
    out[4] = first;
    free(Y);
    return 0;
}

/* The tensor step of the MSE quantizer (NV) for given bytes and codes of x's
 * quantization: the least-squares tensor scale, or st_prev when
 * sum(y p) <= 0.  Returns 0, or -1 on an invalid argument. */
int mxo_mse_tensor_step(const uint16_t *x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                        const uint8_t *codes, const uint8_t *scales, float st_prev, float *st_out)
{
    if (!x || !codes || !scales || !st_out || R < 0 || C < 0 || ldx < C || (axis != 0 && axis != 1)) return -1;
    const int64_t rows = (axis == 1) ? R : C;
    const int64_t K = (axis == 1) ? C : R;
    if (K % 16 != 0 || (hadamard && K % 32 != 0)) return -1;
    if (rows == 0 || K == 0) {
        *st_out = st_prev;
        return 0;
    }
    float *Y = load_operand(x, ldx, hadamard, axis, rows, K);
    if (!Y) return -1;
    *st_out = ls_tensor_scale(Y, rows, K, codes, scales, st_prev);
    free(Y);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Q-EMA weight quantizer [TJ abstract: Q-EMA is named among the methods */
/* that reduce weight oscillation in MXFP4 training; the page gives no   */
/* rule].  PARITY UNPINNED as to the method: the rule below is this      */
/* build's reading, pinned only for its own arithmetic.                  */
/* READING: the quantized weights come from an exponential moving        */
/* average m of the latent weights w instead of w itself.  One call:     */
/*   m <- RN(RN(beta * m) + RN(c * w)),  c = RN_f32(1 - beta),           */
/* in binary32, w the bf16 latent weights [R, C] widened exactly, m the  */
/* binary32 state [R, C] (updated in place, leading dimension lde), then */
/* the updated m is quantized to MXFP4 round-to-nearest along its rows   */
/* (the contraction axis of W in X W^T), with the block Hadamard first   */
/* when hadamard = 1, exactly as mxo_quantize_f32 quantizes it.          */
/* ------------------------------------------------------------------ */
int mxo_qema_quantize(const uint16_t *w, int64_t R, int64_t C, int64_t ldw, float *ema, int64_t lde,
                      float beta, int hadamard, uint8_t *codes, uint8_t *scales)
{
    if (!w || !ema || !codes || !scales || R < 0 || C < 0 || ldw < C || lde < C) return -1;
    if (!(beta >= 0.0f && beta <= 1.0f) || C % 32 != 0) return -1;
    const float c = 1.0f - beta;
    #pragma omp parallel for
    for (int64_t i = 0; i < R; i++)
        for (int64_t k = 0; k < C; k++) {
            float a = beta * ema[i * lde + k];
            float b = c * bf16_to_f32(w[i * ldw + k]);
            ema[i * lde + k] = a + b;
        }
    return quantize_impl(NULL, ema, R, C, lde, FMT_MX, RND_RTN, hadamard, 1, 0, 0, codes, scales, NULL);
}

/* ------------------------------------------------------------------ */
/* MXFP4 with a fixed grid scale [DIG step 1: for MXFP4 with Hadamard     */
/* rotations one fixed scale of the quantization grid serves every model; */
/* the page gives no value].  READING: every block's E8M0 exponent is the */
/* smallest e with 6 * 2^e >= RN(alpha * amax), clamped to [-127, 127],   */
/* alpha > 0 the fixed grid scale (one number for all blocks); alpha = 1  */
/* is the absmax rule of mxo_quantize, alpha < 1 lets the block maximum   */
/* saturate at +-6 for a finer grid.  Elements are then rounded to        */
/* nearest exactly as mxo_quantize rounds them (y * 2^-e, saturating).    */
/* Rotation (hadamard = 1) as in mxo_quantize.  PARITY UNPINNED as to the */
/* value of alpha (a caller's argument).                                   */
/* ------------------------------------------------------------------ */
int mxo_quantize_grid(const uint16_t *x, int64_t R, int64_t C, int64_t ldx, int hadamard, int axis,
                      float alpha, uint8_t *codes, uint8_t *scales)
{
    if (!x || !codes || !scales || R < 0 || C < 0 || ldx < C || (axis != 0 && axis != 1)) return -1;
    if (!(alpha > 0.0f) || !isfinite(alpha)) return -1;
    const int64_t rows = (axis == 1) ? R : C;
    const int64_t K = (axis == 1) ? C : R;
    if (K % 32 != 0) return -1;
    if (rows == 0 || K == 0) return 0;
    #pragma omp parallel
    {
        float *v = (float *)malloc(sizeof(float) * K);
        #pragma omp for
        for (int64_t i = 0; i < rows; i++) {
            load_contraction_row(x, ldx, axis, i, K, hadamard, v);
            for (int64_t b = 0; b < K / 32; b++) {
                const float *blk = v + b * 32;
                float amax;
                int byte;
                double step = 0.0;
                const int finite = block_amax(blk, 32, &amax);
                if (!finite) {
                    byte = 0xFF;
                } else {
                    float a = alpha * amax;                 /* one binary32 multiply */
                    int e = mxo_mx_scale_exponent(a);
                    byte = e + 127;
                    step = ldexp(1.0, -e);
                }
                scales[i * (K / 32) + b] = (uint8_t)byte;
                for (int j = 0; j < 32; j++)
                    put_code(codes, K, i, b * 32 + j, finite ? mxo_rtn_code((double)blk[j] * step) : 0);
            }
        }
        free(v);
    }
    return 0;
}
