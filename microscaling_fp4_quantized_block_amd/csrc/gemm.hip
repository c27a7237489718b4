// gemm.hip -- block-scaled FP4 GEMM, C[M,N] = A[M,K] * B[N,K]^T, for gfx950.
//
// The FP4 GEMM consumes the packed operands of the quantizer ("Bridging the
// Gap Between Promise and Performance for Microscaling FP4 Quantization",
// abstract: FP4 GEMM kernels with rotation fused into the weights; "FP4 All the
// Way: Fully Quantized Training of LLMs", abstract: forward, backward and update
// GEMMs all in FP4).  Every orientation (XW^T, dY.W, dY^T.X) is this one
// contraction-major layout; transposition happens in the quantizer.
//
// MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands.  In that
//   instruction lane l holds row (l % 32) and 32 consecutive contraction
//   elements -- one whole MX block -- plus that block's E8M0 scale in a byte of
//   a 32-bit register (op_sel picks the byte).  The contraction order inside a
//   tile is free as long as A and B agree, so lane group g = l / 32 at sub-step
//   s consumes block 2g + s of the 128-wide stage: a lane's two blocks are
//   32 contiguous bytes and its two scale bytes one aligned 16-bit word.
// NVFP4: the product of an E2M1 code and an E4M3 scale needs up to 6
//   significant bits, which no FP4/FP6/FP8 operand of the scaled MFMA holds,
//   so codes are dequantized exactly to fp16 in registers (hardware FP4->fp16
//   convert, then a packed fp16 multiply by the block scale) and fed to
//   v_mfma_f32_32x32x16_f16.  Each lane dequantizes with its own row's block
//   scale, so the two lane groups of one MFMA step may take different blocks.
//   The two tensor scales multiply the FP32 result in the epilogue.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2, 128 x 128 per
// wave = 4 x 4 MFMA tiles, 256 accumulators per lane), K step 128 per stage,
// four LDS stages (36 KB each) filled by buffer->LDS loads issued three stages
// ahead (no staging registers, no LDS write instructions).  Codes sit in LDS as
// 16-byte chunks, XOR-swizzled per row so that the rows an MFMA operand read
// touches together hit distinct banks.
// Workgroup ids are remapped so that tiles running at the same time on one XCD
// (which owns one L2) share A and B panels.  Long contractions with few
// output tiles are split along K; the partial sums land in the workspace and a
// second kernel adds them in a fixed order.
#include "fp4_device.h"
#include "mxfp4_internal.h"

namespace mxfp4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256, BK = 128;   // BK: contraction elements per stage
constexpr int NSTAGE = 4;
constexpr int ROWB = BK / 2;                   // 64 code bytes per row per stage
constexpr int A_BYTES = BM * ROWB;             // 16 KB
constexpr int B_BYTES = BN * ROWB;             // 16 KB
constexpr int SROW = 8;                        // scale bytes per row per stage (MXFP4 uses 4, NVFP4 8)
constexpr int SA_BYTES = BM * SROW;
constexpr int SB_BYTES = BN * SROW;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;   // 36 KB
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

// 16-byte chunk swizzle within a 64-byte row: rows that one MFMA operand read
// touches together (8 or 16 consecutive rows) land on distinct LDS banks.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* as;
  const uint8_t* b;
  const uint8_t* bs;
  const float* a_ts;
  const float* b_ts;
  int64_t M, N, K;
  float* C;
  int64_t ldc;
  int64_t split_stride;     // floats between split slices of the workspace
  int k_tiles;              // stages over the whole contraction
  int splits;
  int ntm, ntn;
};

// Tile order: consecutive workgroup ids go to consecutive XCDs, so gather
// the ids one XCD receives into a contiguous range, then walk that range in
// groups of GROUP_M tile rows.
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int& tm, int& tn) {
  const int ntiles = p.ntm * p.ntn;
  int id = blockIdx.x;
  if ((ntiles & 7) == 0) {
    const int per = ntiles >> 3;
    id = (id & 7) * per + (id >> 3);
  }
  constexpr int GROUP_M = 4;
  const int group = id / (GROUP_M * p.ntn);
  const int first_m = group * GROUP_M;
  const int gm = min(p.ntm - first_m, GROUP_M);
  const int in_group = id - group * GROUP_M * p.ntn;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// Operand rows are reached through buffer resources whose size ends at the
// last row, so rows past M (or N) read as zero.
struct Operand {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t code_off[4];  // this lane's code offset in stage 0, per load j (row and swizzled chunk)
  uint32_t scale_off;    // this lane's scale offset in stage 0
};

// Per stage, wave w moves rows [64w, 64w + 64) of the tile: four 1 KB code
// loads (16 rows x 64 B each, lane l -> row l/4, LDS slot l holding global
// chunk (l & 3) ^ swz(row)) and the rows' scale bytes (SB_PER_ROW bytes per
// row, 4 bytes per lane).
template <int SB_PER_ROW>
__device__ __forceinline__ Operand make_operand(const uint8_t* codes, const uint8_t* scales, int64_t rows_total,
                                                int64_t row0, int64_t K) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t krow = K / 2;
  constexpr int BS = (SB_PER_ROW == 4) ? 32 : 16;
  const int64_t srow = K / BS;
  Operand o;
  int64_t nrows = rows_total - row0;                 // rows of this tile that exist
  if (nrows > 256) nrows = 256;
  const uint8_t* cbase = codes + row0 * krow;
  const uint8_t* sbase = scales + row0 * srow;
  o.codes = __builtin_amdgcn_make_buffer_rsrc((void*)cbase, (short)0, (int)(nrows * krow), kRsrcWord3);
  o.scales = __builtin_amdgcn_make_buffer_rsrc((void*)sbase, (short)0, (int)(nrows * srow), kRsrcWord3);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int row = 64 * w + 16 * j + (l >> 2);
    const int chunk = (l & 3) ^ swz(row);
    o.code_off[j] = (uint32_t)(row * krow + chunk * 16);
  }
  if (SB_PER_ROW == 4) {
    o.scale_off = (uint32_t)((64 * w + l) * srow);
  } else {
    o.scale_off = (uint32_t)((64 * w + (l >> 1)) * srow + 4 * (l & 1));
  }
  return o;
}

template <int SB_PER_ROW>
__device__ __forceinline__ void issue_operand(const Operand& o, uint8_t* codes_lds, uint8_t* scales_lds, int kt,
                                              int64_t K) {
  const int w = threadIdx.x >> 6;
  const uint32_t kb = (uint32_t)kt * ROWB;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    // rows 64w + 16j .. + 15; LDS destination is wave-uniform
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.codes, (lds_void*)(codes_lds + (64 * w + 16 * j) * ROWB), 16,
                                             o.code_off[j] + kb, 0, 0, 0);
  }
  if (SB_PER_ROW == 4) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.scales, (lds_void*)(scales_lds + 64 * w * 4), 4,
                                             o.scale_off + (uint32_t)kt * 4u, 0, 0, 0);
  } else {
    const uint32_t srow = (uint32_t)(K / 16);
#pragma unroll
    for (int j = 0; j < 2; j++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(o.scales, (lds_void*)(scales_lds + (64 * w + 32 * j) * 8), 4,
                                               o.scale_off + 32u * j * srow + (uint32_t)kt * 8u, 0, 0, 0);
  }
}

// vmcnt wait with the other counters left alone (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Epilogue: lane l of a 32x32 accumulator holds column l % 32 and rows
// 8 (v / 4) + 4 (l / 32) + v % 4 for v = 0..15.
__device__ __forceinline__ void store_acc(const GemmArgs& p, float* Cz, int64_t ldc, int64_t m0, int64_t n0, int wm,
                                          int wn, v16f (&acc)[4][4], float mul) {
  const int l = threadIdx.x & 63;
  const int g = l >> 5;
#pragma unroll
  for (int tm = 0; tm < 4; tm++) {
#pragma unroll
    for (int tn = 0; tn < 4; tn++) {
      const int64_t n = n0 + wn * 128 + tn * 32 + (l & 31);
      if (n >= p.N) continue;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int64_t m = m0 + wm * 128 + tm * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        if (m < p.M) Cz[m * ldc + n] = acc[tm][tn][v] * mul;
      }
    }
  }
}

// Shared prologue/epilogue and the staged main loop; COMPUTE consumes one
// stage from LDS.  Per stage each wave issues LOADS buffer->LDS instructions,
// so "stage kt has landed" is vmcnt <= LOADS * (stages issued after it).
template <int SB_PER_ROW, int LOADS, typename Compute>
__device__ __forceinline__ void gemm_mainloop(const GemmArgs& p, uint8_t* smem, int64_t m0, int64_t n0, int kt0,
                                              int kt1, Compute&& compute) {
  const Operand oa = make_operand<SB_PER_ROW>(p.a, p.as, p.M, m0, p.K);
  const Operand ob = make_operand<SB_PER_ROW>(p.b, p.bs, p.N, n0, p.K);
  auto issue = [&](int kt) {
    uint8_t* st = smem + ((kt - kt0) % NSTAGE) * STAGE_BYTES;
    issue_operand<SB_PER_ROW>(oa, st, st + A_BYTES + B_BYTES, kt, p.K);
    issue_operand<SB_PER_ROW>(ob, st + A_BYTES, st + A_BYTES + B_BYTES + SA_BYTES, kt, p.K);
  };
  const int nk = kt1 - kt0;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; s++)
    if (s < nk) issue(kt0 + s);
  for (int i = 0; i < nk; i++) {
    if (i + 2 < nk) wait_vmcnt<2 * LOADS>();
    else if (i + 1 < nk) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
    // stage i is in LDS for every wave, and stage i-1 is no longer read.  A
    // bare s_barrier: __syncthreads() would also wait for every load still in
    // flight (vmcnt(0)), which would drain the prefetch pipeline.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i + NSTAGE - 1 < nk) issue(kt0 + i + NSTAGE - 1);
    compute(smem + (i % NSTAGE) * STAGE_BYTES);
  }
}

// ---------------------------------------------------------------------------
// MXFP4
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256, 1) gemm_mx_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTAGE * STAGE_BYTES];
  int tm_, tn_;
  tile_coords(p, tm_, tn_);
  const int64_t m0 = (int64_t)tm_ * BM, n0 = (int64_t)tn_ * BN;
  const int z = blockIdx.y;
  const int kt0 = (int)((int64_t)p.k_tiles * z / p.splits), kt1 = (int)((int64_t)p.k_tiles * (z + 1) / p.splits);

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 5;
  const int wm = w >> 1, wn = w & 1;
  // LDS byte offsets of this lane's operand rows (tile t adds t * 32 rows)
  const int ra0 = wm * 128 + (l & 31), rb0 = wn * 128 + (l & 31);
  const int zs = swz(ra0);            // equal for every t (t * 32 leaves bits 1..4 alone)
  const int offc0 = ((2 * g + 0) ^ zs) << 4, offc1 = ((2 * g + 1) ^ zs) << 4;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = (v16f){};

  gemm_mainloop<4, 10>(p, smem, m0, n0, kt0, kt1, [&](const uint8_t* st) {
    const uint8_t* A = st;
    const uint8_t* B = st + A_BYTES;
    const uint8_t* SA = st + A_BYTES + B_BYTES;
    const uint8_t* SB = SA + SA_BYTES;
    int sa[4], sb[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
      sa[t] = *(const uint16_t*)(SA + (ra0 + 32 * t) * 4 + 2 * g);
      sb[t] = *(const uint16_t*)(SB + (rb0 + 32 * t) * 4 + 2 * g);
    }
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const int offc = s ? offc1 : offc0;
      v8i af[4], bf[4];
#pragma unroll
      for (int t = 0; t < 4; t++) {
        v4i x = *(const v4i*)(A + (ra0 + 32 * t) * ROWB + offc);
        v4i y = *(const v4i*)(B + (rb0 + 32 * t) * ROWB + offc);
        af[t] = __builtin_shufflevector(x, x, 0, 1, 2, 3, -1, -1, -1, -1);
        bf[t] = __builtin_shufflevector(y, y, 0, 1, 2, 3, -1, -1, -1, -1);
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          if (s == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 1, sa[i], 1, sb[j]);
        }
    }
  });
  float* Cz = p.C + (int64_t)z * p.split_stride;
  store_acc(p, Cz, p.ldc, m0, n0, wm, wn, acc, 1.0f);
}

// ---------------------------------------------------------------------------
// NVFP4
// ---------------------------------------------------------------------------
// 8 codes (4 bytes) of one block, exactly dequantized to fp16: hardware
// E2M1 -> fp16 convert, then multiply by the block's E4M3 scale (as fp16;
// the product has at most 6 significant bits and lies in [2^-10, 2688]).
__device__ __forceinline__ v8h nv_dequant8(uint32_t codes4, v2h s2) {
  v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes4, 1.0f, 0);
  v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes4, 1.0f, 1);
  v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes4, 1.0f, 2);
  v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes4, 1.0f, 3);
  h0 = h0 * s2; h1 = h1 * s2; h2 = h2 * s2; h3 = h3 * s2;
  return (v8h){h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

__device__ __forceinline__ v2h e4m3_as_h2(uint32_t byte) {
  const _Float16 s = (_Float16)e4m3_value(byte);
  return (v2h){s, s};
}

// A stage holds 8 NVFP4 blocks per row.  Lane group g owns blocks 4g..4g+3
// (32 contiguous bytes); at step u it feeds half (u & 1) of block 4g + u/2 to
// the 32x32x16 fp16 MFMA.  A and B use the same assignment, so every step
// pairs equal contraction indices.
__global__ void __launch_bounds__(256, 1) gemm_nv_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTAGE * STAGE_BYTES];
  int tm_, tn_;
  tile_coords(p, tm_, tn_);
  const int64_t m0 = (int64_t)tm_ * BM, n0 = (int64_t)tn_ * BN;
  const int z = blockIdx.y;
  const int kt0 = (int)((int64_t)p.k_tiles * z / p.splits), kt1 = (int)((int64_t)p.k_tiles * (z + 1) / p.splits);

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 5;
  const int wm = w >> 1, wn = w & 1;
  const int ra0 = wm * 128 + (l & 31), rb0 = wn * 128 + (l & 31);
  const int zs = swz(ra0);
  const int offc0 = ((2 * g + 0) ^ zs) << 4, offc1 = ((2 * g + 1) ^ zs) << 4;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = (v16f){};

  gemm_mainloop<8, 12>(p, smem, m0, n0, kt0, kt1, [&](const uint8_t* st) {
    const uint8_t* A = st;
    const uint8_t* B = st + A_BYTES;
    const uint8_t* SA = st + A_BYTES + B_BYTES;
    const uint8_t* SB = SA + SA_BYTES;
    uint32_t sa[4], sb[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
      sa[t] = *(const uint32_t*)(SA + (ra0 + 32 * t) * 8 + 4 * g);
      sb[t] = *(const uint32_t*)(SB + (rb0 + 32 * t) * 8 + 4 * g);
    }
#pragma unroll
    for (int half = 0; half < 2; half++) {        // 16-byte chunk: blocks 4g + 2 half, +1
      const int offc = half ? offc1 : offc0;
      v4i ca[4], cb[4];
#pragma unroll
      for (int t = 0; t < 4; t++) {
        ca[t] = *(const v4i*)(A + (ra0 + 32 * t) * ROWB + offc);
        cb[t] = *(const v4i*)(B + (rb0 + 32 * t) * ROWB + offc);
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {                // word u of the chunk = half (u & 1) of block 2 half + u/2
        const int blk = 2 * half + (u >> 1);
        v8h af[4], bf[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
          af[t] = nv_dequant8((uint32_t)ca[t][u], e4m3_as_h2((sa[t] >> (8 * blk)) & 0xFFu));
          bf[t] = nv_dequant8((uint32_t)cb[t][u], e4m3_as_h2((sb[t] >> (8 * blk)) & 0xFFu));
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 4; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
  });
  float* Cz = p.C + (int64_t)z * p.split_stride;
  // both tensor scales multiply the sum (for split partials too: the factor
  // distributes over the split sum)
  const float mul = p.a_ts[0] * p.b_ts[0];
  store_acc(p, Cz, p.ldc, m0, n0, wm, wn, acc, mul);
}

// ---------------------------------------------------------------------------
// Split-K reduction: C = sum over splits, in split order.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ ws, int splits, int64_t M,
                                                            int64_t N, float* __restrict__ C, int64_t ldc) {
  const int64_t total = M * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    float s = ws[t];
    for (int z = 1; z < splits; z++) s += ws[(int64_t)z * total + t];
    const int64_t m = t / N, n = t - m * N;
    C[m * ldc + n] = s;
  }
}

// ---------------------------------------------------------------------------
// Planning and launch
// ---------------------------------------------------------------------------
GemmPlan plan_gemm(int fmt, int64_t M, int64_t N, int64_t K) {
  (void)fmt;
  GemmPlan pl;
  pl.k_tiles = (K + BK - 1) / BK;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  int splits = 1;
  // fewer output tiles than compute units: split the contraction so that
  // about one wave of workgroups fills the chip, keeping >= 4 stages per split
  const int64_t cus = 256;
  if (tiles < cus && pl.k_tiles >= 8) {
    int64_t s = cus / tiles;
    if (s > pl.k_tiles / 4) s = pl.k_tiles / 4;
    if (s > 32) s = 32;
    if (s > 1) splits = (int)s;
  }
  pl.splits = splits;
  return pl;
}

static hipError_t launch_gemm_common(bool nv, GemmArgs p, float* C, int64_t ldc, float* workspace,
                                     const GemmPlan& plan, hipStream_t stream) {
  p.ntm = (int)((p.M + BM - 1) / BM);
  p.ntn = (int)((p.N + BN - 1) / BN);
  p.k_tiles = (int)plan.k_tiles;
  p.splits = plan.splits;
  if (plan.splits > 1) {
    p.C = workspace;
    p.ldc = p.N;
    p.split_stride = p.M * p.N;
  } else {
    p.C = C;
    p.ldc = ldc;
    p.split_stride = 0;
  }
  dim3 grid((unsigned)(p.ntm * p.ntn), (unsigned)plan.splits);
  if (nv) hipLaunchKernelGGL(gemm_nv_kernel, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(gemm_mx_kernel, grid, dim3(256), 0, stream, p);
  if (plan.splits > 1) {
    int64_t work = p.M * p.N;
    int64_t g = (work + 255) / 256;
    if (g > 4096) g = 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)g), dim3(256), 0, stream, workspace, plan.splits,
                       p.M, p.N, C, ldc);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* C, int64_t ldc,
                          float* workspace, const GemmPlan& plan, hipStream_t stream) {
  GemmArgs p{};
  p.a = a_codes; p.as = a_scales; p.b = b_codes; p.bs = b_scales;
  p.a_ts = nullptr; p.b_ts = nullptr;
  p.M = M; p.N = N; p.K = K;
  return launch_gemm_common(false, p, C, ldc, workspace, plan, stream);
}

hipError_t launch_gemm_nv(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                          const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts, int64_t M,
                          int64_t N, int64_t K, float* C, int64_t ldc, float* workspace, const GemmPlan& plan,
                          hipStream_t stream) {
  GemmArgs p{};
  p.a = a_codes; p.as = a_scales; p.b = b_codes; p.bs = b_scales;
  p.a_ts = a_ts; p.b_ts = b_ts;
  p.M = M; p.N = N; p.K = K;
  return launch_gemm_common(true, p, C, ldc, workspace, plan, stream);
}

}  // namespace mxfp4
