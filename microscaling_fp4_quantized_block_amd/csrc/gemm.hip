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

// 16-byte chunk swizzle within a 64-byte row.  An MFMA operand read has lane l
// fetch 16 B of row l % 32; with 64-byte rows, rows r and r + 4 fall on the
// same banks, so the chunk index is XORed with bits 2..3 of the row.  (Measured
// on gfx950 with SQ_LDS_BANK_CONFLICT: this pattern is conflict-free, while
// XORing bits 0..1 or 1..2 leaves 2- to 4-way conflicts.)
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

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
#ifndef MXFP4_GROUP_M
#define MXFP4_GROUP_M 4
#endif
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int& tm, int& tn) {
  const int ntiles = p.ntm * p.ntn;
  int id = blockIdx.x;
#ifndef MXFP4_NO_XCD_REMAP
  if ((ntiles & 7) == 0) {
    const int per = ntiles >> 3;
    id = (id & 7) * per + (id >> 3);
  }
#endif
  constexpr int GROUP_M = MXFP4_GROUP_M;
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
// s_waitcnt with vmcnt <= VM and lgkmcnt <= LGKM (expcnt left alone).
template <int VM, int LGKM>
__device__ __forceinline__ void wait_cnt() {
  static_assert(VM < 64 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (LGKM << 8));
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Epilogue of a wave's TM x TN grid of 32x32 fp32 accumulators whose top-left
// output is (mb, nb).  In an accumulator, lane l holds column l % 32 and rows
// 8 (v / 4) + 4 (l / 32) + v % 4 (v = 0..15): four consecutive rows of one
// column per group of four registers.  A 4x4 transpose across each quad of
// lanes (two DPP exchange steps) turns that into one row and four consecutive
// columns per lane, written with one 16-byte store: a quarter of the store
// instructions, each covering whole 128-byte row segments.  Ragged edges and
// unaligned outputs use 4-byte stores.
__device__ __forceinline__ float dpp_xor1_f(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2_f(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(v), 0x4E, 0xF, 0xF, true));
}

template <int TM, int TN>
__device__ __forceinline__ void store_tile_f32x4(const GemmArgs& p, float* Cz, int64_t mb, int64_t nb,
                                                 const v16f (&acc)[TM][TN]) {
  const int l = threadIdx.x & 63, g = l >> 5, c = l & 3;
  const bool vec_ok = ((p.ldc & 3) == 0) && ((((uintptr_t)Cz) & 15) == 0);
#pragma unroll
  for (int tm = 0; tm < TM; tm++) {
#pragma unroll
    for (int tn = 0; tn < TN; tn++) {
      const int64_t ncol0 = nb + tn * 32 + (l & 31);          // this lane's column before the transpose
      const int64_t nq = nb + tn * 32 + (l & 28);             // first column of the lane's quad
#pragma unroll
      for (int a = 0; a < 4; a++) {
        float x[4], z[4], y[4];
#pragma unroll
        for (int b = 0; b < 4; b++) x[b] = acc[tm][tn][4 * a + b];
        // stage 1: keep x[k] where k and c agree in bit 0, else take the partner lane's x[k ^ 1]
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const float o = dpp_xor1_f(x[k ^ 1]);
          z[k] = ((k ^ c) & 1) ? o : x[k];
        }
        // stage 2: the same on bit 1 with the lane two apart
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const float o = dpp_xor2_f(z[k ^ 2]);
          y[k] = ((k ^ c) & 2) ? o : z[k];
        }
        // lane c of the quad now holds row 8a + 4g + c, columns nq .. nq+3
        const int64_t m = mb + tm * 32 + 8 * a + 4 * g + c;
        if (vec_ok && nq + 3 < p.N) {
          if (m < p.M) *(float4*)(Cz + m * p.ldc + nq) = make_float4(y[0], y[1], y[2], y[3]);
        } else {
          // ragged or unaligned: the untransposed values, one column per lane
#pragma unroll
          for (int b = 0; b < 4; b++) {
            const int64_t mm = mb + tm * 32 + 8 * a + 4 * g + b;
            if (mm < p.M && ncol0 < p.N) Cz[mm * p.ldc + ncol0] = x[b];
          }
        }
      }
    }
  }
}

// The MXFP4 kernel runs 8 waves per workgroup (2 per SIMD): one wave per SIMD
// cannot keep enough loads in flight (measured on gfx950: about 40 GB/s per
// CU from L2 with 4 waves, 65 GB/s with 8), and the second wave per SIMD hides
// LDS latency.  Wave w owns output rows 128 (w / 4) .. +128 and columns
// 64 (w % 4) .. +64: 4 x 2 MFMA tiles, 128 accumulators per lane.
//
// LDS: a ring of 4 code stages (A and B, 64 B per row each) and a ring of 3
// scale groups.  A scale group holds 16 scale bytes per row = 4 stages, so each
// row's scales arrive as one 16-byte load instead of four 4-byte loads (the
// scale rows are K/32 bytes apart, so every small load is a separate cache
// line).  Group G is loaded in four 64-row pieces alongside stages 4G-4..4G-1.
constexpr int MX_WAVES = 8;
constexpr int MX_TM = 4;
constexpr int MX_CODE_STAGE = A_BYTES + B_BYTES;               // 32 KB
constexpr int MX_SG_BYTES = BM * 16;                            // one operand's scale group: 4 KB
constexpr int MX_SCALE_OFF = NSTAGE * MX_CODE_STAGE;            // 128 KB
constexpr int MX_SGROUPS = 3;
constexpr int MX_SPARE_OFF = MX_SCALE_OFF + MX_SGROUPS * 2 * MX_SG_BYTES;   // 152 KB
constexpr int MX_LDS = MX_SPARE_OFF + 6 * 1024;                             // + 1 KB sink per wave 2..7

template <int NW>
struct MxOperand {
  static constexpr int CL = 256 / (16 * NW);   // 16-row code loads per wave per stage
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t code_off[CL];  // this lane's code offsets in stage 0
  uint32_t scale_row;     // byte offset of row (lane) in the scales, for 64-row piece 0
};

template <int NW>
__device__ __forceinline__ MxOperand<NW> mx_make_operand(const uint8_t* codes, const uint8_t* scales, int64_t rows_total,
                                                     int64_t row0, int64_t K) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t krow = K / 2, srow = K / 32;
  int64_t nrows = rows_total - row0;
  if (nrows > 256) nrows = 256;
  MxOperand<NW> o;
  constexpr int CL = MxOperand<NW>::CL;
  o.codes = __builtin_amdgcn_make_buffer_rsrc((void*)(codes + row0 * krow), (short)0, (int)(nrows * krow), kRsrcWord3);
  o.scales = __builtin_amdgcn_make_buffer_rsrc((void*)(scales + row0 * srow), (short)0, (int)(nrows * srow), kRsrcWord3);
#pragma unroll
  for (int j = 0; j < CL; j++) {
    const int row = 16 * CL * w + 16 * j + (l >> 2);
    o.code_off[j] = (uint32_t)(row * krow + (((l & 3) ^ swz(row)) * 16));
  }
  o.scale_row = (uint32_t)(l * srow);
  return o;
}

// This wave's 256/NW rows of one operand's codes for absolute stage kt.
template <int NW>
__device__ __forceinline__ void mx_issue_codes(const MxOperand<NW>& o, uint8_t* codes_lds, int kt) {
  constexpr int CL = MxOperand<NW>::CL;
  const int w = threadIdx.x >> 6;
  const uint32_t kb = (uint32_t)kt * ROWB;
#pragma unroll
  for (int j = 0; j < CL; j++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.codes, (lds_void*)(codes_lds + (16 * CL * w + 16 * j) * ROWB), 16,
                                             o.code_off[j] + kb, 0, 0, 0);
}
// Rows 64 piece .. +63 of a scale group starting at absolute stage kt_first:
// 16 bytes (4 stages) per row, from `rsrc` into `dst` (1 KB).
__device__ __forceinline__ void mx_issue_scale_piece_to(__amdgpu_buffer_rsrc_t rsrc, uint32_t scale_row, uint8_t* dst,
                                                        int piece, int kt_first, uint32_t srow) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16,
                                           scale_row + (uint32_t)(64 * piece) * srow + (uint32_t)kt_first * 4u,
                                           0, 0, 0);
}
template <int NW>
__device__ __forceinline__ void mx_issue_scale_piece(const MxOperand<NW>& o, uint8_t* group_lds, int piece, int kt_first,
                                                     uint32_t srow) {
  mx_issue_scale_piece_to(o.scales, o.scale_row, group_lds + piece * 64 * 16, piece, kt_first, srow);
}

template <int MX_TN>
struct MxFrag {
  v4i a[MX_TM], b[MX_TN];
};

// One wave's operand fragments of sub-step s (blocks 2g + s) of a stage.
template <int MX_TN>
__device__ __forceinline__ void mx_load_frag(const uint8_t* st, int ra0, int rb0, int offc, MxFrag<MX_TN>& f) {
  const uint8_t* A = st;
  const uint8_t* B = st + A_BYTES;
#pragma unroll
  for (int t = 0; t < MX_TM; t++) f.a[t] = *(const v4i*)(A + (ra0 + 32 * t) * ROWB + offc);
#pragma unroll
  for (int t = 0; t < MX_TN; t++) f.b[t] = *(const v4i*)(B + (rb0 + 32 * t) * ROWB + offc);
}

// Scale bytes of blocks 2g, 2g+1 of stage j (0..3) of a group, for each of the lane's rows.
template <int MX_TN>
__device__ __forceinline__ void mx_load_scales(const uint8_t* grp, int ra0, int rb0, int j, int g, int (&sa)[MX_TM],
                                               int (&sb)[MX_TN]) {
  const uint8_t* SA = grp;
  const uint8_t* SB = grp + MX_SG_BYTES;
#pragma unroll
  for (int t = 0; t < MX_TM; t++) sa[t] = *(const uint16_t*)(SA + (ra0 + 32 * t) * 16 + 4 * j + 2 * g);
#pragma unroll
  for (int t = 0; t < MX_TN; t++) sb[t] = *(const uint16_t*)(SB + (rb0 + 32 * t) * 16 + 4 * j + 2 * g);
}

template <int S, int MX_TN>
__device__ __forceinline__ void mx_mfma(v16f (&acc)[MX_TM][MX_TN], const MxFrag<MX_TN>& f, const int (&sa)[MX_TM],
                                        const int (&sb)[MX_TN]) {
#pragma unroll
  for (int i = 0; i < MX_TM; i++) {
    const v8i a = __builtin_shufflevector(f.a[i], f.a[i], 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
    for (int j = 0; j < MX_TN; j++) {
      const v8i b = __builtin_shufflevector(f.b[j], f.b[j], 0, 1, 2, 3, -1, -1, -1, -1);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 4, 4, S, sa[i], S, sb[j]);
    }
  }
}

// Main loop, software-pipelined so that LDS reads always run under MFMAs:
//   stage i:  read sub-step 1 fragments | MFMAs of sub-step 0
//             wait for stage i+1, barrier, refill stage i's buffer with i+4
//             read stage i+1 sub-step 0 | MFMAs of sub-step 1
// Stage i's buffer is refilled right after the barrier that follows the last
// read of it, so four buffers keep three stages of loads in flight.  The loop
// body has no branches (stages past the end are loaded into buffers that are
// never read again, and reads past the end are never consumed): a branch would
// let the compiler sink the first MFMA group below the barrier.
template <int NW>
__global__ void __launch_bounds__(64 * NW, 1) gemm_mx_kernel(GemmArgs p) {
  constexpr int MX_TN = 16 / NW;            // 4 waves: 128 x 128 per wave; 8 waves: 128 x 64
  constexpr int WN = NW / 2;                 // waves along N
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX_LDS];
  int tm_, tn_;
  tile_coords(p, tm_, tn_);
  const int64_t m0 = (int64_t)tm_ * BM, n0 = (int64_t)tn_ * BN;
  const int z = blockIdx.y;
  const int kt0 = (int)((int64_t)p.k_tiles * z / p.splits), kt1 = (int)((int64_t)p.k_tiles * (z + 1) / p.splits);
  const int nk = kt1 - kt0;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar branches
  const int l = threadIdx.x & 63, g = l >> 5;
  const int wm = w / WN, wn = w % WN;
  const int ra0 = wm * 128 + (l & 31), rb0 = wn * (32 * MX_TN) + (l & 31);
  const int zs = swz(ra0);            // equal for every t (t * 32 leaves bits 2..3 alone), and for rb0
  const int offc0 = ((2 * g + 0) ^ zs) << 4, offc1 = ((2 * g + 1) ^ zs) << 4;

  v16f acc[MX_TM][MX_TN];
#pragma unroll
  for (int i = 0; i < MX_TM; i++)
#pragma unroll
    for (int j = 0; j < MX_TN; j++) acc[i][j] = (v16f){};

  if (nk > 0) {
    // buffer->LDS instructions per wave per stage: the code loads plus one
    // scale load.  Waves 0 and 1 load the scale pieces; the other waves issue
    // the same instruction on an empty buffer (out of range: no memory
    // traffic, zeros into a private LDS sink), so every wave has the same
    // count and "at most 2 * LOADS outstanding" is exact.
    constexpr int LOADS = 2 * MxOperand<NW>::CL + 1;
    const uint32_t srow = (uint32_t)(p.K / 32);
    const MxOperand<NW> oa = mx_make_operand<NW>(p.a, p.as, p.M, m0, p.K);
    const MxOperand<NW> ob = mx_make_operand<NW>(p.b, p.bs, p.N, n0, p.K);
    const __amdgpu_buffer_rsrc_t srsrc =
        w == 0 ? oa.scales : w == 1 ? ob.scales : __builtin_amdgcn_make_buffer_rsrc((void*)p.as, (short)0, 0, kRsrcWord3);
    // scale destinations as arithmetic on wave-uniform values (no branches in the loop)
    const int sc_real = w < 2 ? 1 : 0;
    uint8_t* const sc_base = sc_real ? smem + MX_SCALE_OFF + w * MX_SG_BYTES : smem + MX_SPARE_OFF + (w - 2) * 1024;
    auto stage = [&](int i) { return smem + (i & (NSTAGE - 1)) * MX_CODE_STAGE; };
    auto group = [&](int h) { return smem + MX_SCALE_OFF + (h % MX_SGROUPS) * 2 * MX_SG_BYTES; };
    // stage i's codes, and scale piece i % 4 of group i / 4 + 1.  Stages and
    // groups at or past the end load whatever lies there (in bounds of the
    // operand buffers, or zero past them) into buffers that are never read.
    auto issue = [&](int i) {
      uint8_t* st = stage(i);
      mx_issue_codes(oa, st, kt0 + i);
      mx_issue_codes(ob, st + A_BYTES, kt0 + i);
      const int h = (i >> 2) + 1;
      uint8_t* sdst = sc_base + sc_real * ((h % MX_SGROUPS) * 2 * MX_SG_BYTES + (i & 3) * 1024);
      mx_issue_scale_piece_to(srsrc, oa.scale_row, sdst, i & 3, kt0 + 4 * h, srow);
    };
    // prologue: scale group 0 (8 pieces spread over the waves), then stages 0..2
#pragma unroll
    for (int q = 0; q < 8 / NW; q++) {
      const int piece = w * (8 / NW) + q;
      if (piece < 4) mx_issue_scale_piece(oa, group(0), piece, kt0, srow);
      else mx_issue_scale_piece(ob, group(0) + MX_SG_BYTES, piece - 4, kt0, srow);
    }
    issue(0);
    issue(1);
    issue(2);
    wait_cnt<2 * LOADS, 15>();
    block_barrier();
    issue(3);

    MxFrag<MX_TN> f0, f1;
    int sa[MX_TM], sb[MX_TN], sa_n[MX_TM], sb_n[MX_TN];
    mx_load_scales(group(0), ra0, rb0, 0, g, sa, sb);
    mx_load_frag(stage(0), ra0, rb0, offc0, f0);
    for (int i = 0; i < nk; i++) {
      // phase A: sub-step 1 fragment reads under the sub-step 0 MFMAs
      mx_load_frag(stage(i), ra0, rb0, offc1, f1);
      mx_mfma<0>(acc, f0, sa, sb);
#pragma unroll
      for (int q = 0; q < MX_TM + MX_TN; q++) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one DS read
        __builtin_amdgcn_sched_group_barrier(0x008, MX_TN / 2 + 1, 0);   // MFMAs
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      __builtin_amdgcn_sched_barrier(0);
      // stage i+1 has landed for this wave, and its own reads of stage i are done
      wait_cnt<2 * LOADS, 0>();
      block_barrier();
      // phase B: the loads of stage i+4, and the scales and sub-step 0
      // fragments of stage i+1, spread under the sub-step 1 MFMAs.  A load
      // instruction can stall its wave while the memory pipeline is full, so
      // each one is separated by MFMAs already queued.
      issue(i + 4);
      mx_load_scales(group((i + 1) >> 2), ra0, rb0, (i + 1) & 3, g, sa_n, sb_n);
      mx_load_frag(stage(i + 1), ra0, rb0, offc0, f0);
      mx_mfma<1>(acc, f1, sa, sb);
#pragma unroll
      for (int q = 0; q < LOADS; q++) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one buffer->LDS load
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < MX_TM; t++) sa[t] = sa_n[t];
#pragma unroll
      for (int t = 0; t < MX_TN; t++) sb[t] = sb_n[t];
    }
    wait_cnt<0, 0>();   // nothing may still write LDS when the workgroup exits
  }
  // epilogue
  float* Cz = p.C + (int64_t)z * p.split_stride;
  store_tile_f32x4<MX_TM, MX_TN>(p, Cz, m0 + wm * 128, n0 + wn * (32 * MX_TN), acc);
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
  const int zs = swz(ra0);            // equal for every t (t * 32 leaves bits 2..3 alone)
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
  else hipLaunchKernelGGL(gemm_mx_kernel<MX_WAVES>, grid, dim3(64 * MX_WAVES), 0, stream, p);
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
