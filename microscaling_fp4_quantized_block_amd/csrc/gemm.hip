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
// Tiling (MXFP4): 256 x 256 output tile per workgroup of 4 waves (2 x 2,
// 128 x 128 per wave = 4 x 4 MFMA tiles, 256 accumulators per lane in AGPRs),
// K stage 256 (one 128-byte line per operand row), two LDS stages of 64 KB
// filled by buffer->LDS loads, three scale-group buffers; details at the
// kernel.  NVFP4 keeps a 128-wide K stage with four 36 KB stages.  Codes sit
// in LDS as 16-byte chunks, XOR-swizzled per row so that the rows an MFMA
// operand read touches together hit distinct banks.
// Workgroup ids are remapped so that tiles running at the same time on one XCD
// (which owns one L2) share A and B panels.  Long contractions with few
// output tiles are split along K; the partial sums land in the workspace and a
// second kernel adds them in a fixed order.  Up to 128 activation rows take
// the decode kernel instead (16-column workgroups over the whole contraction,
// 16x16x128 scaled MFMA), and where its workgroups would hold too many
// operand bytes, the narrow kernel (32-row tiles, split along K).
#include <type_traits>

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
  int rem;                  // MXFP4: remainder tiles run as two 256 x 128 halves (see the kernel)
  // fused activation quantization (MXFP4 narrow tiles): A comes in as bf16
  const uint16_t* x;
  int64_t ldx;
  int x_vec;                // x 16-byte aligned and ldx a multiple of 8: 16-byte loads
  // quantized output (OUT_MXQ): C rounded to bf16, then MXFP4 round-to-nearest
  // along its rows (block Hadamard first when qhad): codes [M, N/2], scales [M, N/32]
  uint8_t* qcodes;
  uint8_t* qscales;
  int qhad;
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
// 8 (v / 4) + 4 (l / 32) + v % 4 (v = 0..15), so one register across the wave
// is two rows of 32 consecutive columns: a 4-byte store per register writes
// two whole 128-byte row segments, straight from the accumulator.  (A 4x4
// transpose across lane quads into 16-byte stores, a quarter of the store
// instructions, measured 4-12 % slower: its DPP exchanges need every value in
// a VGPR.)  Whole blocks inside C store without checks; ragged edges check
// each element.
//
// Every value is multiplied by mul (the NVFP4 tensor scales) when SCALED.
// OUT selects what is written:
//   OUT_F32   fp32 C with non-temporal stores: C is not read again here, and
//             on store-bound shapes (short contractions) streaming stores run
//             ~10-18 % faster (measured);
//   OUT_PART  fp32 split-K partials with plain stores: the reduction re-reads
//             them right after (~7 % faster on a 3072 x 768 x 50432 wgrad,
//             ~12 % on a 16 x 4096 x 14336 decode);
//   OUT_BF16  C rounded to bf16 (round to nearest even, hardware convert).
// The choice is a kernel template parameter: two epilogues in one kernel cost
// the wide kernel ~35 %.
//   OUT_MXQ   C rounded to bf16 and quantized to MXFP4 for the next layer
//             (quantize_tile below); nothing else is written.
constexpr int OUT_F32 = 0, OUT_PART = 1, OUT_BF16 = 2, OUT_MXQ = 3;

//
// bf16 whole blocks: the two column blocks tn, tn + 1 of a row are paired so
// that each lane stores 4 bytes and a wave store covers 128 contiguous bytes
// per row: lanes l and l ^ 1 swap one value (one DPP move), then an even lane
// holds columns l, l + 1 of block tn and an odd lane columns l - 1, l of block
// tn + 1.  (2-byte stores of half lines ran ~9 % slower than FP32 C on a
// store-bound 50432 x 3072 x 768.)
__device__ __forceinline__ float dpp_swap_pairs(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(v), 0xB1, 0xF, 0xF, true));
}

template <int TM, int TN, bool SCALED, int OUT>
__device__ __forceinline__ void store_tile(const GemmArgs& p, float* Cz, int64_t mb, int64_t nb,
                                           const v16f (&acc)[TM][TN], float mul = 1.0f) {
  typedef typename std::conditional<OUT == OUT_BF16, __bf16, float>::type T;
  const int l = threadIdx.x & 63, g = l >> 5;
  const int64_t ldc = p.ldc;
  const bool full = mb + 32 * TM <= p.M && nb + 32 * TN <= p.N;
  if constexpr (OUT == OUT_BF16 && TN % 2 == 0) {
    if (full && (ldc & 1) == 0 && (((uintptr_t)Cz) & 3) == 0) {
      const bool odd = l & 1;
      // this lane's 4-byte pair: block tn (even lanes) or tn + 1 (odd lanes),
      // first column (l & 30)
      __bf16* const pair0 = (__bf16*)Cz + (mb + 4 * g) * ldc + nb + (l & 30) + (odd ? 32 : 0);
#pragma unroll
      for (int tm = 0; tm < TM; tm++) {
#pragma unroll
        for (int a = 0; a < 4; a++) {
#pragma unroll
          for (int b = 0; b < 4; b++) {
            const int r = tm * 32 + 8 * a + b;
            __bf16* const rp = pair0 + (int64_t)r * ldc;
#pragma unroll
            for (int tn = 0; tn < TN; tn += 2) {
              float x = acc[tm][tn][4 * a + b], y = acc[tm][tn + 1][4 * a + b];
              if (SCALED) { x *= mul; y *= mul; }
              const float got = dpp_swap_pairs(odd ? x : y);
              const float lo = odd ? got : x, hi = odd ? y : got;
              typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
              *(bf16x2_t*)(rp + tn * 32) = (bf16x2_t){(__bf16)lo, (__bf16)hi};
            }
          }
        }
      }
      return;
    }
  }
  // this lane's column and its first row (4g) in the block
  T* const lane0 = (T*)Cz + (mb + 4 * g) * ldc + nb + (l & 31);
#pragma unroll
  for (int tm = 0; tm < TM; tm++) {
#pragma unroll
    for (int a = 0; a < 4; a++) {
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const int r = tm * 32 + 8 * a + b;                      // row in the block, less 4g
        T* const rp = lane0 + (int64_t)r * ldc;
#pragma unroll
        for (int tn = 0; tn < TN; tn++) {
          const float v = SCALED ? acc[tm][tn][4 * a + b] * mul : acc[tm][tn][4 * a + b];
          if (full || (mb + r + 4 * g < p.M && nb + tn * 32 + (l & 31) < p.N)) {
            if (OUT == OUT_PART) rp[tn * 32] = v;
            else if (OUT == OUT_BF16) rp[tn * 32] = (T)v;
            else __builtin_nontemporal_store(v, (float*)rp + tn * 32);
          }
        }
      }
    }
  }
}

// FP32 epilogue through LDS (wide tiles): the wave's accumulators go to its
// own LDS slice one 32-row block row at a time (4-byte writes, a register
// across the wave = two rows of 32 columns), and come back as whole rows so
// that each store writes 16 bytes per lane: 64 store instructions per wave
// instead of 256, so far fewer stores are in flight per wave for the same
// bytes (headline shape: 414 K cycles against 428 K with 4-byte stores
// straight from the accumulators, same results).  Rows are padded to
// 128 TN + 32 bytes (the two halves of a register write land on different
// bank halves; 16 consecutive lanes read 256 contiguous bytes).  The caller
// has made every wave finish its main loop.
template <int TM, int TN, int OUT>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& p, uint8_t* smem, float* Cz, int64_t mb, int64_t nb,
                                               const v16f (&acc)[TM][TN]) {
  constexpr int RB = 128 * TN + 32;                // bytes per LDS row
  constexpr int CPR = 8 * TN;                      // 16-byte chunks per row
  const int l = threadIdx.x & 63, g = l >> 5, w = threadIdx.x >> 6;
  uint8_t* slab = smem + w * 32 * RB;
  const int64_t ldc = p.ldc;
  const bool full_cols = nb + 32 * TN <= p.N && (ldc & 3) == 0 && (((uintptr_t)Cz) & 15) == 0;
#pragma unroll
  for (int tm = 0; tm < TM; tm++) {
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int r = 8 * (v >> 2) + 4 * g + (v & 3);
#pragma unroll
      for (int tn = 0; tn < TN; tn++) *(float*)(slab + r * RB + 4 * (32 * tn + (l & 31))) = acc[tm][tn][v];
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0): the slab is written
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; i++) {
      const int c = i * 64 + l, r = c / CPR, q = c - r * CPR;
      const u32v4 v = *(const u32v4*)(slab + r * RB + 16 * q);
      const int64_t row = mb + 32 * tm + r, col = nb + 4 * q;
      if (row >= p.M) continue;
      float* dst = Cz + row * ldc + col;
      if (full_cols) {
        if (OUT == OUT_PART) *(u32v4*)dst = v;
        else __builtin_nontemporal_store(v, (u32v4*)dst);
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++)
          if (col + e < p.N) dst[e] = __uint_as_float(v[e]);
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);            // the slab is read before the next block row overwrites it
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  }
}

// Quantizing epilogue (OUT_MXQ): the wave's TM x TN grid of 32x32 FP32
// accumulators with top-left output (mb, nb) becomes MXFP4 codes and E8M0
// bytes of C rounded to bf16 -- exactly what mxfp4_quantize (round-to-nearest,
// along rows, block Hadamard first when p.qhad) writes for the bf16 C of
// mxfp4_gemm_bf16.  A 32-block of a C row lies in one accumulator register
// across 32 lanes; the wave turns it around through its own slice of LDS, one
// 32-row block row at a time: the bf16 values go in as 4-byte column pairs (the
// pairing of the bf16 epilogue), then each lane reads whole 64-byte blocks
// (row l % 32) and encodes them in its registers with the quantizer's block
// encoder, storing 16 bytes of codes and one scale byte per block.  Rows are
// padded to 64 TN + 16 bytes so that 16 consecutive rows read conflict-free.
// The caller has made every wave finish its main loop (LDS is free).
template <int TM, int TN>
__device__ __forceinline__ void quantize_tile(const GemmArgs& p, uint8_t* smem, int64_t mb, int64_t nb,
                                              const v16f (&acc)[TM][TN]) {
  static_assert(TN % 2 == 0, "column pairs");
  constexpr int RB = 64 * TN + 16;                 // bytes per LDS row
  const int l = threadIdx.x & 63, g = l >> 5, w = threadIdx.x >> 6;
  uint8_t* slab = smem + w * 32 * RB;
  const bool odd = l & 1;
  const int64_t qrow = p.N / 2, srow = p.N / 32;
#pragma unroll
  for (int tm = 0; tm < TM; tm++) {
    // C rows 32 tm .. + 31 of the wave, as bf16, into the slab (row r at r * RB)
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int r = 8 * (v >> 2) + 4 * g + (v & 3);
#pragma unroll
      for (int tn = 0; tn < TN; tn += 2) {
        const float x = acc[tm][tn][v], y = acc[tm][tn + 1][v];
        const float got = dpp_swap_pairs(odd ? x : y);
        const float lo = odd ? got : x, hi = odd ? y : got;
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const int col = tn * 32 + (l & 30) + (odd ? 32 : 0);
        *(bf16x2_t*)(slab + r * RB + 2 * col) = (bf16x2_t){(__bf16)lo, (__bf16)hi};
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0): the slab is written
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    const int r = l & 31;
    const int64_t row = mb + 32 * tm + r;
#pragma unroll
    for (int j = 0; j < TN / 2; j++) {
      const int b = g + 2 * j;                      // block (32 columns) of the wave's row
      const uint8_t* src = slab + r * RB + 64 * b;
      float y[32];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const u32v4 v = *(const u32v4*)(src + 16 * q);
#pragma unroll
        for (int t = 0; t < 4; t++) {
          y[8 * q + 2 * t] = __uint_as_float(v[t] << 16);
          y[8 * q + 2 * t + 1] = __uint_as_float(v[t] & 0xFFFF0000u);
        }
      }
      const int64_t col = nb + 32 * b;
      if (row < p.M && col < p.N) {
        if (p.qhad) fwht32_inlane(y);
        uint32_t cw[4];
        const uint32_t byte = mx_rtn_block32(y, cw);
        __builtin_nontemporal_store((u32v4){cw[0], cw[1], cw[2], cw[3]}, (u32v4*)(p.qcodes + row * qrow + col / 2));
        __builtin_nontemporal_store((uint8_t)byte, p.qscales + row * srow + col / 32);
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);            // the slab is read before the next block row overwrites it
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  }
}

// MXFP4 kernel.  Workgroup = 4 waves (one per SIMD), output tile 256 x 256,
// wave (wm, wn) owns rows 128 wm .. +128 and columns 128 wn .. +128: 4 x 4
// MFMA tiles, 256 fp32 accumulators per lane (held in AGPRs).  Per output
// element pair this reads each LDS fragment once per 128 MACs, so LDS traffic
// (fragment reads plus the buffer->LDS fills) stays under the MFMA time.
//
// K stage = 256 elements: every operand row contributes 128 bytes, one whole
// cache line, to a stage, so each buffer->LDS instruction (64 lanes x 16 B)
// moves 8 complete lines.  Two stages (64 KB each) alternate; the loads for
// stage a + 2 are issued right after the barrier that ends the reads of stage
// a and have a full stage of MFMAs to land.
//
// Stage layout: row r at r * 128, 16-byte chunk c (contraction 32c .. 32c+31,
// one MX block) at position c ^ ((r >> 1) & 7).  The LDS of gfx950 serves 256
// bytes (64 banks) per clock, i.e. 16 lanes of a 16-byte read; an MFMA
// fragment read has lanes l = 0..31 take rows r0 + l at one chunk index, and
// among 16 consecutive rows the rows of equal parity (same 128-byte half of
// the bank space) then sit at eight distinct positions: no bank conflicts
// (measured with SQ_LDS_BANK_CONFLICT; XORing with r & 7 leaves 2-way ones).
//
// Scales: a scale group is 16 bytes per row = two stages.  Group G is loaded
// one operand at a time, A in the iteration of stage 2G - 3 and B in that of
// 2G - 2, into one of three group buffers, so a stage's scales are in LDS a
// full iteration before the stage starts and can be read under the MFMAs of
// the stage before.  Lanes read a row's whole 16 bytes (16 consecutive rows =
// 256 contiguous bytes, conflict-free); the stage's two scale bytes per
// 64-wide step (one per lane half) are then rearranged with one byte permute
// per row block so that step s takes byte s of a register.
constexpr int MX_BK = 256;                       // contraction elements per stage
constexpr int MX_ROW = MX_BK / 2;                // 128 code bytes per row per stage
constexpr int MX_OPND = 256 * MX_ROW;            // one operand's codes per stage: 32 KB
constexpr int MX_STAGE = 2 * MX_OPND;            // 64 KB
constexpr int MX_GROUP_OPND = 256 * 16;          // one operand's scale group: 4 KB
constexpr int MX_GROUP_OFF = 2 * MX_STAGE;       // 128 KB
constexpr int MX_GROUPS = 3;                     // scale group buffers
constexpr int MX_LDS = MX_GROUP_OFF + MX_GROUPS * 2 * MX_GROUP_OPND;   // 152 KB

// Per-wave operand blocks: TM row blocks of A (32 TM rows) and TN column
// blocks of B (32 TN columns).  Wide tiles: TM = 4, TN = 4 (or 2 for the
// 256 x 128 half tiles of the balanced schedule), waves 2 x 2.  Narrow tiles
// (M <= 128): TM = 1, 2 or 4, TN = 2, all four waves side by side along N.
template <int TM, int TN>
struct MxFrag {
  v4i a[TM], b[TN];
};

// Fragments of 64-wide step s of a stage for this lane: rows ra0 + 32t of the
// stage's A codes at sa and rb0 + 32t of its B codes at sb, chunk 2s + (lane
// half).
template <int TM, int TN>
__device__ __forceinline__ void mx_read_frag(const uint8_t* sa, const uint8_t* sb, int ra0, int rb0, int pos_byte,
                                             MxFrag<TM, TN>& f) {
#pragma unroll
  for (int t = 0; t < TM; t++) f.a[t] = *(const v4i*)(sa + (ra0 + 32 * t) * MX_ROW + pos_byte);
#pragma unroll
  for (int t = 0; t < TN; t++) f.b[t] = *(const v4i*)(sb + (rb0 + 32 * t) * MX_ROW + pos_byte);
}

// The 16 scale bytes of this lane's rows in one group (A rows ra0 + 32t of
// the A group at ga, then B rows rb0 + 32t of the B group at gb).
template <int TM, int TN>
__device__ __forceinline__ void mx_read_group(const uint8_t* ga, const uint8_t* gb, int ra0, int rb0,
                                              u32v4 (&d)[TM + TN]) {
#pragma unroll
  for (int t = 0; t < TM; t++) d[t] = *(const u32v4*)(ga + (ra0 + 32 * t) * 16);
#pragma unroll
  for (int t = 0; t < TN; t++) d[TM + t] = *(const u32v4*)(gb + (rb0 + 32 * t) * 16);
}

// Scale registers of one stage from its group's bytes: byte s = this lane's
// block of step s.  HALF = stage parity inside the group; sel picks the lane
// half's bytes; mask clears the bytes of steps past K (their products then
// vanish).
template <int HALF, int TM, int TN>
__device__ __forceinline__ void mx_stage_scales(const u32v4 (&d)[TM + TN], uint32_t sel, uint32_t mask,
                                                uint32_t (&sa)[TM], uint32_t (&sb)[TN]) {
#pragma unroll
  for (int t = 0; t < TM; t++) sa[t] = __builtin_amdgcn_perm(d[t][2 * HALF + 1], d[t][2 * HALF], sel) & mask;
#pragma unroll
  for (int t = 0; t < TN; t++)
    sb[t] = __builtin_amdgcn_perm(d[TM + t][2 * HALF + 1], d[TM + t][2 * HALF], sel) & mask;
}

template <int S, int TM, int TN>
__device__ __forceinline__ void mx_mfma(v16f (&acc)[TM][TN], const MxFrag<TM, TN>& f, const uint32_t (&sa)[TM],
                                        const uint32_t (&sb)[TN]) {
#pragma unroll
  for (int i = 0; i < TM; i++) {
    const v8i a = __builtin_shufflevector(f.a[i], f.a[i], 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const v8i b = __builtin_shufflevector(f.b[j], f.b[j], 0, 1, 2, 3, -1, -1, -1, -1);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 4, 4, S, (int)sa[i], S,
                                                                 (int)sb[j]);
    }
  }
}

// Scheduling of one step: NM MFMAs with, ahead of each of the first ones, one
// buffer->LDS load (NV of them) and one DS read (ND of them), in the program
// order in which they were issued.
template <int NV, int ND, int NM>
__device__ __forceinline__ void mx_sched() {
#pragma unroll
  for (int q = 0; q < NM; q++) {
    if (q < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one buffer->LDS load
    if (q < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // one MFMA
  }
  if (NV > NM) __builtin_amdgcn_sched_group_barrier(0x020, NV - NM, 0);
  if (ND > NM) __builtin_amdgcn_sched_group_barrier(0x100, ND - NM, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Operand resources of one tile: they end at the operand's last row of the
// tile (at most ROWS rows from its first), so rows past M or N read as zeros.
// Each of the NW waves loads RPW = ROWS / NW rows per stage, 8 rows per load.
struct MxOperand {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t code_off[2];  // this lane's offset for loads 0 and 1 of the wave (load j: [j & 1] + (j >> 1) * 16 rows)
  uint32_t scale_off;    // this lane's row in the wave's 64-row scale piece
};

template <int ROWS, int NW = 4>
__device__ __forceinline__ MxOperand mx_make_operand(const uint8_t* codes, const uint8_t* scales, int64_t rows_total,
                                                     int64_t row0, int64_t K, int w, int l) {
  constexpr int RPW = ROWS / NW;
  const int64_t krow = K / 2, srow = K / 32;
  int64_t nrows = rows_total - row0;
  if (nrows > ROWS) nrows = ROWS;
  if (nrows < 0) nrows = 0;   // a half tile wholly past N
  MxOperand o;
  o.codes = __builtin_amdgcn_make_buffer_rsrc((void*)(codes + row0 * krow), (short)0, (int)(nrows * krow), kRsrcWord3);
  o.scales = __builtin_amdgcn_make_buffer_rsrc((void*)(scales + row0 * srow), (short)0, (int)(nrows * srow), kRsrcWord3);
  // load j of wave w fills rows RPW w + 8j .. +7; lane l writes position l & 7
  // of row r = RPW w + 8j + (l >> 3), i.e. chunk (l & 7) ^ ((r >> 1) & 7), where
  // (r >> 1) & 7 = (4j + (l >> 4)) & 7 depends on the parity of j only
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = RPW * w + 8 * j + (l >> 3);
    o.code_off[j] = (uint32_t)(row * krow + (((l & 7) ^ ((row >> 1) & 7)) << 4));
  }
  // scale piece w % 4 is rows 64 (w % 4) .. + 63 (past ROWS: out of range,
  // zeros); with 8 waves, waves 0-3 load A's pieces and waves 4-7 B's
  o.scale_off = (uint32_t)((64 * (w & 3) + l) * srow);
  return o;
}

// Code loads L0 .. L1-1 of this wave for absolute stage kt into stage buffer
// st: loads 0 .. LA-1 are A's (8 LA rows per wave), the next LB are B's
// (8 LB rows per wave).
template <int L0, int L1, int LA, int LB>
__device__ __forceinline__ void mx_issue_codes(const MxOperand& oa, const MxOperand& ob, uint8_t* st, int kt,
                                               uint32_t krow16, int w) {
  const int soff = kt * MX_ROW;
#pragma unroll
  for (int L = L0; L < L1; L++) {
    const int j = L < LA ? L : L - LA;
    const int rpw = L < LA ? 8 * LA : 8 * LB;
    const MxOperand& o = L < LA ? oa : ob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.codes,
                                             (lds_void*)(st + (L < LA ? 0 : MX_OPND) + (rpw * w + 8 * j) * MX_ROW),
                                             16, o.code_off[j & 1] + (uint32_t)(j >> 1) * krow16, soff, 0, 0);
  }
}

// Fused activation quantization for the narrow tiles: stages kt0 ..
// kt0 + nsp - 1 of rows 0 .. 32 TM - 1 of the bf16 input p.x [M, K] (row
// stride p.ldx), quantized to MXFP4 with round-to-nearest per 32-block (block
// Hadamard first when HAD): the same codes and scale bytes as the quantizer
// writes for this input.  Block i of the range is chunk c = i % 8 of row
// r = (i / 8) % Mr in stage st = i / (8 Mr), Mr = min(M, 32 TM) (the rows past
// M are written as zeros separately, so that every wave gets its share of
// the real blocks).  Stage st's codes go to
// aslot(st) in the stage layout (row r at r * 128, chunk c at
// c ^ ((r >> 1) & 7)), its scale bytes to byte 8 (st % 2) + c of row r's 16
// in ascl(st / 2).  Rows past M and blocks past K come out as zero codes with
// scale byte 0, which is what the code loads of the unfused path read there.
struct MxXBlock {
  uint32_t w[16];      // 32 bf16 values, element 2j in the low half of w[j]
  int r, c, st;
  bool ok;             // inside M and K (else the block is zero)
};

__device__ __forceinline__ void mx_fill_load(const GemmArgs& p, int kt0, int i, int Mr, MxXBlock& b) {
  b.c = i & 7;
  b.st = (i >> 3) / Mr;
  b.r = (i >> 3) - b.st * Mr;
  const int64_t k = (int64_t)(kt0 + b.st) * MX_BK + 32 * b.c;
  b.ok = k < p.K;
  if (!b.ok) return;
  const uint16_t* src = p.x + (int64_t)b.r * p.ldx + k;
  if (p.x_vec) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const u32v4 v = *(const u32v4*)(src + 8 * q);
#pragma unroll
      for (int j = 0; j < 4; j++) b.w[4 * q + j] = v[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; j++) b.w[j] = (uint32_t)src[2 * j] | ((uint32_t)src[2 * j + 1] << 16);
  }
}

template <bool HAD, typename AS, typename AG>
__device__ __forceinline__ void mx_fill_store(const MxXBlock& b, AS&& aslot, AG&& ascl) {
  uint32_t cw[4] = {0u, 0u, 0u, 0u};
  uint32_t byte = 0u;
  if (b.ok) {
    float y[32];
#pragma unroll
    for (int j = 0; j < 16; j++) {
      y[2 * j] = __uint_as_float(b.w[j] << 16);
      y[2 * j + 1] = __uint_as_float(b.w[j] & 0xFFFF0000u);
    }
    if (HAD) fwht32_inlane(y);
    byte = mx_rtn_block32(y, cw);
  }
  *(u32v4*)(aslot(b.st) + b.r * MX_ROW + ((b.c ^ ((b.r >> 1) & 7)) << 4)) = (u32v4){cw[0], cw[1], cw[2], cw[3]};
  ascl(b.st >> 1)[b.r * 16 + 8 * (b.st & 1) + b.c] = (uint8_t)byte;
}

// One output tile (32 TM WM x 32 TN (4 / WM)), contraction stages kt0 ..
// kt1-1 (kt0 even).  Iteration a (stage a), each step = TM TN MFMAs with the
// next step's fragment reads under them:
//   step 0: + loads 6..11 of stage a + 1
//   step 1: + loads 12.. of stage a + 1, the scale piece of iteration a, and
//           the scale bytes of stage a + 1 (when a + 1 opens a group)
//   step 2: then stage a + 1's scale registers
//   wait for this wave's loads of stage a + 1 and its LDS reads; barrier
//   step 3: stage a + 1's step-0 fragments first, + loads 0..5 of stage a + 2
//           (into stage a's buffer)
// A stage's buffer->LDS loads are spread over three steps: bunched into one,
// they back up the address unit and the stalled load issue holds back the
// MFMAs queued behind it.  The body has no branches: loads for stages past
// the end land in buffers that are never read again, and reads past the end
// are never consumed.
//
// FA (fused activation quantization, narrow tiles only): A is not loaded as
// codes but quantized here from the bf16 input p.x (MXFP4 round-to-nearest,
// with the block Hadamard when HAD) for the whole contraction range kt0 ..
// kt1 before the main loop, into A slots that take the place of the (unused)
// A halves of the two stage buffers, with its scale bytes in the A halves of
// the scale-group buffers.  The codes and scale bytes are those the
// quantizer writes for the same input, so the products are the same.
template <int TM, int TN, int WM, int OUT, bool FA = false, bool HAD = false>
__device__ __forceinline__ void mx_tile(const GemmArgs& p, uint8_t* smem, int64_t m0, int64_t n0, int kt0, int kt1,
                                        float* Cz) {
  constexpr int WN = 4 / WM;                     // waves along N
  constexpr int LA = TM * WM, LB = TN * WN;      // code row blocks per wave per stage (8 rows each)
  constexpr int LAL = FA ? 0 : LA;               // A code loads per wave per stage
  constexpr int NL = LAL + LB;
  constexpr int P1 = NL < 6 ? NL : 6, P2 = NL < 12 ? NL : 12;   // load parts: [0, P1) [P1, P2) [P2, NL)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, h = l >> 5;
  const int wm = w / WN, wn = w % WN;
  const int ra0 = wm * (32 * TM) + (l & 31), rb0 = wn * (32 * TN) + (l & 31);
  auto pos = [&](int c) { return ((c ^ ((l >> 1) & 7)) << 4); };   // chunk c of a row r with r % 32 == l % 32
  const uint32_t sel = h ? 0x07050301u : 0x06040200u;
  const int ksteps = (int)(p.K / 64);                              // 64-wide steps in the whole contraction

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = (v16f){};

  if (kt1 > kt0) {
    const uint32_t krow16 = (uint32_t)(16 * (p.K / 2));
    // (FA: no A codes are loaded; the descriptor only lends its scale row
    // offset, which is the same for both operands)
    const MxOperand oa = mx_make_operand<32 * TM * WM>(FA ? p.b : p.a, FA ? p.bs : p.as, FA ? p.N : p.M, m0, p.K,
                                                       w, l);
    const MxOperand ob = mx_make_operand<32 * TN * WN>(p.b, p.bs, p.N, n0, p.K, w, l);
    auto stage = [&](int a) { return smem + (a & 1) * MX_STAGE; };
    auto group = [&](int G) { return smem + MX_GROUP_OFF + (G % MX_GROUPS) * 2 * MX_GROUP_OPND; };
    // FA: A codes of stage kt0 + i in slot i (32 TM rows x 128 bytes, the
    // stage layout), slots filling the A half of stage buffer 0, then of
    // stage buffer 1; A scales of group G0 + j in the A halves of the group
    // buffers, 32 TM rows x 16 bytes each
    constexpr int A_SLOT = 32 * TM * MX_ROW, A_GSLOT = 32 * TM * 16, A_GPER = MX_GROUP_OPND / A_GSLOT;
    auto aslot = [&](int i) -> uint8_t* {
      const int off = i * A_SLOT;
      return off < MX_OPND ? smem + off : smem + MX_STAGE + (off - MX_OPND);
    };
    auto ascl = [&](int j) -> uint8_t* {
      return smem + MX_GROUP_OFF + (j / A_GPER) * 2 * MX_GROUP_OPND + (j % A_GPER) * A_GSLOT;
    };
    auto abuf = [&](int a) -> const uint8_t* {
      if constexpr (FA) return aslot(a - kt0);
      else return stage(a);
    };
    auto agrp = [&](int G) -> const uint8_t* {
      if constexpr (FA) return ascl(G - (kt0 >> 1));
      else return group(G);
    };
    // scale-byte mask of absolute stage a: bytes of the 64-wide steps below K
    auto mask_of = [&](int a) -> uint32_t {
      const int v = min(max(ksteps - 4 * a, 0), 4);
      return (uint32_t)((1ull << (8 * v)) - 1ull);
    };
    // piece w of one operand's scale group G (a value select of the resource
    // on a uniform flag; the row offset is the same for both operands)
    auto issue_piece = [&](int G, int b_side) {
      const __amdgpu_buffer_rsrc_t r = b_side ? ob.scales : oa.scales;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(group(G) + b_side * MX_GROUP_OPND + w * 1024), 16,
                                               oa.scale_off, 16 * G, 0, 0);
    };

    // prologue: group kt0/2 (A and B), group kt0/2 + 1's A piece (the piece
    // of iteration kt0 - 1), stage kt0, and the first part of stage kt0 + 1
    // (iteration kt0 issues the rest)
    const int G0 = kt0 >> 1;
    // FA: quantize A for stages kt0 .. kt0 + nsp - 1 (nsp = the stage count
    // rounded up to the loop's pairs; stages past K come out as zero codes);
    // the inputs of this thread's first two blocks are loaded ahead of the B
    // loads (vmcnt counts in order: loads issued after the B loads would wait
    // for them)
    const int nsp = (kt1 - kt0 + 1) & ~1;
    const int Mr = p.M < 32 * TM ? (int)p.M : 32 * TM;   // rows of A that exist
    const int nblk = nsp * Mr * 8;
    constexpr int XPRE = 4;                      // blocks per thread loaded ahead
    MxXBlock xb[XPRE];
    if constexpr (FA) {
#pragma unroll
      for (int q = 0; q < XPRE; q++) {
        xb[q].ok = false;
        if ((int)threadIdx.x + 256 * q < nblk) mx_fill_load(p, kt0, threadIdx.x + 256 * q, Mr, xb[q]);
      }
    }
    if (!FA) issue_piece(G0, 0);
    issue_piece(G0, 1);
    if (!FA) issue_piece(G0 + 1, 0);
    mx_issue_codes<0, NL, LAL, LB>(oa, ob, stage(kt0), kt0, krow16, w);
    mx_issue_codes<0, P1, LAL, LB>(oa, ob, stage(kt0 + 1), kt0 + 1, krow16, w);
    if constexpr (FA) {
#pragma unroll
      for (int q = 0; q < XPRE; q++)
        if ((int)threadIdx.x + 256 * q < nblk) mx_fill_store<HAD>(xb[q], aslot, ascl);
      for (int i = threadIdx.x + 256 * XPRE; i < nblk; i += 256) {
        mx_fill_load(p, kt0, i, Mr, xb[0]);
        mx_fill_store<HAD>(xb[0], aslot, ascl);
      }
      // rows Mr .. 32 TM - 1: zero codes, scale byte 0
      const int zr = 32 * TM - Mr;
      for (int i = threadIdx.x; i < nsp * zr * 8; i += 256) {
        MxXBlock z;
        z.ok = false;
        z.c = i & 7;
        z.st = (i >> 3) / zr;
        z.r = Mr + (i >> 3) - z.st * zr;
        mx_fill_store<HAD>(z, aslot, ascl);
      }
    }
    wait_cnt<P1, FA ? 0 : 15>();
    block_barrier();

    MxFrag<TM, TN> f0, f1;
    uint32_t sa[TM], sb[TN];
    u32v4 gd[TM + TN];
    mx_read_group<TM, TN>(agrp(G0), group(G0) + MX_GROUP_OPND, ra0, rb0, gd);
    mx_stage_scales<0, TM, TN>(gd, sel, mask_of(kt0), sa, sb);
    mx_read_frag<TM, TN>(abuf(kt0), stage(kt0) + MX_OPND, ra0, rb0, pos(h), f0);
    // one iteration; H = a & 1 (kt0 is even, the loop takes stages in pairs)
    auto iteration = [&](auto Hc, int a) {
      constexpr int H = decltype(Hc)::value;
      constexpr int NM = TM * TN;             // MFMAs per step
      constexpr int NF = TM + TN;             // fragment reads per step
      const uint8_t* st = stage(H) + MX_OPND;   // this stage's B codes
      const uint8_t* sta = abuf(a);             // and its A codes
      mx_issue_codes<P1, P2, LAL, LB>(oa, ob, stage(H ^ 1), a + 1, krow16, w);
      mx_read_frag<TM, TN>(sta, st, ra0, rb0, pos(2 + h), f1);
      mx_mfma<0, TM, TN>(acc, f0, sa, sb);
      mx_sched<P2 - P1, NF, NM>();
      mx_issue_codes<P2, NL, LAL, LB>(oa, ob, stage(H ^ 1), a + 1, krow16, w);
      // iteration a's scale piece: group (a + 3) / 2's A piece when a is odd,
      // group a / 2 + 1's B piece when a is even.  Group G is then complete at
      // the barrier of iteration 2G - 2, before stage 2G's scale bytes are
      // read in iteration 2G - 1, and its buffer last held group G - 3.
      if (!FA || !H) issue_piece(H ? (a + 3) >> 1 : (a >> 1) + 1, H ^ 1);
      if (H)   // stage a + 1 opens the next group
        mx_read_group<TM, TN>(agrp((a + 1) >> 1), group((a + 1) >> 1) + MX_GROUP_OPND, ra0, rb0, gd);
      mx_read_frag<TM, TN>(sta, st, ra0, rb0, pos(4 + h), f0);
      mx_mfma<1, TM, TN>(acc, f1, sa, sb);
      mx_sched<NL - P2 + 1, NF + (H ? TM + TN : 0), NM>();
      mx_read_frag<TM, TN>(sta, st, ra0, rb0, pos(6 + h), f1);
      mx_mfma<2, TM, TN>(acc, f0, sa, sb);
      uint32_t sa_n[TM], sb_n[TN];
      mx_stage_scales<H ^ 1, TM, TN>(gd, sel, mask_of(a + 1), sa_n, sb_n);
      mx_sched<0, NF, NM>();
      wait_cnt<0, 0>();
      block_barrier();
      mx_read_frag<TM, TN>(abuf(a + 1), stage(H ^ 1) + MX_OPND, ra0, rb0, pos(h), f0);
      mx_issue_codes<0, P1, LAL, LB>(oa, ob, stage(H), a + 2, krow16, w);
      mx_mfma<3, TM, TN>(acc, f1, sa, sb);
      // the fragment reads first, then the loads, over the MFMAs
#pragma unroll
      for (int q = 0; q < NF; q++) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      }
#pragma unroll
      for (int q = 0; q < P1; q++) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one buffer->LDS load
        if (NF + q < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      }
      if (NM > NF + P1) __builtin_amdgcn_sched_group_barrier(0x008, NM - NF - P1, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < TM; t++) sa[t] = sa_n[t];
#pragma unroll
      for (int t = 0; t < TN; t++) sb[t] = sb_n[t];
    };
    // an odd stage count only happens at the end of K: the extra stage then
    // lies past K, so its scale mask is zero and it adds nothing
    for (int a = kt0; a < kt1; a += 2) {
      iteration(std::integral_constant<int, 0>{}, a);
      iteration(std::integral_constant<int, 1>{}, a + 1);
    }
    wait_cnt<0, 0>();   // nothing may still write LDS when the workgroup exits
  }
  if constexpr (OUT == OUT_MXQ) {
    block_barrier();   // every wave is past its main loop: LDS is free for the epilogue
    quantize_tile<TM, TN>(p, smem, m0 + wm * (32 * TM), n0 + wn * (32 * TN), acc);
  } else if constexpr (TM == 4 && WM == 2 && (OUT == OUT_F32 || OUT == OUT_PART)) {
    block_barrier();   // LDS is free for the turn-around
    store_tile_lds<TM, TN, OUT>(p, smem, Cz, m0 + wm * (32 * TM), n0 + wn * (32 * TN), acc);
  } else {
    store_tile<TM, TN, false, OUT>(p, Cz, m0 + wm * (32 * TM), n0 + wn * (32 * TN), acc);
  }
}

// Work items.  Workgroups are dispatched in id order to whichever compute
// unit frees first, so the first wave of ids sets each compute unit's phase
// and the last ids fill the compute units that free up last.  Without split-K
// the grid is laid out as
//   [R first halves] [T - R full tiles] [R second halves]
// where T = 256 x 256 tiles and R = T mod (compute units) (p.rem; 0 when the
// tiles divide evenly or a split is used): the R remainder tiles are cut into
// two 256 x 128 halves, one run by the first workgroups and one by the last,
// so every compute unit ends at the same time, and the C stores of the two
// groups of compute units fall at alternating times.  With at most half as
// many tiles as compute units, R = T: every tile runs as two halves on two
// compute units (measured: 256 x 14336 x 4096 29.3 -> 22.4 us, 4096 x 1024 x
// 4096 28.0 -> 20.2 us).  (Four phases, with
// quarter and three-quarter pieces, measured ~10 % slower.)  Within each range, consecutive workgroup ids go to consecutive XCDs, so the
// ids one XCD runs are gathered into a contiguous run of tiles, walked in
// groups of GROUP_M tile rows.
__device__ __forceinline__ int mx_walk(const GemmArgs& p, int t, int& tn) {
  constexpr int GROUP_M = MXFP4_GROUP_M;
  const int group = t / (GROUP_M * p.ntn);
  const int first_m = group * GROUP_M;
  const int gm = min(p.ntm - first_m, GROUP_M);
  const int in_group = t - group * GROUP_M * p.ntn;
  tn = in_group / gm;
  return first_m + in_group % gm;
}
__device__ __forceinline__ int xcd_gather(int id, int n) {
  return (n & 7) == 0 ? (id & 7) * (n >> 3) + (id >> 3) : id;
}

// Split ranges start on even stages (a scale group spans two stages).
// OUT: what the launch writes (fp32 C, split-K partials or bf16 C).
template <int OUT>
__global__ void __launch_bounds__(256, 1) gemm_mx_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX_LDS];
  int b = blockIdx.x, z = blockIdx.y;
  if (p.splits > 1) {
    // Split launches: the (split, tile) pairs in split-major order are cut
    // into eight contiguous runs, one per XCD (dispatch id i goes to XCD
    // i % 8), so the workgroups sharing an L2 mostly share one split's
    // contraction range and neighbouring tiles, i.e. the same operand panels.
    // (Measured: 768x3072x50432 109 -> 78 us, 3072x768x50432 90 -> 78 us.)
    const int total = gridDim.x * gridDim.y, id = z * gridDim.x + b;
    const int base = total >> 3, extra = total & 7, x = id & 7, slot = id >> 3;
    const int pos = (x < extra ? x * (base + 1) : extra * (base + 1) + (x - extra) * base) + slot;
    z = pos / gridDim.x;
    b = pos - z * gridDim.x;
  }
  const int pairs = (p.k_tiles + 1) >> 1;
  const int kt0 = 2 * (int)((int64_t)pairs * z / p.splits);
  int kt1 = 2 * (int)((int64_t)pairs * (z + 1) / p.splits);
  if (kt1 > p.k_tiles) kt1 = p.k_tiles;
  float* Cz = p.C + (int64_t)z * p.split_stride;
  const int R = p.rem, T = p.ntm * p.ntn;
  int tm, tn;
  const int F = T - R;
  if (b >= R && b < R + F) {
    tm = mx_walk(p, p.splits > 1 ? b : xcd_gather(b - R, F), tn);   // (split runs are already per XCD)
    mx_tile<4, 4, 2, OUT>(p, smem, (int64_t)tm * BM, (int64_t)tn * BN, kt0, kt1, Cz);
  } else {
    const int second = b >= R + F;
    const int i = second ? b - R - F : b;
    tm = mx_walk(p, F + xcd_gather(i, R), tn);
    mx_tile<4, 2, 2, OUT>(p, smem, (int64_t)tm * BM, (int64_t)tn * BN + 128 * second, kt0, kt1, Cz);
  }
}

// Wide tiles with 8 waves (two per SIMD), for short contractions (at most
// four stages): measured against the 4-wave kernel, 50432 x 3072 x 768 161 ->
// 128 us and 1024^3 17.2 -> 13.0 us, but 10-23 % slower at K >= 3072 (the two
// waves of a SIMD wait at the same barriers), so plan_gemm takes it for
// K <= 1024 only.  Wave w owns rows 64 (w / 2) .. + 63
// and columns (32 TN) (w % 2) .. of the 256 x (64 TN) tile, 2 x TN MFMA tiles
// (128 accumulators at TN = 4).  The loop is deliberately simple -- each step
// reads its fragments and waits for them -- because the other wave on the SIMD
// issues its MFMAs meanwhile.  Stage a + 1's loads are issued right after the
// barrier that frees its buffer and waited for at the end of stage a; scale
// group G + 1 is loaded in stage 2G.  Same LDS layout as mx_tile.
template <int TN, int OUT>
__device__ __forceinline__ void mx8_tile(const GemmArgs& p, uint8_t* smem, int64_t m0, int64_t n0, int kt0, int kt1,
                                         float* Cz) {
  constexpr int TM = 2, NW = 8, WN = 2;           // 4 x 2 waves
  constexpr int LA = 4, LB = TN;                 // code loads (8 rows each) per wave per stage: A 32 rows, B 8 TN rows
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, h = l >> 5;
  const int wm = w / WN, wn = w % WN;
  const int ra0 = wm * (32 * TM) + (l & 31), rb0 = wn * (32 * TN) + (l & 31);
  auto pos = [&](int c) { return ((c ^ ((l >> 1) & 7)) << 4); };
  const uint32_t sel = h ? 0x07050301u : 0x06040200u;
  const int ksteps = (int)(p.K / 64);
  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = (v16f){};
  if (kt1 > kt0) {
    const uint32_t krow16 = (uint32_t)(16 * (p.K / 2));
    const MxOperand oa = mx_make_operand<256, NW>(p.a, p.as, p.M, m0, p.K, w, l);
    const MxOperand ob = mx_make_operand<32 * TN * WN, NW>(p.b, p.bs, p.N, n0, p.K, w, l);
    auto stage = [&](int a) { return smem + (a & 1) * MX_STAGE; };
    auto group = [&](int G) { return smem + MX_GROUP_OFF + (G % MX_GROUPS) * 2 * MX_GROUP_OPND; };
    auto issue_group = [&](int G) {               // waves 0-3 load A's pieces, 4-7 B's
      const int side = w >> 2;
      const __amdgpu_buffer_rsrc_t r = side ? ob.scales : oa.scales;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(group(G) + side * MX_GROUP_OPND + (w & 3) * 1024), 16,
                                               oa.scale_off, 16 * G, 0, 0);
    };
    auto mask_of = [&](int a) -> uint32_t {
      const int v = min(max(ksteps - 4 * a, 0), 4);
      return (uint32_t)((1ull << (8 * v)) - 1ull);
    };
    issue_group(kt0 >> 1);
    mx_issue_codes<0, LA + LB, LA, LB>(oa, ob, stage(kt0), kt0, krow16, w);
    wait_cnt<0, 15>();
    block_barrier();
    for (int a = kt0; a < kt1; a++) {
      const uint8_t* sa_ = stage(a);
      const uint8_t* sb_ = stage(a) + MX_OPND;
      if (a + 1 < kt1) mx_issue_codes<0, LA + LB, LA, LB>(oa, ob, stage(a + 1), a + 1, krow16, w);
      if (!(a & 1) && a + 2 < kt1) issue_group((a >> 1) + 1);
      // this stage's scale bytes: 8 per row (half a group), one byte per 64-wide step in each register
      const uint8_t* ga = group(a >> 1) + 8 * (a & 1);
      const uint8_t* gb = ga + MX_GROUP_OPND;
      uint32_t sa[TM], sb[TN];
      const uint32_t mask = mask_of(a);
#pragma unroll
      for (int t = 0; t < TM; t++) {
        const uint2 v = *(const uint2*)(ga + (ra0 + 32 * t) * 16);
        sa[t] = __builtin_amdgcn_perm(v.y, v.x, sel) & mask;
      }
#pragma unroll
      for (int t = 0; t < TN; t++) {
        const uint2 v = *(const uint2*)(gb + (rb0 + 32 * t) * 16);
        sb[t] = __builtin_amdgcn_perm(v.y, v.x, sel) & mask;
      }
      MxFrag<TM, TN> f;
      mx_read_frag<TM, TN>(sa_, sb_, ra0, rb0, pos(0 + h), f);
      mx_mfma<0, TM, TN>(acc, f, sa, sb);
      mx_read_frag<TM, TN>(sa_, sb_, ra0, rb0, pos(2 + h), f);
      mx_mfma<1, TM, TN>(acc, f, sa, sb);
      mx_read_frag<TM, TN>(sa_, sb_, ra0, rb0, pos(4 + h), f);
      mx_mfma<2, TM, TN>(acc, f, sa, sb);
      mx_read_frag<TM, TN>(sa_, sb_, ra0, rb0, pos(6 + h), f);
      mx_mfma<3, TM, TN>(acc, f, sa, sb);
      wait_cnt<0, 0>();      // this wave's loads of stage a + 1 (and scale pieces) landed; its reads done
      block_barrier();
    }
  }
  if constexpr (OUT == OUT_MXQ) {
    block_barrier();
    quantize_tile<TM, TN>(p, smem, m0 + wm * (32 * TM), n0 + wn * (32 * TN), acc);
  } else {
    store_tile<TM, TN, false, OUT>(p, Cz, m0 + wm * (32 * TM), n0 + wn * (32 * TN), acc);
  }
}

// The wide kernel with 8 waves (mx8_tile): 64 x 128 per wave (half tiles
// 64 x 64), 128 accumulators, two waves per SIMD.
template <int OUT>
__global__ void __launch_bounds__(512, 1) gemm_mx8_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX_LDS];
  int b = blockIdx.x, z = blockIdx.y;
  if (p.splits > 1) {
    const int total = gridDim.x * gridDim.y, id = z * gridDim.x + b;
    const int base = total >> 3, extra = total & 7, x = id & 7, slot = id >> 3;
    const int pos = (x < extra ? x * (base + 1) : extra * (base + 1) + (x - extra) * base) + slot;
    z = pos / gridDim.x;
    b = pos - z * gridDim.x;
  }
  const int pairs = (p.k_tiles + 1) >> 1;
  const int kt0 = 2 * (int)((int64_t)pairs * z / p.splits);
  int kt1 = 2 * (int)((int64_t)pairs * (z + 1) / p.splits);
  if (kt1 > p.k_tiles) kt1 = p.k_tiles;
  float* Cz = p.C + (int64_t)z * p.split_stride;
  const int R = p.rem, T = p.ntm * p.ntn;
  int tm, tn;
  const int F = T - R;
  if (b >= R && b < R + F) {
    tm = mx_walk(p, p.splits > 1 ? b : xcd_gather(b - R, F), tn);
    mx8_tile<4, OUT>(p, smem, (int64_t)tm * BM, (int64_t)tn * BN, kt0, kt1, Cz);
  } else {
    const int second = b >= R + F;
    const int i = second ? b - R - F : b;
    tm = mx_walk(p, F + xcd_gather(i, R), tn);
    mx8_tile<2, OUT>(p, smem, (int64_t)tm * BM, (int64_t)tn * BN + 128 * second, kt0, kt1, Cz);
  }
}

// Narrow MXFP4 GEMM (M <= 32 TM <= 128 where the decode kernel is not taken:
// long contractions against short weights): 32 TM x 256 tiles, the four waves
// side by side along N, so no MFMA work is spent on rows past M; these shapes
// stream the weights from HBM and are split along K for enough workgroups.
// Grid: (N tiles, splits).
template <int TM, int OUT>
__global__ void __launch_bounds__(256, 1) gemm_mx_narrow_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX_LDS];
  const int z = blockIdx.y;
  const int pairs = (p.k_tiles + 1) >> 1;
  const int kt0 = 2 * (int)((int64_t)pairs * z / p.splits);
  int kt1 = 2 * (int)((int64_t)pairs * (z + 1) / p.splits);
  if (kt1 > p.k_tiles) kt1 = p.k_tiles;
  float* Cz = p.C + (int64_t)z * p.split_stride;
  mx_tile<TM, 2, 1, OUT>(p, smem, 0, (int64_t)blockIdx.x * 256, kt0, kt1, Cz);
}

// Narrow MXFP4 GEMM whose A operand is quantized inside the kernel from the
// bf16 activations (online activation quantization, "Bridging the Gap Between
// Promise and Performance for Microscaling FP4 Quantization", abstract:
// activations rotated and quantized on the fly in front of FP4 GEMMs whose
// weights were rotated offline).  Same grid, split and tile pipeline as
// gemm_mx_narrow_kernel, so the result equals quantize-then-GEMM bit for bit.
// Each workgroup quantizes the activation rows for its own contraction range
// (at most 16 / TM stages; the planner checks, and uses it for TM = 1 only).
template <int TM, bool HAD, int OUT>
__global__ void __launch_bounds__(256, 1) gemm_mx_fused_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX_LDS];
  const int z = blockIdx.y;
  const int pairs = (p.k_tiles + 1) >> 1;
  const int kt0 = 2 * (int)((int64_t)pairs * z / p.splits);
  int kt1 = 2 * (int)((int64_t)pairs * (z + 1) / p.splits);
  if (kt1 > p.k_tiles) kt1 = p.k_tiles;
  float* Cz = p.C + (int64_t)z * p.split_stride;
  mx_tile<TM, 2, 1, OUT, true, HAD>(p, smem, 0, (int64_t)blockIdx.x * 256, kt0, kt1, Cz);
}

// Decode-shaped MXFP4 GEMM (up to 128 activation rows against the weights):
// the weights stream from HBM once, so the kernel is built for bytes in
// flight rather than MFMA rate.  A workgroup owns 16 output columns (weight
// rows) over the whole contraction; its NW waves take contiguous ranges of
// rounds (four 128-wide steps each), and the per-wave sums are added in LDS in
// wave order: no split-K workspace and no second launch.
//
// One step is v_mfma_scale_f32_16x16x128_f8f6f4 with the weights as the
// first operand: lane l holds block 4s + l / 16 of weight row n0 + l % 16
// (16 code bytes) and that block's scale byte, and the same block of
// activation row 16t + l % 16 (TMR = 1 .. 8 tiles of 16 rows); the output
// lane l holds is C[16t + l % 16][n0 + 4 (l / 16) + v], v = 0..3.
//
// That operand layout gives each row only 64 bytes per load instruction,
// and half-line loads stream at about half the rate of whole 128-byte lines
// (measured on the configuration-3 decode shapes), so codes travel through
// LDS: each wave owns R slots of one step pair (16 weight rows and 16 TMR
// activation rows, 128 bytes each) filled by buffer->LDS loads of whole
// lines (8 rows x 128 bytes per instruction, chunk c of row q stored at
// position c ^ ((q >> 1) & 7), which keeps the fragment reads free of bank
// conflicts), and reads its fragments back from its own slots, so no barrier
// is needed.  Scale bytes come straight to registers, 16 bytes (one round)
// per lane and operand.  Rows past M or N read as zeros through the buffer
// resources and are not stored; code chunks past K are loaded as zeros and
// the scale bytes of steps past K are cleared, so those products vanish.
constexpr uint32_t kOutOfRange = 0x80000000u;   // a buffer offset past every operand the kernel reads
#ifndef MXFP4_DECODE_NW
#define MXFP4_DECODE_NW 4     // waves per workgroup, each on its own range of the contraction
#endif

// TMR activation tiles and TN weight tiles of 16 rows (16 TN output columns
// per workgroup); R slots per wave (R / 2 rounds in flight).
template <int TMR, int TN, int R>
struct DecodeShape {
  static constexpr int ROWS = 16 * (TN + TMR);    // slot rows: 16 TN weight rows, then 16 TMR activation rows
  static constexpr int SLOT = ROWS * 128;
  static constexpr int LDS = MXFP4_DECODE_NW * R * SLOT;
};

template <int TMR, int TN, int R, int OUT>
__global__ void __launch_bounds__(64 * MXFP4_DECODE_NW) gemm_mx_decode_kernel(GemmArgs p) {
  static_assert(OUT == OUT_F32 || OUT == OUT_BF16, "the decode kernel writes C directly");
  static_assert(R % 2 == 0 && R >= 2, "slots come in rounds of two");
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef DecodeShape<TMR, TN, R> Shape;
  constexpr int NW = MXFP4_DECODE_NW;
  constexpr int SLOT = Shape::SLOT;
  constexpr int NDMA = Shape::ROWS / 8;         // buffer->LDS loads per slot
  constexpr int NB = 2 * TN;                    // the first NB of them move weight rows
  constexpr int RQ = R / 2;                     // rounds in flight
  constexpr int VM_ROUND = 2 * NDMA + TN + TMR; // vector memory operations issued per round
  static_assert(NW * TMR * TN * 64 * 16 <= Shape::LDS, "the wave sums reuse the slots");
  __shared__ __attribute__((aligned(16))) uint8_t smem[Shape::LDS];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * TN);
  const int64_t krow = p.K / 2, srow = p.K / 32;
  const int steps = (int)(p.K / 128);
  const int rounds = (steps + 3) >> 2;
  const int c0 = (int)((int64_t)rounds * w / NW), c1 = (int)((int64_t)rounds * (w + 1) / NW);
  const int64_t nb = p.N - n0 < 16 * TN ? p.N - n0 : 16 * TN;
  const __amdgpu_buffer_rsrc_t bc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.b + n0 * krow), (short)0, (int)(nb * krow), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t bs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.bs + n0 * srow), (short)0, (int)(nb * srow), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ac =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.a, (short)0, (int)(p.M * krow), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t as =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.as, (short)0, (int)(p.M * srow), kRsrcWord3);
  uint8_t* const ring = smem + w * (R * SLOT);

  // buffer->LDS load h of a slot moves slot rows 8h .. 8h + 7; lane l fills
  // position l & 7 of row q = 8h + (l >> 3) with global chunk ch[h & 1] of it
  // (the swizzle (q >> 1) & 7 depends on h & 1 only)
  uint32_t ch[2], rowoff[NDMA];
#pragma unroll
  for (int e = 0; e < 2; e++) ch[e] = (uint32_t)((l & 7) ^ ((4 * e + (l >> 4)) & 7));
#pragma unroll
  for (int h = 0; h < NDMA; h++) {
    const int q = 8 * h + (l >> 3);              // slot row
    rowoff[h] = (uint32_t)((h < NB ? q : q - 16 * TN) * krow);   // row within its operand
  }
  // fragment position of step u (0, 1) of a slot in this lane's rows (all
  // fragment rows are 16 apart, so they share the swizzle of row r)
  const uint32_t pos0 = (uint32_t)(16 * (g ^ ((r >> 1) & 7)));
  const uint32_t pos1 = (uint32_t)(16 * ((4 + g) ^ ((r >> 1) & 7)));
  const uint32_t sq = (uint32_t)(r * srow), sq16 = (uint32_t)(16 * srow);
  const int shift = 8 * g;

  v4f acc[TMR][TN];
#pragma unroll
  for (int t = 0; t < TMR; t++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[t][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  v4i bsc[RQ][TN], asc[RQ][TMR];

  // round c into slots 2k, 2k + 1 and scale registers k; rounds past the
  // wave's range read zeros (so their products vanish)
  auto issue = [&](int k, int c) {
    const bool live = c < c1;
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int pair = 2 * c + e;
      uint8_t* sl = ring + (2 * k + e) * SLOT;
#pragma unroll
      for (int h = 0; h < NDMA; h++) {
        const uint32_t chunk = ch[h & 1];
        const bool in = live && 2 * pair + (int)(chunk >> 2) < steps;
        const uint32_t off = rowoff[h] + 16u * chunk + 128u * (uint32_t)pair;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(h < NB ? bc : ac, (lds_void*)(sl + h * 1024), 16,
                                                 in ? off : kOutOfRange, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < TN; j++)
      bsc[k][j] = __builtin_amdgcn_raw_buffer_load_b128(bs, live ? sq + j * sq16 + 16u * (uint32_t)c : kOutOfRange,
                                                        0, 0);
#pragma unroll
    for (int t = 0; t < TMR; t++)
      asc[k][t] = __builtin_amdgcn_raw_buffer_load_b128(as, live ? sq + t * sq16 + 16u * (uint32_t)c : kOutOfRange,
                                                        0, 0);
  };
#pragma unroll
  for (int k = 0; k < RQ; k++) {
    issue(k, c0 + k);
    __builtin_amdgcn_sched_barrier(0);   // round order, as in the loop
  }
  for (int base = c0; base < c1; base += RQ) {
#pragma unroll
    for (int k = 0; k < RQ; k++) {
      const int c = base + k;
      wait_cnt<(RQ - 1) * VM_ROUND, 15>();       // this round's slots have landed
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const uint8_t* sl = ring + (2 * k + (u >> 1)) * SLOT;
        const uint32_t pos = (u & 1) ? pos1 : pos0;
        v4i fb[TN], fa[TMR];
#pragma unroll
        for (int j = 0; j < TN; j++) fb[j] = *(const v4i*)(sl + (16 * j + r) * 128 + pos);
#pragma unroll
        for (int t = 0; t < TMR; t++) fa[t] = *(const v4i*)(sl + (16 * TN + 16 * t + r) * 128 + pos);
        // steps past K: scale byte 0 (their codes are zero), never a NaN byte from the next row
        const bool ok = 4 * c + u < steps;
#pragma unroll
        for (int j = 0; j < TN; j++) {
          const int sb = ok ? (int)((uint32_t)bsc[k][j][u] >> shift) : 0;
          const v8i b8 = __builtin_shufflevector(fb[j], fb[j], 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
          for (int t = 0; t < TMR; t++) {
            const int sa = ok ? (int)((uint32_t)asc[k][t][u] >> shift) : 0;
            const v8i a8 = __builtin_shufflevector(fa[t], fa[t], 0, 1, 2, 3, -1, -1, -1, -1);
            acc[t][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, acc[t][j], 4, 4, 0, sb, 0, sa);
          }
        }
      }
      wait_cnt<63, 0>();                          // the slots' reads are done before they are refilled
      asm volatile("" ::: "memory");
      issue(k, c + RQ);
      // keep the next round's scale shifts behind its own wait (the
      // scheduler would hoist them here, waiting for every load in flight)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_cnt<0, 0>();   // nothing may still write LDS when the workgroup exits

  // wave sums in wave order: ((w0 + w1) + w2) + ..., through the slots once
  // every wave is done reading them
  __syncthreads();
  v4f(*red)[TMR][TN][64] = (v4f(*)[TMR][TN][64])smem;
#pragma unroll
  for (int t = 0; t < TMR; t++)
#pragma unroll
    for (int j = 0; j < TN; j++) red[w][t][j][l] = acc[t][j];
  __syncthreads();
  if (w != 0) return;
  typedef typename std::conditional<OUT == OUT_BF16, __bf16, float>::type T;
#pragma unroll
  for (int t = 0; t < TMR; t++) {
    const int64_t m = 16 * t + r;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < TN; j++) {
      v4f s = red[0][t][j][l];
#pragma unroll
      for (int q = 1; q < NW; q++) s += red[q][t][j][l];
      const int64_t n = n0 + 16 * j + 4 * g;
      T* dst = (T*)p.C + m * p.ldc + n;
      if (n + 4 <= p.N && (((uintptr_t)dst) & (4 * sizeof(T) - 1)) == 0) {
        if constexpr (OUT == OUT_BF16) {
          typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
          *(bf16x4_t*)dst = (bf16x4_t){(__bf16)s[0], (__bf16)s[1], (__bf16)s[2], (__bf16)s[3]};
        } else {
          __builtin_nontemporal_store(s, (v4f*)dst);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; v++)
          if (n + v < p.N) dst[v] = (T)s[v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// NVFP4
// ---------------------------------------------------------------------------
// 8 codes (4 bytes) of one block, exactly dequantized to fp16: hardware
// E2M1 -> fp16 convert, then a packed fp16 multiply by the block's E4M3
// scale (code x scale has at most 6 significant bits and lies in
// [2^-10, 2688]).  (The convert's own f32 scale operand only takes a power
// of two, so it cannot carry an E4M3 scale.)
__device__ __forceinline__ v8h nv_dequant8(uint32_t codes4, v2h s2) {
  v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes4, 1.0f, 0);
  v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes4, 1.0f, 1);
  v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes4, 1.0f, 2);
  v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes4, 1.0f, 3);
  h0 = h0 * s2; h1 = h1 * s2; h2 = h2 * s2; h3 = h3 * s2;
  return (v8h){h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// E4M3 scale byte k of a word -> an fp16 pair (hardware FP8 convert, OCP
// E4M3: 0x7F / 0xFF decode to NaN; every E4M3 value is exact in fp16).
template <int K>
__device__ __forceinline__ v2h e4m3_pair(int word) {
  const _Float16 v = (_Float16)__builtin_amdgcn_cvt_f32_fp8(word, K);
  return (v2h){v, v};
}

// A stage holds 8 NVFP4 blocks per row.  Lane group g owns blocks 4g..4g+3
// (32 contiguous bytes); at step u (0..7) it feeds half (u & 1) of block
// 4g + u/2 to the 32x32x16 fp16 MFMA.  A and B use the same assignment, so
// every step pairs equal contraction indices.
//
// Schedule of a stage: all its code chunks and scale words are read from LDS
// first, step 0's fragments are dequantized, then each step's 16 MFMAs run
// with the next step's dequantization (64 VALU instructions) interleaved one
// MFMA, four VALU: an MFMA keeps the matrix pipe busy for 8 passes while the
// wave issues the independent VALU work behind it.  (Left to itself the
// compiler bunches the conversions ahead of the MFMAs and the two serialize.)
__device__ __forceinline__ void nv_sched_step(bool with_valu) {
#pragma unroll
  for (int q = 0; q < 16; q++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
    if (with_valu) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int OUT>
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
    // the stage's code chunks (half h = blocks 4g + 2h, +1) and the lane's
    // four block scales per row
    v4i ca[2][4], cb[2][4];
    int sa[4], sb[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
      sa[t] = *(const int*)(SA + (ra0 + 32 * t) * 8 + 4 * g);
      sb[t] = *(const int*)(SB + (rb0 + 32 * t) * 8 + 4 * g);
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int t = 0; t < 4; t++) {
        ca[h][t] = *(const v4i*)(A + (ra0 + 32 * t) * ROWB + (h ? offc1 : offc0));
        cb[h][t] = *(const v4i*)(B + (rb0 + 32 * t) * ROWB + (h ? offc1 : offc0));
      }
    v2h fa[4][4], fb[4][4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
      fa[t][0] = e4m3_pair<0>(sa[t]); fa[t][1] = e4m3_pair<1>(sa[t]); fa[t][2] = e4m3_pair<2>(sa[t]); fa[t][3] = e4m3_pair<3>(sa[t]);
      fb[t][0] = e4m3_pair<0>(sb[t]); fb[t][1] = e4m3_pair<1>(sb[t]); fb[t][2] = e4m3_pair<2>(sb[t]); fb[t][3] = e4m3_pair<3>(sb[t]);
    }
    // step u: word u & 3 of half u >> 2, block 2 (u >> 2) + ((u & 3) >> 1)
    v8h af[2][4], bf[2][4];
    auto dequant = [&](int u, v8h (&xa)[4], v8h (&xb)[4]) {
      const int h = u >> 2, wd = u & 3, blk = 2 * h + (wd >> 1);
#pragma unroll
      for (int t = 0; t < 4; t++) {
        xa[t] = nv_dequant8((uint32_t)ca[h][t][wd], fa[t][blk]);
        xb[t] = nv_dequant8((uint32_t)cb[h][t][wd], fb[t][blk]);
      }
    };
    dequant(0, af[0], bf[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; u++) {
      if (u < 7) dequant(u + 1, af[(u + 1) & 1], bf[(u + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[u & 1][i], bf[u & 1][j], acc[i][j], 0, 0, 0);
      nv_sched_step(u < 7);
    }
  });
  float* Cz = p.C + (int64_t)z * p.split_stride;
  // both tensor scales multiply the sum (for split partials too: the factor
  // distributes over the split sum)
  const float mul = p.a_ts[0] * p.b_ts[0];
  store_tile<4, 4, true, OUT>(p, Cz, m0 + wm * 128, n0 + wn * 128, acc, mul);
}

// ---------------------------------------------------------------------------
// Split-K reduction: C = sum over splits, in split order.
// ---------------------------------------------------------------------------
// T = float (fp32 C) or __bf16 (the fp32 sum rounded to nearest even).
// V = 4: four consecutive outputs per thread (N and ldc multiples of 4, C and
// the workspace aligned), 16-byte loads of the partials, up to eight splits'
// loads in flight before they are added (in split order, so the sums are the
// same as one output at a time); V = 1 otherwise.
template <typename T, int V>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ ws, int splits, int64_t M,
                                                            int64_t N, T* __restrict__ C, int64_t ldc) {
  typedef float fv __attribute__((ext_vector_type(V)));
  const int64_t total = M * N, units = total / V;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const int64_t t = u * V;
    fv s = *(const fv*)(ws + t);
    for (int z0 = 1; z0 < splits; z0 += 8) {
      fv v[8];
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (z0 + j < splits) v[j] = *(const fv*)(ws + (int64_t)(z0 + j) * total + t);
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (z0 + j < splits) s += v[j];
    }
    const int64_t m = t / N, n = t - m * N;
    T* dst = C + m * ldc + n;
    if constexpr (V == 1) {
      dst[0] = (T)s[0];
    } else if constexpr (sizeof(T) == 4) {
      *(fv*)dst = s;
    } else {
      typedef T tv __attribute__((ext_vector_type(V)));
      tv o;
#pragma unroll
      for (int j = 0; j < V; j++) o[j] = (T)s[j];
      *(tv*)dst = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Planning and launch
// ---------------------------------------------------------------------------
GemmPlan plan_gemm(int fmt, int64_t M, int64_t N, int64_t K) {
  const bool mx = fmt == FMT_MX;
  GemmPlan pl;
  pl.k_tiles = (K + (mx ? MX_BK : BK) - 1) / (mx ? MX_BK : BK);
  pl.narrow_tm = 0;
  pl.waves8 = 0;
  pl.decode = 0;
  // decode shapes: 16-column workgroups over the whole contraction, when
  // there are enough of them or each one's operand bytes ((M + 16) K / 2) stay
  // small (measured against the narrow kernel: better on every shape with at
  // least 2048 weight rows up to 128 activation rows, and on shorter weights
  // up to ~0.5 MB per workgroup; 128 x 512 x 16384, 1.2 MB per workgroup
  // over 32 workgroups, is 28 % slower)
  if (mx && M <= MXFP4_DECODE_MAX_M &&
      (N >= MXFP4_DECODE_MIN_N || (M + 16) * (K / 2) <= MXFP4_DECODE_WG_BYTES)) {
    pl.decode = (int)((M + 15) / 16);
    pl.splits = 1;
    return pl;
  }
  if (mx && M <= 128) {
    // narrow tiles (32 TM x 256), split along K (in stage pairs) into at most
    // one workgroup per compute unit, each split at least two pairs long
    // (measured on the decode shapes: more, shorter splits pay the prologue
    // latency more often than they gain in parallel streams)
    pl.narrow_tm = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
    const int64_t tiles = (N + 255) / 256, pairs = (pl.k_tiles + 1) / 2;
    int64_t s = 256 / tiles;
    if (s > pairs / 2) s = pairs / 2;
    if (s > 32) s = 32;
    pl.splits = s < 1 ? 1 : (int)s;
    return pl;
  }
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  pl.waves8 = mx && pl.k_tiles <= 4 ? 1 : 0;     // short contractions: the 8-wave kernel (mx8_tile)
  // the MXFP4 kernel splits in pairs of stages (one scale group)
  const int64_t units = mx ? (pl.k_tiles + 1) / 2 : pl.k_tiles;
  const int64_t min_units = mx ? 2 : 4;        // at least 4 stages of 256 / 128 per split
  int splits = 1;
  // fewer output tiles than compute units: split the contraction so that
  // about one wave of workgroups fills the chip ...
  const int64_t cus = 256;
  if (tiles < cus && units >= 2 * min_units) {
    int64_t s = cus / tiles;
    if (s > units / min_units) s = units / min_units;
    if (s > 32) s = 32;
    // ... while the time a split saves, (1 - 1/s) of a tile's contraction at
    // the kernel's measured MFMA rate, exceeds what it adds: the fp32
    // partials written and read back (8 s bytes per output at ~5 TB/s) and the
    // reduction's launch, ~4 us (measured: 8192 x 1024 x 2048 took 46.5 us in
    // two splits and 20.1 us whole, 4096 x 2048 x 4096 53.2 and 30.0 us,
    // 2048 x 1024 x 4096 31.5 in three and 27.8 whole; 1024 x 1024 x 8192
    // 29.7 in eight and 45.1 whole)
    // (unsplit MXFP4 launches of at most half as many tiles as compute units
    // run every tile as two 256 x 128 halves, so they take about half a
    // tile's contraction time)
    const double t_k = (double)K * (mx ? 5.2e-9 : 2.1e-8);
    const double whole = (mx && tiles * 2 <= cus) ? 0.5 : 1.0;
    while (s > 1 && t_k * (whole - 1.0 / (double)s) <= (double)M * (double)N * 8.0 * (double)s / 5.0e12 + 4.0e-6) s--;
    if (s > 1) splits = (int)s;
  }
  pl.splits = splits;
  return pl;
}

// Compute units of the current device (cached per device).
static int compute_units() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Decode launch: one workgroup per 16 TN weight rows.  Two weight tiles per
// workgroup halve the activation bytes each weight byte brings through L2
// when that still leaves at least 256 workgroups; contractions of at most two
// rounds per wave take R = 2 (more workgroups resident, one round in flight
// each), longer ones four slots where they fit in LDS.
template <int TMR, int TN, int R, int OUT>
static void launch_decode_kernel(const GemmArgs& p, hipStream_t stream) {
  static_assert(DecodeShape<TMR, TN, R>::LDS <= 160 * 1024, "LDS");
  const dim3 grid((unsigned)((p.N + 16 * TN - 1) / (16 * TN)));
  hipLaunchKernelGGL((gemm_mx_decode_kernel<TMR, TN, R, OUT>), grid, dim3(64 * MXFP4_DECODE_NW), 0, stream, p);
}

#ifndef MXFP4_DECODE_R11
#define MXFP4_DECODE_R11 4
#endif
template <int TMR, int OUT>
static void launch_decode_tmr(const GemmArgs& p, bool tn2, bool short_k, hipStream_t stream) {
  constexpr int LDS_MAX = 160 * 1024;
  if (tn2) {
    if constexpr (DecodeShape<TMR, 2, 4>::LDS <= LDS_MAX) {
      if (!short_k) return launch_decode_kernel<TMR, 2, 4, OUT>(p, stream);
    }
    launch_decode_kernel<TMR, 2, 2, OUT>(p, stream);
  } else {
    constexpr int RL = TMR == 1 ? MXFP4_DECODE_R11 : 4;
    if constexpr (DecodeShape<TMR, 1, RL>::LDS <= LDS_MAX) {
      if (!short_k) return launch_decode_kernel<TMR, 1, RL, OUT>(p, stream);
    }
    launch_decode_kernel<TMR, 1, 2, OUT>(p, stream);
  }
}

template <int OUT>
static void launch_decode(const GemmArgs& p, const GemmPlan& plan, hipStream_t stream) {
  const int64_t rounds = (p.K / 128 + 3) / 4;
  const bool short_k = rounds <= 2 * MXFP4_DECODE_NW;
  const bool tn2 = p.N >= MXFP4_DECODE_TN2_MIN_N;
  switch (plan.decode) {
    case 1: launch_decode_tmr<1, OUT>(p, tn2, short_k, stream); break;
    case 2: launch_decode_tmr<2, OUT>(p, tn2, short_k, stream); break;
#if MXFP4_DECODE_MAX_M > 32
    case 3: launch_decode_tmr<3, OUT>(p, tn2, short_k, stream); break;
    case 4: launch_decode_tmr<4, OUT>(p, tn2, short_k, stream); break;
#endif
#if MXFP4_DECODE_MAX_M > 64
    case 5: launch_decode_tmr<5, OUT>(p, tn2, short_k, stream); break;
    case 6: launch_decode_tmr<6, OUT>(p, tn2, short_k, stream); break;
    case 7: launch_decode_tmr<7, OUT>(p, tn2, short_k, stream); break;
    case 8: launch_decode_tmr<8, OUT>(p, tn2, short_k, stream); break;
#endif
    default: break;
  }
}

template <int OUT>
static void launch_gemm_kernel(bool nv, const GemmArgs& p, const GemmPlan& plan, int fused_had, dim3 grid,
                               dim3 ngrid, hipStream_t stream) {
  if (nv) {
    if constexpr (OUT != OUT_MXQ) hipLaunchKernelGGL(gemm_nv_kernel<OUT>, grid, dim3(256), 0, stream, p);
  } else if (plan.decode) {
    if constexpr (OUT == OUT_F32 || OUT == OUT_BF16) launch_decode<OUT>(p, plan, stream);
  } else if (plan.narrow_tm && fused_had >= 0) {
    // fused plans have 32-row tiles (fused_plan_ok)
    if (fused_had) hipLaunchKernelGGL((gemm_mx_fused_kernel<1, true, OUT>), ngrid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((gemm_mx_fused_kernel<1, false, OUT>), ngrid, dim3(256), 0, stream, p);
  } else if (plan.narrow_tm == 1) {
    hipLaunchKernelGGL((gemm_mx_narrow_kernel<1, OUT>), ngrid, dim3(256), 0, stream, p);
  } else if (plan.narrow_tm == 2) {
    hipLaunchKernelGGL((gemm_mx_narrow_kernel<2, OUT>), ngrid, dim3(256), 0, stream, p);
  } else if (plan.narrow_tm) {
    hipLaunchKernelGGL((gemm_mx_narrow_kernel<4, OUT>), ngrid, dim3(256), 0, stream, p);
  } else if (plan.waves8) {
    hipLaunchKernelGGL(gemm_mx8_kernel<OUT>, grid, dim3(512), 0, stream, p);
  } else {
    hipLaunchKernelGGL(gemm_mx_kernel<OUT>, grid, dim3(256), 0, stream, p);
  }
}

// C: fp32, or bf16 when c_bf16 (then written by the epilogue, or by the
// split-K reduction from fp32 partials).
static hipError_t launch_gemm_common(bool nv, GemmArgs p, void* C, int64_t ldc, int c_bf16, float* workspace,
                                     const GemmPlan& plan, hipStream_t stream, int fused_had = -1) {
  p.ntm = (int)((p.M + BM - 1) / BM);
  p.ntn = (int)((p.N + BN - 1) / BN);
  p.k_tiles = (int)plan.k_tiles;
  p.splits = plan.splits;
  if (plan.splits > 1) {
    p.C = workspace;
    p.ldc = p.N;
    p.split_stride = p.M * p.N;
  } else {
    p.C = (float*)C;
    p.ldc = ldc;
    p.split_stride = 0;
  }
  p.rem = 0;
  const int64_t tiles = (int64_t)p.ntm * p.ntn;
  if (!nv && plan.splits == 1 && !plan.narrow_tm && !plan.decode) {
    const int64_t cus = compute_units();
    if (tiles > cus && tiles % cus != 0) p.rem = (int)(tiles % cus);
    else if (tiles * 2 <= cus) p.rem = (int)tiles;   // few tiles: every one as two 256 x 128 halves
  }
  dim3 grid((unsigned)(tiles + p.rem), (unsigned)plan.splits);
  dim3 ngrid((unsigned)((p.N + 255) / 256), (unsigned)plan.splits);
  if (plan.splits > 1) launch_gemm_kernel<OUT_PART>(nv, p, plan, fused_had, grid, ngrid, stream);
  else if (p.qcodes) launch_gemm_kernel<OUT_MXQ>(nv, p, plan, fused_had, grid, ngrid, stream);
  else if (c_bf16) launch_gemm_kernel<OUT_BF16>(nv, p, plan, fused_had, grid, ngrid, stream);
  else launch_gemm_kernel<OUT_F32>(nv, p, plan, fused_had, grid, ngrid, stream);
  if (plan.splits > 1) {
    const size_t esz = c_bf16 ? 2 : 4;
    // 16-byte loads with many splits (measured: 16 x 4096 x 14336, 16 splits,
    // 13.7 -> 12.4 us; the wgrads 3072 x 768 x 50432, 7 splits, -2 %); with
    // four or fewer the scalar kernel's four times as many threads hide the
    // load latency better (16 x 14336 x 4096, 4 splits: 11.3 against 11.7 us)
    const bool vec = plan.splits > 4 && p.N % 4 == 0 && ldc % 4 == 0 && (uintptr_t)C % (4 * esz) == 0 &&
                     (uintptr_t)workspace % 16 == 0;
    int64_t work = p.M * p.N / (vec ? 4 : 1);
    int64_t g = (work + 255) / 256;
    if (g > 4096) g = 4096;
    if (c_bf16) {
      if (vec)
        hipLaunchKernelGGL((splitk_reduce_kernel<__bf16, 4>), dim3((unsigned)g), dim3(256), 0, stream, workspace,
                           plan.splits, p.M, p.N, (__bf16*)C, ldc);
      else
        hipLaunchKernelGGL((splitk_reduce_kernel<__bf16, 1>), dim3((unsigned)g), dim3(256), 0, stream, workspace,
                           plan.splits, p.M, p.N, (__bf16*)C, ldc);
    } else {
      if (vec)
        hipLaunchKernelGGL((splitk_reduce_kernel<float, 4>), dim3((unsigned)g), dim3(256), 0, stream, workspace,
                           plan.splits, p.M, p.N, (float*)C, ldc);
      else
        hipLaunchKernelGGL((splitk_reduce_kernel<float, 1>), dim3((unsigned)g), dim3(256), 0, stream, workspace,
                           plan.splits, p.M, p.N, (float*)C, ldc);
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* C, int64_t ldc,
                          int c_bf16, float* workspace, const GemmPlan& plan, hipStream_t stream) {
  GemmArgs p{};
  p.a = a_codes; p.as = a_scales; p.b = b_codes; p.bs = b_scales;
  p.a_ts = nullptr; p.b_ts = nullptr;
  p.M = M; p.N = N; p.K = K;
  return launch_gemm_common(false, p, C, ldc, c_bf16, workspace, plan, stream);
}

hipError_t launch_gemm_mx_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                                   const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, uint8_t* q_codes,
                                   uint8_t* q_scales, int hadamard, const GemmPlan& plan, hipStream_t stream) {
  GemmArgs p{};
  p.a = a_codes; p.as = a_scales; p.b = b_codes; p.bs = b_scales;
  p.a_ts = nullptr; p.b_ts = nullptr;
  p.M = M; p.N = N; p.K = K;
  p.qcodes = q_codes;
  p.qscales = q_scales;
  p.qhad = hadamard;
  return launch_gemm_common(false, p, nullptr, N, 0, nullptr, plan, stream);
}

bool fused_plan_ok(const GemmPlan& plan) {
  // up to 32 activation rows: with more, every column-tile workgroup repeats
  // the quantization of more rows than a separate quantizer pass costs
  // (measured: 64 and 128 rows against 14336 x 4096 and 4096 x 14336 weights
  // ran 15-35 % slower fused than quantize-then-GEMM)
  if (plan.narrow_tm != 1) return false;
  const int64_t pairs = (plan.k_tiles + 1) / 2;
  const int64_t stages = 2 * ((pairs + plan.splits - 1) / plan.splits);   // most stages of one split
  return stages <= 16 / plan.narrow_tm;
}

hipError_t launch_gemm_mx_fused(const uint16_t* x, int64_t ldx, int hadamard, const uint8_t* b_codes,
                                const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* C, int64_t ldc,
                                float* workspace, const GemmPlan& plan, hipStream_t stream) {
  GemmArgs p{};
  p.a = nullptr; p.as = nullptr; p.b = b_codes; p.bs = b_scales;
  p.a_ts = nullptr; p.b_ts = nullptr;
  p.M = M; p.N = N; p.K = K;
  p.x = x;
  p.ldx = ldx;
  p.x_vec = (((uintptr_t)x & 15) == 0 && (ldx % 8) == 0) ? 1 : 0;
  return launch_gemm_common(false, p, C, ldc, 0, workspace, plan, stream, hadamard ? 1 : 0);
}

hipError_t launch_gemm_nv(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                          const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts, int64_t M,
                          int64_t N, int64_t K, void* C, int64_t ldc, int c_bf16, float* workspace,
                          const GemmPlan& plan, hipStream_t stream) {
  GemmArgs p{};
  p.a = a_codes; p.as = a_scales; p.b = b_codes; p.bs = b_scales;
  p.a_ts = a_ts; p.b_ts = b_ts;
  p.M = M; p.N = N; p.K = K;
  return launch_gemm_common(true, p, C, ldc, c_bf16, workspace, plan, stream);
}

}  // namespace mxfp4
