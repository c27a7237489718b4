// Host-only exercise of the C ABI's argument checks and size queries and of
// the CPU oracle, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (host code only; nothing here launches a kernel or needs a GPU).  Exits 0
// when every status is the documented one; a sanitizer report aborts it.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "mxfp4.h"

extern "C" {
int mxo_quantize(const uint16_t*, int64_t, int64_t, int64_t, int, int, int, int, uint64_t, uint8_t*, uint8_t*,
                 float*);
int mxo_dequantize(int, int64_t, int64_t, const uint8_t*, const uint8_t*, const float*, float*, int64_t);
int mxo_gemm(int, int64_t, const uint8_t*, const uint8_t*, const float*, const uint8_t*, const uint8_t*,
             const float*, const int64_t*, int64_t, const int64_t*, int64_t, double*, double*);
int mxo_quantize_mse(const uint16_t*, int64_t, int64_t, int64_t, int, int, int, int, uint8_t*, uint8_t*, float*);
int mxo_mse_check(const uint16_t*, int64_t, int64_t, int64_t, int, int, int, float, const uint8_t*,
                  const uint8_t*, double, int64_t*);
int mxo_noise_stats(const uint16_t*, int64_t, int64_t, int64_t, int, int, int, const uint8_t*, const uint8_t*,
                    const float*, double*);
}

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);   \
      failures++;                                                      \
    }                                                                  \
  } while (0)

static uint16_t bf16(float f) {
  uint32_t b;
  std::memcpy(&b, &f, 4);
  return (uint16_t)((b + 0x7FFF + ((b >> 16) & 1)) >> 16);
}

static void abi_checks() {
  for (int s = -6; s <= 1; s++) EXPECT(mxfp4_status_string(s) != nullptr);
  size_t cb = 0, sb = 0, ws = 0;
  EXPECT(mxfp4_tensor_bytes(MXFP4_FMT_MX, 4096, 8192, &cb, &sb) == MXFP4_OK && cb == 4096u * 4096u);
  EXPECT(mxfp4_tensor_bytes(MXFP4_FMT_NV, 3, 40, &cb, &sb) == MXFP4_ERR_UNSUPPORTED_SHAPE);
  EXPECT(mxfp4_tensor_bytes(7, 3, 64, &cb, &sb) == MXFP4_ERR_INVALID_ARG);
  EXPECT(mxfp4_tensor_bytes(MXFP4_FMT_MX, -1, 64, &cb, &sb) == MXFP4_ERR_INVALID_ARG);
  EXPECT(mxfp4_quantize_workspace_bytes(MXFP4_FMT_NV, 16384, 12288, 1, &ws) == MXFP4_OK && ws > 0);
  EXPECT(mxfp4_quantize_workspace_bytes(MXFP4_FMT_NV, INT64_C(1) << 20, INT64_C(1) << 20, 0, &ws) == MXFP4_OK);
  // a fake, aligned, never dereferenced device address
  uint8_t* fake = (uint8_t*)(uintptr_t)0x100000;
  mxfp4_tensor a{MXFP4_FMT_MX, 0, 4096, 8192, fake, fake, nullptr};
  mxfp4_tensor b{MXFP4_FMT_MX, 0, 14336, 8192, fake, fake, nullptr};
  mxfp4_tensor n{MXFP4_FMT_NV, 0, 14336, 8192, fake, fake, (float*)fake};
  mxfp4_tensor h{MXFP4_FMT_MX, 1, 14336, 8192, fake, fake, nullptr};
  EXPECT(mxfp4_gemm_workspace_bytes(&a, &b, &ws) == MXFP4_OK);
  EXPECT(mxfp4_gemm_workspace_bytes(&a, &n, &ws) == MXFP4_ERR_FORMAT_MISMATCH);
  EXPECT(mxfp4_gemm(&a, &h, (float*)fake, 14336, nullptr, 0, nullptr) == MXFP4_ERR_FORMAT_MISMATCH);
  mxfp4_tensor odd{MXFP4_FMT_MX, 0, 16, 8224, fake, fake, nullptr};
  EXPECT(mxfp4_gemm(&odd, &odd, (float*)fake, 16, nullptr, 0, nullptr) == MXFP4_ERR_UNSUPPORTED_SHAPE);
  EXPECT(mxfp4_gemm(&a, &b, nullptr, 14336, nullptr, 0, nullptr) == MXFP4_ERR_INVALID_ARG);
  EXPECT(mxfp4_gemm(&a, &b, (float*)fake, 100, nullptr, 0, nullptr) == MXFP4_ERR_INVALID_ARG);
  // a long contraction with few tiles needs a workspace
  mxfp4_tensor w1{MXFP4_FMT_MX, 0, 768, 50432, fake, fake, nullptr};
  mxfp4_tensor w2{MXFP4_FMT_MX, 0, 3072, 50432, fake, fake, nullptr};
  EXPECT(mxfp4_gemm_workspace_bytes(&w1, &w2, &ws) == MXFP4_OK && ws > 0);
  EXPECT(mxfp4_gemm(&w1, &w2, (float*)fake, 3072, nullptr, 0, nullptr) == MXFP4_ERR_WORKSPACE);
  mxfp4_tensor out{MXFP4_FMT_MX, 0, 64, 256, fake, fake, nullptr};
  EXPECT(mxfp4_quantize(nullptr, 64, 256, 256, MXFP4_FMT_MX, MXFP4_RTN, 0, 1, 0, &out, nullptr, 0, nullptr) ==
         MXFP4_ERR_INVALID_ARG);
  EXPECT(mxfp4_quantize((const uint16_t*)fake, 64, 256, 200, MXFP4_FMT_MX, MXFP4_RTN, 0, 1, 0, &out, nullptr, 0,
                        nullptr) == MXFP4_ERR_INVALID_ARG);
  EXPECT(mxfp4_quantize((const uint16_t*)fake, 64, 250, 256, MXFP4_FMT_MX, MXFP4_RTN, 0, 1, 0, &out, nullptr, 0,
                        nullptr) == MXFP4_ERR_UNSUPPORTED_SHAPE);
  EXPECT(mxfp4_quantize((const uint16_t*)fake, 64, 256, 256, MXFP4_FMT_MX, 3, 0, 1, 0, &out, nullptr, 0, nullptr) ==
         MXFP4_ERR_INVALID_ARG);
  mxfp4_tensor nvout{MXFP4_FMT_NV, 0, 64, 256, fake, fake, (float*)fake};
  EXPECT(mxfp4_quantize((const uint16_t*)fake, 64, 256, 256, MXFP4_FMT_NV, MXFP4_SR, 0, 1, 0, &nvout, nullptr, 0,
                        nullptr) == MXFP4_ERR_WORKSPACE);
  EXPECT(mxfp4_quantize_mse_workspace_bytes(MXFP4_FMT_NV, 0, 4096, 4096, 1, &ws) == MXFP4_OK && ws > 0);
  EXPECT(mxfp4_quantize_noise_workspace_bytes(MXFP4_FMT_MX, 0, 50432, 3072, 0, &ws) == MXFP4_OK && ws > 0);
  EXPECT(mxfp4_quantize_gemm_workspace_bytes(16, 4096, 1, &h, &ws) == MXFP4_ERR_FORMAT_MISMATCH);
  double stats[3] = {12.0, 3.0, 0.0}, ratio = 0.0;
  int below = -1;
  EXPECT(mxfp4_noise_ratio(stats, &ratio, &below) == MXFP4_OK && ratio == 2.0 && below == 0);
}

static void oracle_checks() {
  std::mt19937 g(7);
  std::student_t_distribution<float> t(3.0f);
  const int R = 96, C = 128;
  std::vector<uint16_t> x(R * C);
  for (auto& v : x) v = bf16(t(g));
  x[5] = 0x7FC0;   // a NaN block
  for (int fmt = 0; fmt < 2; fmt++)
    for (int had = 0; had < 2; had++)
      for (int axis = 0; axis < 2; axis++)
        for (int rnd = 0; rnd < 2; rnd++) {
          const int rows = axis ? R : C, K = axis ? C : R, bs = fmt ? 16 : 32;
          std::vector<uint8_t> codes(rows * K / 2), scales(rows * K / bs);
          float ts = 0.0f;
          EXPECT(mxo_quantize(x.data(), R, C, C, fmt, rnd, had, axis, 11, codes.data(), scales.data(), &ts) == 0);
          std::vector<float> y(rows * K);
          EXPECT(mxo_dequantize(fmt, rows, K, codes.data(), scales.data(), &ts, y.data(), K) == 0);
          double stats[3];
          EXPECT(mxo_noise_stats(x.data(), R, C, C, fmt, had, axis, codes.data(), scales.data(), &ts, stats) == 0);
          std::vector<int64_t> ri = {0, 3, rows - 1}, cj = {1, rows - 2};
          std::vector<double> Cm(6), Sm(6);
          EXPECT(mxo_gemm(fmt, K, codes.data(), scales.data(), &ts, codes.data(), scales.data(), &ts, ri.data(), 3,
                          cj.data(), 2, Cm.data(), Sm.data()) == 0);
          if (rnd == 0) {
            EXPECT(mxo_quantize_mse(x.data(), R, C, C, fmt, had, axis, 2, codes.data(), scales.data(), &ts) == 0);
            int64_t out[5];
            EXPECT(mxo_mse_check(x.data(), R, C, C, fmt, had, axis, ts, codes.data(), scales.data(), 0.0, out) == 0);
            EXPECT(out[1] == 0 && out[2] == 0);
          }
        }
  // rejected arguments
  uint8_t c1[16], s1[1];
  EXPECT(mxo_quantize(x.data(), 2, 30, 30, 0, 0, 0, 1, 0, c1, s1, nullptr) == -1);
}

int main() {
  abi_checks();
  oracle_checks();
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer run: all checks passed\n");
  return 0;
}
