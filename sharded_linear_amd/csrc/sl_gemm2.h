// Internal interface of the direct-to-LDS bf16 GEMM kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

struct Gemm2Args {
  const void* a;        // A operand storage (bf16)
  const void* b;        // B operand storage (bf16)
  void* c;              // bf16 output, or fp32 main_grad for the accumulating kernel
  int64_t lda, ldb, ldc;
  uint32_t a_bytes, b_bytes;   // operand extents: loads past them return zeros
  int M, N, K;
  int tiles_m, tiles_n;
  int splits, kt_per_split;
  float* ws;            // split-K partial planes [splits][M][N] (accumulating kernel)
  int cfg;              // tile configuration, see gemm2_tile()
  float alpha = 1.0f;   // bf16 results are alpha * (A . B^T), scaled in fp32 before rounding
};

constexpr int kGemm2Configs = 26;
constexpr int kGemm2FwdOnlyConfig = 25;   // 256x192 tiles: forward only

// A K-major (k contiguous) and B K-major: forward.
int gemm2_fwd(hipStream_t st, Gemm2Args g);
// A K-major, B MN-major: dgrad.
int gemm2_dgrad(hipStream_t st, Gemm2Args g);
// A and B MN-major, fp32 accumulate into C: wgrad.
int gemm2_wgrad(hipStream_t st, Gemm2Args g);
// Macro-tile (and k extent of one LDS stage) of configuration cfg.
void gemm2_tile(int cfg, int* bm, int* bn, int* bk);
// Fewest k stages each split must have under configuration cfg.
int gemm2_min_stages(int cfg);
