// Internal interface of the MXFP8 kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

struct F8Args {
  const void* a;        // A codes (E4M3), K-major [M][K]
  const void* b;        // B codes (E4M3), K-major [N][K]
  const void* sa;       // A scales (E8M0) [M][K/32]
  const void* sb;       // B scales (E8M0) [N][K/32]
  void* c;              // bf16 output [M][N]
  int64_t lda, ldb, ldc;
  uint32_t a_bytes, b_bytes, sa_bytes, sb_bytes;
  int M, N, K;          // K a multiple of 128
  int tiles_m, tiles_n;
  int cfg;              // 0: 256x256 (8 waves), 1: 128x128 (4 waves)
};

int f8_fwd(hipStream_t st, F8Args g);
// bf16 out[r][c] = E4M3(codes[r][c]) * 2^(scales[r][c/32] - 127); cols a multiple of 32
int mx_dequant(hipStream_t st, const uint8_t* codes, const uint8_t* scales, void* out, int64_t rows, int64_t cols);
