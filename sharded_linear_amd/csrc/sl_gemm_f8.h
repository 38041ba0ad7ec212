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
  int splits = 1;       // split-K (accumulating kernel): K stages of 128 per split
  int kt_per_split = 0;
  float* ws = nullptr;  // split-K partial planes [splits][M][N]
  float alpha = 1.0f;   // bf16 results are alpha * (A . B^T)
};

// C = A.B^T (bf16 out) over block-scaled fp8 operands.
int f8_fwd(hipStream_t st, F8Args g);
// fp32 C += A.B^T, or with splits > 1 the partial of each split into its plane of ws (the
// caller then adds the planes into C in split order).
int f8_accum(hipStream_t st, F8Args g);
// bf16 out[r][c] = E4M3(codes[r][c]) * 2^(scales[r][c/32] - 127); cols a multiple of 32
int mx_dequant(hipStream_t st, const uint8_t* codes, const uint8_t* scales, void* out, int64_t rows, int64_t cols);

// NVFP4 -> bf16 products E2M1 x E4M3 (exact; the tensor scale is not applied): q [rows][cols/2]
// packed codes, s [rows][cols/16] scales, w [rows][cols] bf16; cols % 16 == 0, q and w 16-aligned.
int nvfp4_expand(hipStream_t st, const uint8_t* q, const uint8_t* s, void* w, int64_t rows, int64_t cols);

// MX quantisation of a bf16 matrix x[R][C] (row-major): rowwise codes qr[R][C] / scales
// sr[R][C/32] (blocks of 32 along C) and/or columnwise codes qc[C][R] / scales sc[C][R/32]
// (blocks of 32 along R, stored transposed).  Null outputs are skipped.  C % 32 == 0 for the
// rowwise copy; R % 32 == 0 and C % 8 == 0 for the columnwise one.
int mx_quantize(hipStream_t st, const void* x, int64_t R, int64_t C, uint8_t* qr, uint8_t* sr, uint8_t* qc,
                uint8_t* sc);
