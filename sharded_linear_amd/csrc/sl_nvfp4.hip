// NVFP4 weight materialisation for gfx950.
//
// NVIDIA Megatron-Core guide "Generalized Tensor Parallelism", section 1.3 (native NVFP4 param):
// the weight shard is kept as packed 4-bit E2M1 codes with one E4M3 scale per 16 elements and a
// per-tensor fp32 scale.  gfx950's scaled matrix instructions take FP4 data only with E8M0 scales
// per 32 elements, which cannot hold an E4M3 scale's mantissa, so the products run on the bf16
// matrix path instead: this kernel writes W[r][c] = E2M1(code) * E4M3(scale) in bf16.  That
// product has at most six significant bits and lies between 2^-10 and 2688 in magnitude, so it is
// a bf16 value and no rounding happens here; the tensor scale is applied by the GEMM epilogue.
//
// Formats: E2M1 = sign, 2 exponent bits (bias 1), 1 mantissa bit, exponent field 0 giving 0.5 * m
// (values 0, 0.5, 1, 1.5, 2, 3, 4, 6); element 2j of a row sits in the low nibble of byte j.
// E4M3 = sign, 4 exponent bits (bias 7), 3 mantissa bits, exponent field 0 giving m * 2^-9, and
// S.1111.111 the only NaN.
//
// A thread expands 16-element blocks: 8 code bytes and 1 scale byte in, 32 bytes out, so a wave
// reads 512 contiguous code bytes and writes 2 KiB contiguous bf16 per block of each lane.  Each
// thread loads four blocks before it expands any (4.6 % shorter launches than one block at a
// time on the 1B MLP shard's weights).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sl_gemm_f8.h"

namespace {

// bf16 bit pattern of the E2M1 magnitude m (0..7)
__device__ __forceinline__ uint32_t e2m1_mag_bf16(uint32_t m) {
  // exponent field e = m >> 1, mantissa bit m & 1: value (1 + (m & 1) / 2) * 2^(e - 1) for e > 0
  const uint32_t normal = (((m >> 1) + 126u) << 7) | ((m & 1u) << 6);
  return m == 0 ? 0u : m == 1 ? 0x3F00u : normal;             // 0.5 is the one subnormal
}

__device__ __forceinline__ float e4m3_value(uint32_t s) {
  const uint32_t e = (s >> 3) & 15u, m = s & 7u;
  float v = e == 0 ? float(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if ((s & 0x7Fu) == 0x7Fu) v = __builtin_nanf("");
  return (s & 0x80u) ? -v : v;
}

__global__ void __launch_bounds__(256) nvfp4_expand_kernel(const uint2* __restrict__ q,
                                                           const uint8_t* __restrict__ s,
                                                           uint4* __restrict__ w, int64_t blocks) {
  constexpr int U = 4;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t b0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; b0 < blocks; b0 += U * stride) {
    uint2 c[U];
    uint32_t sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b = b0 + u * stride;
      if (b < blocks) {
        c[u] = q[b];
        sb[u] = s[b];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b = b0 + u * stride;
      if (b >= blocks) continue;
      const float sv = e4m3_value(sb[u]);
      uint32_t out[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t byte = ((i < 4 ? c[u].x : c[u].y) >> (8 * (i & 3))) & 0xFFu;
        uint32_t h[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t code = (byte >> (4 * j)) & 0xFu;
          const float v = __uint_as_float(((code & 8u) << 28) | (e2m1_mag_bf16(code & 7u) << 16)) * sv;
          h[j] = __float_as_uint(v) >> 16;                        // exact: v is a bf16 value
        }
        out[i] = h[0] | (h[1] << 16);
      }
      w[2 * b] = make_uint4(out[0], out[1], out[2], out[3]);
      w[2 * b + 1] = make_uint4(out[4], out[5], out[6], out[7]);
    }
  }
}

}  // namespace

int nvfp4_expand(hipStream_t st, const uint8_t* q, const uint8_t* s, void* w, int64_t rows, int64_t cols) {
  const int64_t blocks = rows * (cols / 16);
  if (blocks == 0) return 0;
  int64_t grid = (blocks + 1023) / 1024;        // 256 threads x 4 blocks each
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(nvfp4_expand_kernel, dim3(unsigned(grid)), dim3(256), 0, st, reinterpret_cast<const uint2*>(q),
                     s, static_cast<uint4*>(w), blocks);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
