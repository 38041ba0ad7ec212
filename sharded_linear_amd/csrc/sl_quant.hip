// MX quantisation of bf16 matrices for the all-MXFP8 step (gfx950).
//
// NVIDIA Megatron-Core guide "Generalized Tensor Parallelism", section 1.3: in the MXFP8 recipe
// every GEMM of the step -- forward, dgrad and wgrad -- reads E4M3 elements with one E8M0 scale
// per 32 elements along its own contraction axis, so a tensor consumed along both of its axes
// (X, W, dY) is quantised twice: rowwise (blocks along the last axis) and columnwise (blocks down
// the columns, stored transposed so that the consuming GEMM again reads k contiguously).  The
// pages fix the block of 32 and the per-block scale; the conversion rule is the OCP MX v1.0 one:
//   X = clamp(floor(log2 amax) - 8, -127, 127)   (8 = the largest E4M3 exponent), stored X + 127
//   code(x) = E4M3 round-to-nearest-even of x / 2^X, saturating at +-448, sign kept
//   an all-zero block stores scale 0 and zero codes.
// The codes come from v_cvt_scalef32_pk_fp8_bf16, which divides two bf16 elements by an fp32
// scale and rounds to E4M3, nearest-even, in one instruction.  Measured over every bf16 pattern
// against the rule above (scales 2^-126 .. 2^100): identical, except that a quotient rounding past
// 448 gives the NaN code S.1111.111 instead of saturating; those bytes are rewritten to S.1111.110
// (448), the only change needed (E4M3 has no other NaN pattern).  A block whose shared exponent is
// -127 (2^-127 is not a normal fp32 scale) takes a bit-field path instead: x times the exact fp32
// power of two 2^127, rounded on the fp32 bit fields.  The GPU tests check every bf16 pattern.
//
// One workgroup quantises a 128 x 128 tile.  Each thread loads eight 16-byte chunks, 16 adjacent
// lanes covering the 256 bytes of a tile row, so a quad of lanes holds one 32-element row block:
// for the rowwise copy the quad shares the block's amax through two DPP quad permutes and each lane
// stores the 8 codes of its chunk.  For the columnwise copy the tile is staged in LDS, from which
// each thread reads two 32-row column blocks; their codes go back into the same LDS (a column's
// four blocks make one 128-byte line of the transposed output, 16-byte chunks XOR-swizzled by the
// column against bank conflicts) and leave as whole lines, eight lanes to a line, with each
// column's four scales as one dword.  Storing each column block straight from its thread (32 bytes
// at a stride of R between lanes) cost about a fifth of the kernel's time on [8192, 8192].
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sl_device.h"
#include "sl_gemm_f8.h"

namespace sl2 {

// E4M3 code of v (finite, |v| < 512): the fp32 mantissa rounded to 3 bits, nearest-even, for
// |v| >= 2^-6; a fixed step of 2^-9, nearest-even, below (code 8 is 2^-6 itself); 448 caps.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t ab = b & 0x7FFFFFFFu;
  uint32_t code;
  if (ab >= 0x3C800000u) {                                     // 2^-6
    uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) & 0xFFF00000u;
    if (r > 0x43E00000u) r = 0x43E00000u;                      // 448
    code = ((((r >> 23) & 0xFFu) - 120u) << 3) | ((r >> 20) & 7u);   // biased exponent 127 -> 7
  } else {
    code = uint32_t(__builtin_rintf(__uint_as_float(ab) * 512.0f));
  }
  return code | ((b >> 24) & 0x80u);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4q __attribute__((ext_vector_type(4)));

// Largest magnitude field of N words of two bf16 elements: |bf16| orders like its 15-bit magnitude.
// Both halves are compared at once (packed 16-bit max).
template <int N>
__device__ __forceinline__ uint32_t mag_max(const uint32_t (&w)[N]) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < N; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  return m[0] > m[1] ? m[0] : m[1];
}

// Encodes N words of two bf16 elements (element 2i in the low half of word i) of a block whose
// amax has the bf16 bits `amax`: returns the biased scale and packs the codes into q[N / 2] (code of
// element e in byte e).
template <int N>
__device__ __forceinline__ uint32_t mx_encode(const uint32_t (&w)[N], uint32_t amax, uint32_t (&q)[N / 2]) {
  if (amax == 0) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) q[i] = 0;
    return 0;
  }
  int X = int((amax >> 7) & 0xFFu) - 127 - 8;          // floor(log2 amax) - 8 (bf16 exponent field)
  X = X < -127 ? -127 : X > 127 ? 127 : X;
  if (X > -127) {
    const float scale = __uint_as_float(uint32_t(X + 127) << 23);
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16((s16x2){0, 0}, __builtin_bit_cast(bf16x2, w[2 * i]), scale, false);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, w[2 * i + 1]), scale, true);
      uint32_t c = __builtin_bit_cast(uint32_t, r);
      // quotients that rounded past 448 came back as the NaN code x.1111.111: saturate to x.1111.110
      const uint32_t nan = ((c & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
      q[i] = c - (nan >> 7);
    }
  } else {
    const float mult = __uint_as_float(0x7F000000u);     // 2^127, exact
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t h = w[2 * i + e / 2];
        const float x = __uint_as_float((e & 1) ? (h & 0xFFFF0000u) : (h << 16));
        word |= e4m3_code(x * mult) << (8 * e);
      }
      q[i] = word;
    }
  }
  return uint32_t(X + 127);
}

// One block of 32 elements held by one thread.
__device__ __forceinline__ uint32_t mx_block(const uint32_t (&w)[16], uint32_t (&q)[8]) {
  return mx_encode(w, mag_max(w), q);
}

// Largest value of m over the four lanes of a quad (DPP quad permutes [1,0,3,2] and [2,3,0,1]).
__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  uint32_t o = uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0xB1, 0xF, 0xF, false));
  m = o > m ? o : m;
  o = uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0x4E, 0xF, 0xF, false));
  return o > m ? o : m;
}

constexpr int kQT = 128;                 // tile edge
// LDS row stride (bf16 elements): 288 bytes, so the 4 rows x 4 column quads that one 16-lane group
// of a transposing read touches fall in distinct banks
constexpr int kQStride = kQT + 16;

template <bool ROWS, bool COLS>
__global__ void __launch_bounds__(256) mx_quant_tile(const uint16_t* x, int64_t R, int64_t C, uint8_t* qr, uint8_t* sr,
                                                      uint8_t* qc, uint8_t* sc) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[COLS ? kQT * kQStride : 1];
  // After the columnwise blocks are encoded, the same LDS holds their codes, one 128-byte line per
  // column (its run in q_cols), and the scales after them, so that each line leaves as 8 adjacent
  // 16-byte stores and each column's scales as one group.
  uint8_t* const qbuf = reinterpret_cast<uint8_t*>(tile);
  uint8_t* const sbuf = qbuf + kQT * kQT;
  // one-dimensional grid (row tiles can outnumber grid.y's 65535), column tile fastest
  const int64_t ntc = (C + kQT - 1) / kQT;
  const int64_t r0 = int64_t(blockIdx.x) / ntc * kQT, c0 = int64_t(blockIdx.x) % ntc * kQT;
  const int t = threadIdx.x, ch = t & 15;       // 16-byte chunk of a tile row; a quad holds one block
  uint4 raw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {                    // 8-element chunks (C % 8 == 0): all or nothing
    const int64_t gr = r0 + (t >> 4) + 16 * k, gc = c0 + 8 * ch;
    raw[k] = (gr < R && gc + 8 <= C) ? *reinterpret_cast<const uint4*>(x + gr * C + gc) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = (t >> 4) + 16 * k;
    const int64_t gr = r0 + row, gc = c0 + 8 * ch;
    if constexpr (COLS) reinterpret_cast<uint4*>(tile + row * kQStride)[ch] = raw[k];
    if constexpr (ROWS) {
      const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
      const uint32_t amax = quad_max(mag_max(w));  // every lane takes part; out-of-range chunks are 0
      uint32_t q[2];
      const uint32_t s = mx_encode(w, amax, q);
      if (gr < R && gc < C) {                      // rowwise copies: C % 32 == 0, whole blocks
        *reinterpret_cast<uint2*>(qr + gr * C + gc) = make_uint2(q[0], q[1]);
        if ((ch & 3) == 0) sr[gr * (C / 32) + gc / 32] = uint8_t(s);
      }
    }
  }
  if constexpr (COLS) {
    __syncthreads();
    uint32_t q[2][8], s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int idx = t + 256 * h, rb = idx >> 7;
      // Thread idx holds column idx % 128 (a wave: 64 adjacent columns), rows 32 rb .. 32 rb + 31.
      // ds_read_b64_tr_b16 transposes 4 x 4 blocks of 16-bit values within each 16-lane group:
      // source lane 4j + q reads 4 adjacent columns (quad q of the group's 16) of row j, and result
      // lane 4q + e receives element e of those four rows -- its own column, 4 adjacent rows,
      // packed two to a word as v expects.  Eight reads cover the 32-row block.
      const int s16 = t & 15, jr = s16 >> 2, qc4 = s16 & 3;
      const int col4 = ((idx & (kQT - 1)) & ~15) + 4 * qc4;
      const uint32_t a0 = uint32_t(reinterpret_cast<uintptr_t>(
          (const __attribute__((address_space(3))) uint16_t*)(tile + (rb * 32 + jr) * kQStride + col4)));
      uint32_t v[16];
#pragma unroll
      for (int r4 = 0; r4 < 8; ++r4) {
        const i16x4q x4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4q*)(uintptr_t)(a0 + r4 * 4 * kQStride * 2));
        const uint2 p = __builtin_bit_cast(uint2, x4);
        v[2 * r4] = p.x;
        v[2 * r4 + 1] = p.y;
      }
      s[h] = mx_block(v, q[h]);                  // blocks past the edges are encoded and never stored
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int idx = t + 256 * h, col = idx & (kQT - 1), rb = idx >> 7;
      uint8_t* line = qbuf + col * kQT;          // 16-byte chunk c of the line sits in slot c ^ (col & 7)
      *reinterpret_cast<uint4*>(line + ((2 * rb) ^ (col & 7)) * 16) = make_uint4(q[h][0], q[h][1], q[h][2], q[h][3]);
      *reinterpret_cast<uint4*>(line + ((2 * rb + 1) ^ (col & 7)) * 16) = make_uint4(q[h][4], q[h][5], q[h][6], q[h][7]);
      sbuf[col * 4 + rb] = uint8_t(s[h]);
    }
    __syncthreads();
    // Column c of the tile is line c0 + c of q_cols, bytes [r0, r0 + 128) (fewer at the R edge,
    // whole 32-row blocks since R % 32 == 0): lanes 8c' .. 8c'+7 of a pass store its 16-byte chunks.
    const int nrb = int(R - r0 < kQT ? (R - r0) / 32 : 4);       // row blocks of this tile
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = t + 256 * p, col = idx >> 3, ch = idx & 7;
      const int64_t gc = c0 + col;
      if (gc < C && ch < 2 * nrb)
        *reinterpret_cast<uint4*>(qc + gc * R + r0 + ch * 16) = *reinterpret_cast<const uint4*>(qbuf + col * kQT + (ch ^ (col & 7)) * 16);
    }
    if (t < kQT && c0 + t < C) {
      uint8_t* d = sc + (c0 + t) * (R / 32) + r0 / 32;
      if (nrb == 4 && (reinterpret_cast<uintptr_t>(d) & 3) == 0) *reinterpret_cast<uint32_t*>(d) = *reinterpret_cast<const uint32_t*>(sbuf + t * 4);
      else for (int b = 0; b < nrb; ++b) d[b] = sbuf[t * 4 + b];
    }
  }
}

}  // namespace sl2

int mx_quantize(hipStream_t st, const void* x, int64_t R, int64_t C, uint8_t* qr, uint8_t* sr, uint8_t* qc,
                uint8_t* sc) {
  if (R == 0 || C == 0 || (!qr && !qc)) return 0;
  const dim3 grid(unsigned(((C + sl2::kQT - 1) / sl2::kQT) * ((R + sl2::kQT - 1) / sl2::kQT)));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (qr && qc) hipLaunchKernelGGL((sl2::mx_quant_tile<true, true>), grid, dim3(256), 0, st, xp, R, C, qr, sr, qc, sc);
  else if (qr) hipLaunchKernelGGL((sl2::mx_quant_tile<true, false>), grid, dim3(256), 0, st, xp, R, C, qr, sr, qc, sc);
  else hipLaunchKernelGGL((sl2::mx_quant_tile<false, true>), grid, dim3(256), 0, st, xp, R, C, qr, sr, qc, sc);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
