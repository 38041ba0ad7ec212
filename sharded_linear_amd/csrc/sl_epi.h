// Epilogue shared by the GEMM kernels of the linear step (gfx950): results staged through LDS
// so that every global access is 16 bytes per lane along a row.  G is the kernel's argument
// struct; it provides c, ldc, M, N, splits, ws and alpha.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sl_device.h"

namespace sl2 {

// ---- epilogue -------------------------------------------------------------------------------
// The MFMAs take the B fragment as their first operand, so block (i, j) of a wave holds C^T:
// lane l has row 32 i + l%32 of the wave tile, and registers 4q..4q+3 hold its four consecutive
// columns 32 j + 8q + 4(l/32) + 0..3.  Results go through the wave's own LDS region (the operand
// ring is idle by then): lanes write their 4-column pieces, then read back whole 16-byte row
// chunks, so every global access is 16 bytes per lane along a row.  16-byte chunks are
// XOR-swizzled by row, which keeps the row reads and most column-piece writes free of bank
// conflicts.  M-edge rows and N (a multiple of 8) cut only whole chunks, so edge tiles need one
// predicate per chunk.  bf16 results stage the whole wave tile at once; fp32 results go 32 rows
// at a time, with the old main_grad values of the next 32 rows loaded while the current ones
// are staged (or, for wide wave tiles, the current rows' values loaded before their staging).
//
// A row of 6 chunks (48-column bf16 wave tiles) has no whole number of rows per 64 lanes: its
// read-back walks the wave tile's chunks in order instead, and its swizzle flips only bit 0,
// which keeps every chunk index inside the row.
template <int WN, int ROWS, bool ACC>
struct Epi {
  static constexpr int kES = ACC ? 4 : 2;               // bytes per element
  static constexpr int kRowBytes = WN * kES;
  static constexpr int kCPR = kRowBytes / 16;           // 16-byte chunks per row
  static constexpr bool kWhole = 64 % kCPR == 0;        // a wave instruction reads whole rows
  static constexpr int kRPI = kWhole ? 64 / kCPR : 0;   // rows per wave instruction
  static constexpr int kSwz = (kCPR & -kCPR) - 1;       // swizzle bits: kCPR is a multiple of kSwz + 1
  static constexpr int kBytes = ROWS * kRowBytes;       // LDS per wave
  __device__ static __forceinline__ int off(int r, int c) { return r * kRowBytes + ((c ^ (r & kSwz)) << 4); }
};
template <int WM, int WN, bool ACC>
using EpiOf = Epi<WN, ACC ? 32 : WM, ACC>;

template <int WM, int WN, int TM, int TN, bool ACC, class G>
__device__ __forceinline__ void store_tile(const G& g, f32x16 (&acc)[TM][TN], char* smem, int mw, int nw,
                                           int split, int lane, int wave) {
  using E = EpiOf<WM, WN, ACC>;
  static_assert(E::kWhole, "32x32 blocks give wave tiles of whole-row chunks");
  char* ep = smem + wave * E::kBytes;
  const int rl = lane & 31, hl = lane >> 5;
  const int rr = lane / E::kCPR, cr = lane % E::kCPR;    // read-back: row within an instruction, chunk
  const int n = nw + cr * (16 / E::kES);
  if constexpr (!ACC) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(acc[i][j][4 * q + e] * g.alpha);
          *reinterpret_cast<bf16x4*>(ep + E::off(i * 32 + rl, (j * 32 + 8 * q) / 8) + 8 * hl) = v;
        }
    __bf16* C = static_cast<__bf16*>(g.c);
#pragma unroll
    for (int t = 0; t < WM / E::kRPI; ++t) {
      const int r = t * E::kRPI + rr, m = mw + r;
      const uint4 v = *reinterpret_cast<const uint4*>(ep + E::off(r, cr));
      if (m < g.M && n < g.N) *reinterpret_cast<uint4*>(C + int64_t(m) * g.ldc + n) = v;
    }
  } else {
    // Unsplit: the single fp32 read-modify-write of main_grad.  Split-K: this split's partial
    // goes to its own plane ws[split][M][N] with plain stores; the reduce kernel launched next
    // on the stream adds the planes in split order into main_grad.
    constexpr int RI = 32 / E::kRPI;
    const bool direct = g.splits == 1;
    float* C = direct ? static_cast<float*>(g.c) : g.ws + int64_t(split) * g.M * g.N;
    const int64_t ldc = direct ? g.ldc : g.N;
    constexpr int NB = RI <= 8 ? 2 : 1;   // double-buffer the old values when registers allow
    float4 old[NB][RI];
    auto load_old = [&](int i, float4 (&o)[RI]) {
#pragma unroll
      for (int t = 0; t < RI; ++t) {
        const int m = mw + i * 32 + t * E::kRPI + rr;
        o[t] = (m < g.M && n < g.N) ? *reinterpret_cast<const float4*>(C + int64_t(m) * ldc + n)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    if (direct && NB == 2) load_old(0, old[0]);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (NB == 2) {
        if (direct && i + 1 < TM) load_old(i + 1, old[(i + 1) & 1]);
      } else {
        if (direct) load_old(i, old[0]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(ep + E::off(rl, (j * 32 + 8 * q + 4 * hl) / 4)) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
#pragma unroll
      for (int t = 0; t < RI; ++t) {
        const int r = t * E::kRPI + rr, m = mw + i * 32 + r;
        float4 x = *reinterpret_cast<const float4*>(ep + E::off(r, cr));
        if (m < g.M && n < g.N) {
          if (direct) {
            const float4 o = old[i % NB][t];
            x = make_float4(o.x + x.x, o.y + x.y, o.z + x.z, o.w + x.w);
          }
          *reinterpret_cast<float4*>(C + int64_t(m) * ldc + n) = x;
        }
      }
    }
  }
}

// The same epilogue for 16x16 accumulator blocks (v_mfma_f32_16x16x32_bf16, again with the B
// fragment first): lane l holds row 16 i + l%16 of the wave tile and, in its four registers, the
// four consecutive columns 16 j + 4(l/16) + 0..3.  bf16 tiles are staged whole; fp32 tiles go
// through the same 32-row rounds as above, two 16-row blocks per round.
template <int WM, int WN, int TM, int TN, bool ACC, class G>
__device__ __forceinline__ void store_tile16(const G& g, f32x4v (&acc)[TM][TN], char* smem, int mw, int nw,
                                             int split, int lane, int wave) {
  using E = EpiOf<WM, WN, ACC>;
  char* ep = smem + wave * E::kBytes;
  const int rl = lane & 15, gl = lane >> 4;
  const int rr = lane / E::kCPR, cr = lane % E::kCPR;
  const int n = nw + cr * (16 / E::kES);
  if constexpr (!ACC) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(acc[i][j][e] * g.alpha);
        *reinterpret_cast<bf16x4*>(ep + E::off(i * 16 + rl, 2 * j + (gl >> 1)) + 8 * (gl & 1)) = v;
      }
    __bf16* C = static_cast<__bf16*>(g.c);
    if constexpr (E::kWhole) {
#pragma unroll
      for (int t = 0; t < WM / E::kRPI; ++t) {
        const int r = t * E::kRPI + rr, m = mw + r;
        const uint4 v = *reinterpret_cast<const uint4*>(ep + E::off(r, cr));
        if (m < g.M && n < g.N) *reinterpret_cast<uint4*>(C + int64_t(m) * g.ldc + n) = v;
      }
    } else {
      // chunk x = 64 t + lane of the wave tile, row-major: row x / kCPR, chunk x % kCPR
      static_assert(WM * E::kCPR % 64 == 0, "the wave tile's chunks fill whole wave instructions");
#pragma unroll
      for (int t = 0; t < WM * E::kCPR / 64; ++t) {
        const int x = t * 64 + lane, r = x / E::kCPR, c = x % E::kCPR, m = mw + r, nc = nw + c * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(ep + E::off(r, c));
        if (m < g.M && nc < g.N) *reinterpret_cast<uint4*>(C + int64_t(m) * g.ldc + nc) = v;
      }
    }
  } else {
    static_assert(E::kWhole, "fp32 wave tiles of whole-row chunks");
    static_assert(TM % 2 == 0, "two 16-row blocks per round");
    constexpr int RI = 32 / E::kRPI;
    const bool direct = g.splits == 1;
    float* C = direct ? static_cast<float*>(g.c) : g.ws + int64_t(split) * g.M * g.N;
    const int64_t ldc = direct ? g.ldc : g.N;
    constexpr int NB = RI <= 8 ? 2 : 1;
    float4 old[NB][RI];
    auto load_old = [&](int h, float4 (&o)[RI]) {
#pragma unroll
      for (int t = 0; t < RI; ++t) {
        const int m = mw + h * 32 + t * E::kRPI + rr;
        o[t] = (m < g.M && n < g.N) ? *reinterpret_cast<const float4*>(C + int64_t(m) * ldc + n)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    if (direct && NB == 2) load_old(0, old[0]);
#pragma unroll
    for (int h = 0; h < TM / 2; ++h) {
      if constexpr (NB == 2) {
        if (direct && h + 1 < TM / 2) load_old(h + 1, old[(h + 1) & 1]);
      } else {
        if (direct) load_old(h, old[0]);
      }
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const f32x4v a = acc[2 * h + ii][j];
          *reinterpret_cast<float4*>(ep + E::off(ii * 16 + rl, 4 * j + gl)) = make_float4(a[0], a[1], a[2], a[3]);
        }
#pragma unroll
      for (int t = 0; t < RI; ++t) {
        const int r = t * E::kRPI + rr, m = mw + h * 32 + r;
        float4 x = *reinterpret_cast<const float4*>(ep + E::off(r, cr));
        if (m < g.M && n < g.N) {
          if (direct) {
            const float4 o = old[h % NB][t];
            x = make_float4(o.x + x.x, o.y + x.y, o.z + x.z, o.w + x.w);
          }
          *reinterpret_cast<float4*>(C + int64_t(m) * ldc + n) = x;
        }
      }
    }
  }
}

}  // namespace sl2
