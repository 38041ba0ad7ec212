// MXFP8 operand kernels of the linear step (gfx950).
//
// NVIDIA Megatron-Core guide "Generalized Tensor Parallelism", section 1.3: weights (and here
// activations) travel as E4M3 elements with one E8M0 scale per 32 elements along `in`.
//
//  * fwd Y = deq(Xq) . deq(Wq)^T: both operands are blocked along the contraction axis, so the
//    block-scaled fp8 MFMA v_mfma_scale_f32_32x32x64_f8f6f4 consumes the codes and scales
//    directly.  Its operand layout (checked on the hardware): for a 64-wide k step, lane l of a
//    32-row fragment holds row l%32; lane group g = l/32 carries elements [16g, 16g+16) in
//    bytes 0..15 and [32+16g, 32+16g+16) in bytes 16..31, and the scale supplied by the lane of
//    row m in group g multiplies the 32-element block g of that row.  So each lane loads the two
//    16-byte chunks 16g and 32+16g of the k step and the scale of block (k0/32 + g).
//    Codes travel HBM->LDS directly (buffer_load ... lds, rows of 128 bytes, swizzled like the
//    bf16 tiles); block scales come with each stage (one dword of 4 per row) or, where K % 512 ==
//    0, four stages at a time into a scale cache.  The MFMAs take the B fragment (with its
//    scales) first, so the accumulators hold C^T blocks as in the bf16 kernels, and both the bf16
//    result and the fp32 read-modify-write of main_grad go through the same LDS-staged epilogue
//    (16-byte row accesses; for the bf16 result 1 % ahead on the all-MXFP8 step of direct
//    two-byte stores from the accumulator layout).
//  * dgrad / wgrad see the MXFP8 operand blocked along their N, not K; it is dequantised
//    exactly into a bf16 workspace by mx_dequant_bf16 (an E4M3 value times a power of two has
//    at most 4 significant bits) and the bf16 GEMM kernels run on it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sl_device.h"
#include "sl_epi.h"
#include "sl_gemm_f8.h"

namespace sl2 {

constexpr int kF8RowBytes = 128;      // fp8 k elements per LDS row per stage
constexpr int kF8CPR = kF8RowBytes / 16;

__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int R>
struct F8Tile {
  static constexpr int kBytes = R * kF8RowBytes;
  static constexpr int kLoads = kBytes / 1024;
  static constexpr int kScaleBytes = R * 4;
  static constexpr int kScaleLoads = (kScaleBytes + 255) / 256;

  template <int WAVES>
  static constexpr int kScaleLoadsPerWave = (kScaleLoads + WAVES - 1) / WAVES;

  // Every wave issues kLoads/WAVES code loads and kScaleLoadsPerWave scale loads, so per-wave
  // vmcnt arithmetic is uniform; surplus scale loads read out of range into `pad` (zeros).
  template <int WAVES>
  __device__ static __forceinline__ void load(i32x4 rs, i32x4 rss, char* lds, char* lds_s, char* pad, int lane,
                                              int wave, int row0, int rows, int k0, int K, int64_t ld) {
#pragma unroll
    for (int it = 0; it < kLoads / WAVES; ++it) {
      const int wl = it * WAVES + wave;
      const int p = wl * 64 + lane;
      const int r = p / kF8CPR, c = (p % kF8CPR) ^ swz128(p / kF8CPR);
      const int gr = row0 + r, k = k0 + c * 16;
      const uint32_t off = (gr < rows && k < K) ? uint32_t(int64_t(gr) * ld + k) : kOOB;
      lds_dma16(rs, lds_addr(lds + wl * 1024), off);
    }
    // scale dwords: row r holds the E8M0 scales of blocks k0/32 .. k0/32+3
    const int nb = K / 32;
#pragma unroll
    for (int it = 0; it < kScaleLoadsPerWave<WAVES>; ++it) {
      const int wl = it * WAVES + wave;
      if (wl < kScaleLoads) {
        const int r = wl * 64 + lane;
        const int gr = row0 + r, b = k0 / 32;
        const uint32_t off = (r < R && gr < rows && b < nb) ? uint32_t(int64_t(gr) * nb + b) : kOOB;
        lds_dma4(rss, lds_addr(lds_s + wl * 256), off);
      } else {
        lds_dma4(rss, lds_addr(pad), kOOB);
      }
    }
  }
  // The code loads of load() alone (the kernels that cache their scales by groups).
  template <int WAVES>
  __device__ static __forceinline__ void load_codes(i32x4 rs, char* lds, int lane, int wave, int row0, int rows,
                                                    int k0, int K, int64_t ld) {
#pragma unroll
    for (int it = 0; it < kLoads / WAVES; ++it) {
      const int wl = it * WAVES + wave;
      const int p = wl * 64 + lane;
      const int r = p / kF8CPR, c = (p % kF8CPR) ^ swz128(p / kF8CPR);
      const int gr = row0 + r, k = k0 + c * 16;
      const uint32_t off = (gr < rows && k < K) ? uint32_t(int64_t(gr) * ld + k) : kOOB;
      lds_dma16(rs, lds_addr(lds + wl * 1024), off);
    }
  }
  // Scale group G: the E8M0 scales of blocks 16G .. 16G+15 (stages 4G .. 4G+3), 16 bytes per
  // row, row r at LDS byte 16 r.  Wave-load q covers rows 64q .. 64q+63, one 16-byte lane each;
  // the row's bytes are contiguous and 16-byte aligned in HBM when K % 512 == 0 and the scale
  // array is 16-byte aligned.
  static constexpr int kGroupBytes = R * 16;
  static constexpr int kGroupLoads = R / 64;
  __device__ static __forceinline__ void load_group(i32x4 rss, char* lds_s, int q, int lane, int row0, int rows, int G,
                                                    int K) {
    const int gr = row0 + q * 64 + lane, nb = K / 32, b = 16 * G;
    const uint32_t off = (gr < rows && b < nb) ? uint32_t(int64_t(gr) * nb + b) : kOOB;
    lds_dma16(rss, lds_addr(lds_s + q * 1024), off);
  }
  // 32 bytes of fragment row r0 + l%32 for k64 step ks: chunks 4ks+g and 4ks+2+g
  __device__ static __forceinline__ i32x8 frag(const char* lds, int r0, int ks, int lane) {
    const int r = r0 + (lane & 31), g = lane >> 5;
    const char* row = lds + r * kF8RowBytes;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + (((4 * ks + g) ^ swz128(r)) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + (((4 * ks + 2 + g) ^ swz128(r)) << 4));
    i32x8 v;
    v[0] = int(lo.x); v[1] = int(lo.y); v[2] = int(lo.z); v[3] = int(lo.w);
    v[4] = int(hi.x); v[5] = int(hi.y); v[6] = int(hi.z); v[7] = int(hi.w);
    return v;
  }
  __device__ static __forceinline__ uint32_t scales(const char* lds_s, int r0, int lane) {
    return *reinterpret_cast<const uint32_t*>(lds_s + (r0 + (lane & 31)) * 4);
  }
};

// Block scales, two ways.  SC false: each stage carries one dword of 4 scales per row, loaded
// with the stage (a 4-byte gather per row at the scale array's row stride).  SC true: the scales
// of four stages are loaded at once, 16 bytes per row, into a double-buffered group cache after
// the operand ring; group G + 1 is loaded at the first stage of group G, into the buffer group
// G - 1 has finished with, and before that stage's code loads, so the per-stage vmcnt waits
// (which count code loads only) cover it.  That needs a quarter of the scale loads and of the
// cache lines they touch.
template <int BM, int BN, int S, int WGM, int WGN, bool ACC, bool SC>
struct F8Layout {
  using TA = F8Tile<BM>;
  using TB = F8Tile<BN>;
  static constexpr int WAVES = WGM * WGN;
  // SC false, stage layout: A codes | B codes | A scale dwords | B scale dwords | 256-byte pad
  static constexpr int kScaleOff = TA::kBytes + TB::kBytes;
  static constexpr int kPadOff = kScaleOff + ((TA::kScaleBytes + TB::kScaleBytes + 255) / 256) * 256;
  static constexpr int kStage = SC ? TA::kBytes + TB::kBytes : kPadOff + 256;
  // SC true: group cache [2 buffers][A rows | B rows][16 bytes] after the S stages
  static constexpr int kCacheOff = S * kStage;
  static constexpr int kGroupBytes = TA::kGroupBytes + TB::kGroupBytes;
  static constexpr int kGroupLoads = TA::kGroupLoads + TB::kGroupLoads;
  static constexpr int kRing = kCacheOff + (SC ? 2 * kGroupBytes : 0);
  static constexpr int kEpi = WAVES * EpiOf<BM / WGM, BN / WGN, ACC>::kBytes;
  static constexpr int kLds = kRing > kEpi ? kRing : kEpi;
  static_assert(kLds <= 160 * 1024, "LDS");
};

template <int BM, int BN, int S, int WGM, int WGN, bool ACC, bool SC>
__global__ void __launch_bounds__(WGM * WGN * 64) gemm_f8fwd(F8Args g) {
  using L = F8Layout<BM, BN, S, WGM, WGN, ACC, SC>;
  constexpr int WAVES = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 32, TN = WN / 32;
  using TA = F8Tile<BM>;
  using TB = F8Tile<BN>;
  constexpr int kScaleOff = L::kScaleOff, kPadOff = L::kPadOff, kStage = L::kStage;
  static_assert(TA::kLoads % WAVES == 0 && TB::kLoads % WAVES == 0, "loads per wave");
  constexpr int kLoadsPerWave = (TA::kLoads + TB::kLoads) / WAVES +
                                (SC ? 0 : TA::template kScaleLoadsPerWave<WAVES> + TB::template kScaleLoadsPerWave<WAVES>);
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  const int ntiles = g.tiles_m * g.tiles_n;
  const int t = xcd_remap(blockIdx.x, ntiles);
  const int group = t / (8 * g.tiles_n);
  const int first_m = group * 8;
  const int gsz = min(g.tiles_m - first_m, 8);
  const int tm = first_m + (t % (8 * g.tiles_n)) % gsz;
  const int tn = (t % (8 * g.tiles_n)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;
  const int split = blockIdx.z;
  const int nkt = (g.K + kF8RowBytes - 1) / kF8RowBytes;
  const int kt0 = ACC ? split * g.kt_per_split : 0;
  const int nk = ACC ? min(nkt, kt0 + g.kt_per_split) - kt0 : nkt;

  const i32x4 ra = rsrc(g.a, g.a_bytes), rb = rsrc(g.b, g.b_bytes);
  const i32x4 rsa = rsrc(g.sa, g.sa_bytes), rsb = rsrc(g.sb, g.sb_bytes);

  // A stage's loads go out in two halves, A's at the top of the stage (right after the barrier
  // that frees its slot) and B's after the stage's first row of MFMAs.
  auto issue = [&](int kt, int slot) {
    char* base = smem + slot * kStage;
    const int k0 = kt * kF8RowBytes;
    if constexpr (SC) {
      TA::template load_codes<WAVES>(ra, base, lane, wave, m0, g.M, k0, g.K, g.lda);
    } else {
      char* sbase = base + kScaleOff;
      TA::template load<WAVES>(ra, rsa, base, sbase, base + kPadOff, lane, wave, m0, g.M, k0, g.K, g.lda);
    }
  };
  auto issue_b = [&](int kt, int slot) {
    char* base = smem + slot * kStage;
    const int k0 = kt * kF8RowBytes;
    if constexpr (SC) {
      TB::template load_codes<WAVES>(rb, base + TA::kBytes, lane, wave, n0, g.N, k0, g.K, g.ldb);
    } else {
      char* sbase = base + kScaleOff;
      TB::template load<WAVES>(rb, rsb, base + TA::kBytes, sbase + TA::kScaleBytes, base + kPadOff, lane, wave, n0,
                               g.N, k0, g.K, g.ldb);
    }
  };
  // scale group G into cache buffer G % 2: wave w issues the group's wave-loads w, w + WAVES, ...
  auto issue_group = [&](int G) {
    if constexpr (SC) {
      char* cb = smem + L::kCacheOff + (G & 1) * L::kGroupBytes;
#pragma unroll
      for (int q0 = 0; q0 < L::kGroupLoads; q0 += WAVES) {
        const int q = q0 + wave;
        if (q < TA::kGroupLoads) TA::load_group(rsa, cb, q, lane, m0, g.M, G, g.K);
        else if (q < L::kGroupLoads) TB::load_group(rsb, cb + TA::kGroupBytes, q - TA::kGroupLoads, lane, n0, g.N, G, g.K);
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // the scale groups of the first two groups go out before any code load
  issue_group(kt0 / 4);
  issue_group(kt0 / 4 + 1);
#pragma unroll
  for (int s = 0; s < S - 1; ++s) { issue(kt0 + (s < nk ? s : nk), s); issue_b(kt0 + (s < nk ? s : nk), s); }

  for (int it = 0; it < nk; ++it) {
    wait_vmcnt<(S - 2) * kLoadsPerWave>();
    __syncthreads();
    const int kt = kt0 + it;
    if (SC && it > 0 && kt % 4 == 0) issue_group(kt / 4 + 1);
    {
      const int nxt = it + S - 1;
      issue(kt0 + (nxt < nk ? nxt : nk), nxt % S);
    }
    const char* la = smem + (it % S) * kStage;
    const char* lb = la + TA::kBytes;
    uint32_t sca[TM], scb[TN];
    if constexpr (SC) {
      // dword kt % 4 of each row's 16 bytes in buffer (kt / 4) % 2
      const char* cb = smem + L::kCacheOff + ((kt / 4) & 1) * L::kGroupBytes + (kt % 4) * 4;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        sca[i] = *reinterpret_cast<const uint32_t*>(cb + (wm * WM + i * 32 + (lane & 31)) * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        scb[j] = *reinterpret_cast<const uint32_t*>(cb + TA::kGroupBytes + (wn * WN + j * 32 + (lane & 31)) * 16);
    } else {
      const char* lsa = la + kScaleOff;
      const char* lsb = lsa + TA::kScaleBytes;
#pragma unroll
      for (int i = 0; i < TM; ++i) sca[i] = TA::scales(lsa, wm * WM + i * 32, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) scb[j] = TB::scales(lsb, wn * WN + j * 32, lane);
    }
    // The stage's two k64 steps as 2 TM rows u = ks * TM + i of TN MFMAs each, in a fixed order:
    // row u runs while A fragment u + 2 is read (and, two rows before step 1, step 1's B
    // fragments), so a wave waits on LDS once per stage, for the first rows' fragments, instead of
    // before nearly every row as the compiler's own order did (it kept one A fragment live).  B's
    // code loads for the stage S - 1 ahead go out after row 0.  Against the previous order this
    // measured 0.5-1.0 % ahead on the all-MXFP8 step; with it, A's loads moved after row 0 lost
    // 3.7 % and B's at the top tied.  Every accumulator still takes its k steps in order.
    constexpr int NU = 2 * TM;
    static_assert(TM >= 2, "rows per k64 step");
    i32x8 fa[NU], fb[2][TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = TB::frag(lb, wn * WN + j * 32, 0, lane);
    fa[0] = TA::frag(la, wm * WM, 0, lane);
    fa[1] = TA::frag(la, wm * WM + 32, 0, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int ks = u / TM, i = u % TM;
      const int sh = 8 * (2 * ks + (lane >> 5));
      // odd rows run j backwards, so every MFMA shares an operand with the one before it
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) {
        const int j = (u & 1) ? TN - 1 - jj : jj;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fb[ks][j], fa[u], acc[i][j], 0, 0, 0, int((scb[j] >> sh) & 0xFFu), 0, int((sca[i] >> sh) & 0xFFu));
      }
      if (u + 2 < NU) {
        const int v = u + 2;
        if (v == TM) {
#pragma unroll
          for (int j = 0; j < TN; ++j) fb[1][j] = TB::frag(lb, wn * WN + j * 32, 1, lane);
        }
        fa[v] = TA::frag(la, wm * WM + (v % TM) * 32, v / TM, lane);
      }
      if (u == 0) {
        const int nxt = it + S - 1;
        issue_b(kt0 + (nxt < nk ? nxt : nk), nxt % S);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();    // every wave is past its last operand read: the stage ring becomes epilogue space
  store_tile<WM, WN, TM, TN, ACC>(g, acc, smem, m0 + wm * WM, n0 + wn * WN, split, lane, wave);
}


// bf16 out[r][c] = E4M3(codes[r][c]) * 2^(scales[r][c/32] - 127).  Rows hold whole 32-element
// blocks and the scales one byte per block in the same order, so the arrays are linear in the
// block index: 8-element chunk i is codes[8i, 8i+8), scale byte i/4 and out[8i, 8i+8), with no
// row or column arithmetic.  A lane's chunk leaves as one 16-byte store, so every store
// instruction of a wave covers 1 KiB contiguously (0.6-0.9 % ahead on the MXFP8-operand step of
// 16-element chunks stored as two halves 32 bytes apart).  Each thread keeps four chunks in
// flight (the kernel is bound by HBM bytes, 3 per element).  The product is formed by
// v_cvt_scalef32_pk_bf16_fp8 with the scale as an fp32 power of two; it is exact whenever the
// result is a normal bf16, which the entry points require.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  if (s == 0xFFu) return __builtin_bit_cast(float, 0x7FC00000u);             // NaN scale
  return s ? __builtin_bit_cast(float, s << 23) : __builtin_bit_cast(float, 0x00400000u);  // 2^-127
}

__global__ void __launch_bounds__(256) mx_dequant_bf16(const uint2* codes, const uint8_t* scales, uint4* out,
                                                       int64_t n8) {
  constexpr int U = 4;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t base = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; base < n8; base += U * stride) {
    uint2 q[U];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * stride;
      if (i < n8) {
        q[u] = codes[i];
        sc[u] = e8m0_to_f32(scales[i >> 2]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * stride;
      if (i < n8) {
        uint32_t o[4];
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[u].x, sc[u], false));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[u].x, sc[u], true));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[u].y, sc[u], false));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[u].y, sc[u], true));
        out[i] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

template <int BM, int BN, int S, int WGM, int WGN, bool ACC, bool SC>
int launch_f8_sc(hipStream_t st, F8Args g) {
  constexpr int lds = F8Layout<BM, BN, S, WGM, WGN, ACC, SC>::kLds;
  auto kfn = gemm_f8fwd<BM, BN, S, WGM, WGN, ACC, SC>;
  static std::atomic<uint64_t> attr{0};
  if (smem_attr_once(reinterpret_cast<const void*>(kfn), lds, attr)) return -5;
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + BN - 1) / BN;
  hipLaunchKernelGGL(kfn, dim3(g.tiles_m * g.tiles_n, 1, ACC ? g.splits : 1), dim3(WGM * WGN * 64), lds, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// The group scale cache takes 16-byte loads from each scale row: rows of K/32 scale bytes must
// start 16-byte aligned (K % 512 == 0, aligned arrays).
template <int BM, int BN, int S, int WGM, int WGN, bool ACC = false>
int launch_f8(hipStream_t st, F8Args g) {
  const bool sc = g.K % 512 == 0 && (reinterpret_cast<uintptr_t>(g.sa) & 15u) == 0 &&
                  (reinterpret_cast<uintptr_t>(g.sb) & 15u) == 0;
  return sc ? launch_f8_sc<BM, BN, S, WGM, WGN, ACC, true>(st, g) : launch_f8_sc<BM, BN, S, WGM, WGN, ACC, false>(st, g);
}

}  // namespace sl2

int f8_fwd(hipStream_t st, F8Args g) {
  switch (g.cfg) {
    case 0: return sl2::launch_f8<256, 256, 2, 2, 4>(st, g);
    case 1: return sl2::launch_f8<128, 128, 3, 2, 2>(st, g);
    case 2: return sl2::launch_f8<256, 128, 3, 4, 2>(st, g);
    default: return -1;
  }
}

int f8_accum(hipStream_t st, F8Args g) {
  switch (g.cfg) {
    case 0: return sl2::launch_f8<256, 256, 2, 2, 4, true>(st, g);
    case 1: return sl2::launch_f8<128, 128, 3, 2, 2, true>(st, g);
    case 2: return sl2::launch_f8<256, 128, 3, 4, 2, true>(st, g);
    default: return -1;
  }
}

int mx_dequant(hipStream_t st, const uint8_t* codes, const uint8_t* scales, void* out, int64_t rows, int64_t cols) {
  const int64_t n8 = rows * (cols / 8);
  if (n8 == 0) return 0;
  int64_t blocks = (n8 + 1023) / 1024;          // 256 threads x 4 chunks each
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(sl2::mx_dequant_bf16, dim3(unsigned(blocks)), dim3(256), 0, st, reinterpret_cast<const uint2*>(codes),
                     scales, static_cast<uint4*>(out), n8);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
