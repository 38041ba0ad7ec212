// bf16 GEMM core of the linear step with direct HBM->LDS operand staging (gfx950).
//
// Same three products as the register-staged kernels (forward, dgrad, fused wgrad-accumulate),
// C[m][n] (+)= sum_k A(m,k) B(n,k), but operands travel from HBM straight into LDS with
// buffer_load_dwordx4 ... lds: lane i of a wave writes 16 bytes at LDS base + 16 i, and lanes
// whose element lies outside the matrix are given an out-of-range offset, so the hardware
// writes zeros there.  A ring of S LDS stages keeps S-1 stages of loads in flight.
//
//  * K-major operand (k contiguous in HBM): LDS rows of BK k values, 16-byte chunks XOR-swizzled
//    by row; MFMA fragments are read with ds_read_b128.
//  * MN-major operand (m or n contiguous in HBM): LDS keeps the HBM orientation, rows of R free
//    indices per k; MFMA fragments are read with ds_read_b64_tr_b16, which transposes 4x4 blocks
//    of 16-bit values across each group of 16 lanes: result lane 4q+e, element j comes from
//    source lane 4j+q, element e.  Source lane 4j+q reads 4 consecutive free indices at k row
//    kb+j, so every result lane holds 4 consecutive k of one free index -- the MFMA layout.
//
// MFMA: v_mfma_f32_32x32x16_bf16 (lane l: row/column l%32, k = 8*(l/32)+0..7; result lane l
// holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "sl_gemm2.h"
#include "sl_device.h"

namespace sl2 {


// ---- K-major operand: LDS [R rows][BK] bf16 -----------------------------------------------
template <int R, int BK>
struct KMaj {
  static constexpr int kRowBytes = BK * 2;
  static constexpr int kCPR = BK / 8;                  // 16-byte chunks per row
  static constexpr int kBytes = R * kRowBytes;
  static constexpr int kLoads = kBytes / 1024;         // wave-loads of 1 KiB per stage
  static_assert(BK == 32 || BK == 64, "row swizzles are defined for BK 32 and 64");
  // XOR swizzle of 16-byte chunks: 8 consecutive rows (a 128-byte bank window per 8 lanes of a
  // 32-bank LDS phase) and 16 consecutive rows (256 bytes per 16 lanes of a 64-bank phase)
  // reading the same logical chunk all land on distinct banks.
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (BK == 64) return (r & 7) ^ ((r >> 3) & 1);
    else return ((r >> 1) ^ (r >> 3)) & 3;
  }

  // Wave `w` issues loads wl = w, w + waves, ...; lane i fills LDS bytes [1024 wl + 16 i, +16).
  template <int WAVES, int LO = 0, int HI = kLoads / WAVES>
  __device__ static __forceinline__ void load(i32x4 rs, char* lds, int lane, int wave,
                                              int row0, int rows, int k0, int K, int64_t ld) {
#pragma unroll
    for (int it = LO; it < HI; ++it) {
      const int wl = it * WAVES + wave;
      const int p = wl * 64 + lane;                      // 16-byte slot
      const int r = p / kCPR, c = (p % kCPR) ^ swz(p / kCPR);
      const int gr = row0 + r, k = k0 + c * 8;
      const uint32_t off = (gr < rows && k < K) ? uint32_t((int64_t(gr) * ld + k) * 2) : kOOB;
      lds_dma16(rs, lds_addr(lds + wl * 1024), off);
    }
  }
  // fragment of 32 rows starting at r0, k16 step ks: lane l gets row r0 + l%32, k 8(l/32)..+7
  __device__ static __forceinline__ bf16x8 frag(const char* lds, int r0, int ks, int lane) {
    const int r = r0 + (lane & 31);
    const int c = ks * 2 + (lane >> 5);
    const uint4 v = *reinterpret_cast<const uint4*>(lds + r * kRowBytes + ((c ^ swz(r)) << 4));
    return __builtin_bit_cast(bf16x8, v);
  }
};

// ---- MN-major operand: LDS [BK rows (k)][R] bf16 -------------------------------------------
template <int R, int BK>
struct MNMaj {
  static constexpr int kRowBytes = R * 2;
  static constexpr int kCPR = R / 8;
  static constexpr int kBytes = BK * kRowBytes;
  static constexpr int kLoads = kBytes / 1024;
  static_assert(kRowBytes % 128 == 0, "rows must span whole bank windows");
  // XOR swizzle of 16-byte chunks by k row: for the 4 rows x 16 free indices read by each
  // 16-lane group of ds_read_b64_tr_b16 (and the 4 x 32 read by 32 lanes), the 32-byte chunk
  // pairs are pair ^ {0, 5, 2, 7}, distinct within 128- and 256-byte bank windows.
  __device__ static __forceinline__ int swz(int k) { return ((k & 3) ^ ((k & 1) << 2)) << 1; }

  template <int WAVES, int LO = 0, int HI = kLoads / WAVES>
  __device__ static __forceinline__ void load(i32x4 rs, char* lds, int lane, int wave,
                                              int col0, int cols, int k0, int K, int64_t ld) {
#pragma unroll
    for (int it = LO; it < HI; ++it) {
      const int wl = it * WAVES + wave;
      const int p = wl * 64 + lane;
      const int k = p / kCPR, c = (p % kCPR) ^ swz(p / kCPR);
      const int gk = k0 + k, gc = col0 + c * 8;
      const uint32_t off = (gk < K && gc < cols) ? uint32_t((int64_t(gk) * ld + gc) * 2) : kOOB;
      lds_dma16(rs, lds_addr(lds + wl * 1024), off);
    }
  }
  // fragment of 32 free indices from f0, k16 step ks, via two transposing reads
  __device__ static __forceinline__ bf16x8 frag(const char* lds, int f0, int ks, int lane) {
    const int g = lane >> 4, s = lane & 15, j = s >> 2, q = s & 3;
    const int f = f0 + 16 * (g & 1) + 4 * q;
    const int k = ks * 16 + 8 * (g >> 1) + j;
    const int cb = f >> 3, eb = (f & 7) << 1;
    const char* p0 = lds + k * kRowBytes + ((cb ^ swz(k)) << 4) + eb;
    const char* p1 = lds + (k + 4) * kRowBytes + ((cb ^ swz(k + 4)) << 4) + eb;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
    const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

template <int I>
using ic = std::integral_constant<int, I>;

// Calls f(ic<0>), ..., f(ic<N-1>): a compile-time loop.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(ic<I>{});
    static_for<N, I + 1>(f);
  }
}

template <bool KM, int R, int BK>
struct OpSel { using T = KMaj<R, BK>; };
template <int R, int BK>
struct OpSel<false, R, BK> { using T = MNMaj<R, BK>; };

// SCHED 0 leaves instruction order to the compiler; SCHED 1 asks it (sched_group_barrier) to
// alternate MFMAs with the LDS fragment reads of the next k16 step.
template <int BM, int BN, int BK, int S, int WGM, int WGN, bool A_KM, bool B_KM, bool ACC, int SCHED, int OCC>
__global__ void __launch_bounds__(WGM * WGN * 64, OCC) gemm2(Gemm2Args g) {
  constexpr int WAVES = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 32, TN = WN / 32;
  using OA = typename OpSel<A_KM, BM, BK>::T;
  using OB = typename OpSel<B_KM, BN, BK>::T;
  constexpr int kStage = OA::kBytes + OB::kBytes;
  constexpr int kLoadsPerThread = (OA::kLoads + OB::kLoads) / WAVES;
  static_assert(OA::kLoads % WAVES == 0 && OB::kLoads % WAVES == 0, "loads per wave");
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
  const int nkt = (g.K + BK - 1) / BK;
  const int kt0 = split * g.kt_per_split;
  const int kt1 = min(nkt, kt0 + g.kt_per_split);
  const int nk = kt1 - kt0;

  const i32x4 ra = rsrc(g.a, g.a_bytes), rb = rsrc(g.b, g.b_bytes);

  auto issue = [&](int kt, int slot) {
    char* base = smem + slot * kStage;
    const int k0 = kt * BK;
    OA::template load<WAVES>(ra, base, lane, wave, m0, g.M, k0, g.K, g.lda);
    OB::template load<WAVES>(rb, base + OA::kBytes, lane, wave, n0, g.N, k0, g.K, g.ldb);
  };
  // The loads of one stage, split into BK/16 parts issued one per k16 step of the loop.
  constexpr int NP = BK / 16;
  constexpr int LA = OA::kLoads / WAVES, LB = OB::kLoads / WAVES;
  constexpr bool kSpread = LA % NP == 0 && LB % NP == 0;
  auto issue_part = [&](int kt, int slot, auto part) {
    constexpr int P = decltype(part)::value;
    char* base = smem + slot * kStage;
    const int k0 = kt * BK;
    if constexpr (kSpread) {
      OA::template load<WAVES, P * LA / NP, (P + 1) * LA / NP>(ra, base, lane, wave, m0, g.M, k0, g.K, g.lda);
      OB::template load<WAVES, P * LB / NP, (P + 1) * LB / NP>(rb, base + OA::kBytes, lane, wave, n0, g.N, k0, g.K, g.ldb);
    } else if constexpr (P == 0) {
      OA::template load<WAVES>(ra, base, lane, wave, m0, g.M, k0, g.K, g.lda);
      OB::template load<WAVES>(rb, base + OA::kBytes, lane, wave, n0, g.N, k0, g.K, g.ldb);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // prologue: S-1 stages in flight (stages past the end load zeros: uniform wait counts)
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(kt0 + (s < nk ? s : nk), s);

  for (int it = 0; it < nk; ++it) {
    wait_vmcnt<(S - 2) * kLoadsPerThread>();
    __syncthreads();
    const int nxt = it + S - 1;
    const int kt_next = kt0 + (nxt < nk ? nxt : nk), slot_next = nxt % S;
    const char* la = smem + (it % S) * kStage;
    const char* lb = la + OA::kBytes;
    // fragments double-buffered in registers: the reads for k16 step ks+1 are in flight while
    // the MFMAs of step ks issue; the next stage's HBM->LDS loads are spread over the steps
    bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = OA::frag(la, wm * WM + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = OB::frag(lb, wn * WN + j * 32, 0, lane);
    static_for<NP>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      constexpr int cur = ks & 1;
      issue_part(kt_next, slot_next, ksc);
      if constexpr (ks + 1 < NP) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[cur ^ 1][i] = OA::frag(la, wm * WM + i * 32, ks + 1, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[cur ^ 1][j] = OB::frag(lb, wn * WN + j * 32, ks + 1, lane);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
      if constexpr (SCHED == 1 && ks + 1 < NP) {
        constexpr int kDs = TM * (A_KM ? 1 : 2) + TN * (B_KM ? 1 : 2);
#pragma unroll
        for (int q = 0; q < TM * TN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (q < kDs) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (kDs > TM * TN) __builtin_amdgcn_sched_group_barrier(0x100, kDs - TM * TN, 0);
      }
    });
  }
  wait_vmcnt<0>();

  // ---- epilogue ----------------------------------------------------------------------------
  // Lane l holds column l%32 of each 32x32 block, rows 8*(r/4) + 4*(l/32) + r%4.  Tiles fully
  // inside the matrix take a branch-free path (loads of a block batched before its adds).
  const int rib = 4 * (lane >> 5), cib = lane & 31;
  const bool interior = m0 + BM <= g.M && n0 + BN <= g.N;
  if constexpr (!ACC) {
    __bf16* C = static_cast<__bf16*>(g.c);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + cib;
        const int mb = m0 + wm * WM + i * 32 + rib;
        if (interior) {
          __bf16* p = C + int64_t(mb) * g.ldc + n;
#pragma unroll
          for (int r = 0; r < 16; ++r) p[int64_t(8 * (r >> 2) + (r & 3)) * g.ldc] = static_cast<__bf16>(acc[i][j][r]);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = mb + 8 * (r >> 2) + (r & 3);
            if (m < g.M && n < g.N) C[int64_t(m) * g.ldc + n] = static_cast<__bf16>(acc[i][j][r]);
          }
        }
      }
  } else {
    // Unsplit: the single fp32 read-modify-write of main_grad.  Split-K: this split's partial
    // goes to its own plane ws[split][M][N] with plain stores; the reduce kernel launched next
    // on the stream adds the planes in split order into main_grad.
    const bool direct = g.splits == 1;
    float* C = direct ? static_cast<float*>(g.c) : g.ws + int64_t(split) * g.M * g.N;
    const int64_t ldc = direct ? g.ldc : g.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + cib;
        const int mb = m0 + wm * WM + i * 32 + rib;
        if (interior) {
          float* p = C + int64_t(mb) * ldc + n;
          if (direct) {
            float old[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) old[r] = p[int64_t(8 * (r >> 2) + (r & 3)) * ldc];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[int64_t(8 * (r >> 2) + (r & 3)) * ldc] = old[r] + acc[i][j][r];
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) p[int64_t(8 * (r >> 2) + (r & 3)) * ldc] = acc[i][j][r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = mb + 8 * (r >> 2) + (r & 3);
            if (m < g.M && n < g.N) {
              float* p = C + int64_t(m) * ldc + n;
              *p = direct ? *p + acc[i][j][r] : acc[i][j][r];
            }
          }
        }
      }
  }
}

template <int BM, int BN, int BK, int S, int WGM, int WGN, bool A_KM, bool B_KM, bool ACC, int SCHED = 0, int OCC = 1>
int launch_cfg(hipStream_t st, Gemm2Args g) {
  using OA = typename OpSel<A_KM, BM, BK>::T;
  using OB = typename OpSel<B_KM, BN, BK>::T;
  constexpr int lds = S * (OA::kBytes + OB::kBytes);
  auto kfn = gemm2<BM, BN, BK, S, WGM, WGN, A_KM, B_KM, ACC, SCHED, OCC>;
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kfn), hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
      return -5;
    attr = true;
  }
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + BN - 1) / BN;
  hipLaunchKernelGGL(kfn, dim3(g.tiles_m * g.tiles_n, 1, g.splits), dim3(WGM * WGN * 64), lds, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace sl2

// ---- dispatch ------------------------------------------------------------------------------
// Tile configurations, indexed by Gemm2Args::cfg:
//   0: 256x256, BK 32, 4 stages, 4 waves (128x128 wave tiles)    LDS 128 KiB
//   1: 256x256, BK 64, 2 stages, 4 waves                          LDS 128 KiB
//   2: 128x128, BK 64, 3 stages, 4 waves (64x64 wave tiles)       LDS  96 KiB
//   3: 256x128, BK 64, 2 stages, 4 waves (128x64 wave tiles)      LDS  96 KiB
//   4: 128x256, BK 64, 2 stages, 4 waves (64x128 wave tiles)      LDS  96 KiB
//   5: 256x256, BK 64, 2 stages, 8 waves 2x4 (128x64 wave tiles)  LDS 128 KiB
//   6: 256x256, BK 64, 2 stages, 8 waves 4x2 (64x128 wave tiles)  LDS 128 KiB
//   7: 256x256, BK 32, 4 stages, 8 waves 2x4 (128x64 wave tiles)  LDS 128 KiB
//   8: 256x256, BK 32, 3 stages, 8 waves 2x4 (128x64 wave tiles)  LDS  96 KiB
//   9: as 1 (4 waves, 128x128 wave tiles) with MFMA / LDS-read interleaving
//  10: as 5 with MFMA / LDS-read interleaving
//  11: as 6 with MFMA / LDS-read interleaving
//  12: 256x128, BK 32, 2 stages, 4 waves (128x64 wave tiles), 2 workgroups per CU   LDS 48 KiB
//  13: 128x256, BK 32, 2 stages, 4 waves (64x128 wave tiles), 2 workgroups per CU   LDS 48 KiB
//  14: 256x128, BK 32, 3 stages, 4 waves (128x64 wave tiles), 2 workgroups per CU   LDS 72 KiB
#define SL2_DISPATCH(AK, BKM, ACC)                                                                 \
  switch (g.cfg) {                                                                                 \
    case 0: return sl2::launch_cfg<256, 256, 32, 4, 2, 2, AK, BKM, ACC>(st, g);                   \
    case 1: return sl2::launch_cfg<256, 256, 64, 2, 2, 2, AK, BKM, ACC>(st, g);                   \
    case 2: return sl2::launch_cfg<128, 128, 64, 3, 2, 2, AK, BKM, ACC>(st, g);                   \
    case 3: return sl2::launch_cfg<256, 128, 64, 2, 2, 2, AK, BKM, ACC>(st, g);                   \
    case 4: return sl2::launch_cfg<128, 256, 64, 2, 2, 2, AK, BKM, ACC>(st, g);                   \
    case 5: return sl2::launch_cfg<256, 256, 64, 2, 2, 4, AK, BKM, ACC>(st, g);                   \
    case 6: return sl2::launch_cfg<256, 256, 64, 2, 4, 2, AK, BKM, ACC>(st, g);                   \
    case 7: return sl2::launch_cfg<256, 256, 32, 4, 2, 4, AK, BKM, ACC>(st, g);                   \
    case 8: return sl2::launch_cfg<256, 256, 32, 3, 2, 4, AK, BKM, ACC>(st, g);                   \
    case 9: return sl2::launch_cfg<256, 256, 64, 2, 2, 2, AK, BKM, ACC, 1>(st, g);                \
    case 10: return sl2::launch_cfg<256, 256, 64, 2, 2, 4, AK, BKM, ACC, 1>(st, g);               \
    case 11: return sl2::launch_cfg<256, 256, 64, 2, 4, 2, AK, BKM, ACC, 1>(st, g);               \
    case 12: return sl2::launch_cfg<256, 128, 32, 2, 2, 2, AK, BKM, ACC, 0, 2>(st, g);            \
    case 13: return sl2::launch_cfg<128, 256, 32, 2, 2, 2, AK, BKM, ACC, 0, 2>(st, g);            \
    case 14: return sl2::launch_cfg<256, 128, 32, 3, 2, 2, AK, BKM, ACC, 0, 2>(st, g);            \
    default: return -1;                                                                            \
  }

int gemm2_fwd(hipStream_t st, Gemm2Args g) { SL2_DISPATCH(true, true, false) }
int gemm2_dgrad(hipStream_t st, Gemm2Args g) { SL2_DISPATCH(true, false, false) }
int gemm2_wgrad(hipStream_t st, Gemm2Args g) { SL2_DISPATCH(false, false, true) }

void gemm2_tile(int cfg, int* bm, int* bn, int* bk) {
  *bk = (cfg == 0 || cfg == 7 || cfg == 8 || cfg >= 12) ? 32 : 64;
  static const int t[15][2] = {{256, 256}, {256, 256}, {128, 128}, {256, 128}, {128, 256}, {256, 256},
                               {256, 256}, {256, 256}, {256, 256}, {256, 256}, {256, 256}, {256, 256},
                               {256, 128}, {128, 256}, {256, 128}};
  *bm = t[cfg][0];
  *bn = t[cfg][1];
}
