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
// MFMA: v_mfma_f32_32x32x16_bf16 (operand lane l: row/column l%32, k = 8*(l/32)+0..7; result
// lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4).
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
  // Byte offsets of this thread's loads relative to the stage's first k (rows outside the matrix
  // -> kOOB).  A stage wholly inside K then loads with these and a scalar offset of 2 k0.
  template <int WAVES, int N = kLoads / WAVES>
  __device__ static __forceinline__ void prep(uint32_t (&voff)[N], int lane, int wave, int row0, int rows,
                                              int64_t ld) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int p = (it * WAVES + wave) * 64 + lane;
      const int r = p / kCPR, c = (p % kCPR) ^ swz(p / kCPR);
      voff[it] = row0 + r < rows ? uint32_t((int64_t(row0 + r) * ld + c * 8) * 2) : kOOB;
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
  // Byte offsets relative to the stage's first k row (columns outside the matrix -> kOOB); a
  // stage wholly inside K loads with these and a scalar offset of 2 k0 ld.
  template <int WAVES, int N = kLoads / WAVES>
  __device__ static __forceinline__ void prep(uint32_t (&voff)[N], int lane, int wave, int col0, int cols,
                                              int64_t ld) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int p = (it * WAVES + wave) * 64 + lane;
      const int k = p / kCPR, c = (p % kCPR) ^ swz(p / kCPR);
      const int gc = col0 + c * 8;
      voff[it] = gc < cols ? uint32_t((int64_t(k) * ld + gc) * 2) : kOOB;
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

// Workgroup -> macro-tile: blocks are dealt round-robin to the XCDs, so the block id is first
// remapped to make each XCD's blocks a contiguous run of tile ids; tile ids then walk groups of
// 8 tile rows column by column, so the tiles one XCD runs at a time share A and B panels in its L2.
template <int BM, int BN>
__device__ __forceinline__ void tile_origin(const Gemm2Args& g, int& m0, int& n0) {
  const int ntiles = g.tiles_m * g.tiles_n;
  const int t = xcd_remap(blockIdx.x, ntiles);
  const int group = t / (8 * g.tiles_n);
  const int first_m = group * 8;
  const int gsz = min(g.tiles_m - first_m, 8);
  const int tm = first_m + (t % (8 * g.tiles_n)) % gsz;
  const int tn = (t % (8 * g.tiles_n)) / gsz;
  m0 = tm * BM;
  n0 = tn * BN;
}

// Loads [LO, HI) of one stage of an operand with precomputed offsets (wave `w` issues wave-loads
// it * WAVES + w, each 1 KiB of LDS).
// `koff` is the stage's byte offset along k, applied through the instruction's scalar offset.
template <int WAVES, int LO, int HI, int N>
__device__ __forceinline__ void load_pre(i32x4 rs, char* lds, int wave, const uint32_t (&voff)[N], uint32_t koff) {
#pragma unroll
  for (int it = LO; it < HI; ++it) lds_dma16s(rs, lds_addr(lds + (it * WAVES + wave) * 1024), voff[it], koff);
}

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
template <int WN, int ROWS, bool ACC>
struct Epi {
  static constexpr int kES = ACC ? 4 : 2;               // bytes per element
  static constexpr int kRowBytes = WN * kES;
  static constexpr int kCPR = kRowBytes / 16;           // 16-byte chunks per row
  static constexpr int kRPI = 64 / kCPR;                // rows per wave instruction
  static constexpr int kBytes = ROWS * kRowBytes;       // LDS per wave
  __device__ static __forceinline__ int off(int r, int c) { return r * kRowBytes + ((c ^ (r & (kCPR - 1))) << 4); }
};
template <int WM, int WN, bool ACC>
using EpiOf = Epi<WN, ACC ? 32 : WM, ACC>;

template <int WM, int WN, int TM, int TN, bool ACC>
__device__ __forceinline__ void store_tile(const Gemm2Args& g, f32x16 (&acc)[TM][TN], char* smem, int mw, int nw,
                                           int split, int lane, int wave) {
  using E = EpiOf<WM, WN, ACC>;
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
          for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(acc[i][j][4 * q + e]);
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

  int m0, n0;
  tile_origin<BM, BN>(g, m0, n0);

  const int split = blockIdx.z;
  const int nkt = (g.K + BK - 1) / BK;
  const int kt0 = split * g.kt_per_split;
  const int kt1 = min(nkt, kt0 + g.kt_per_split);
  const int nk = kt1 - kt0;

  const i32x4 ra = rsrc(g.a, g.a_bytes), rb = rsrc(g.b, g.b_bytes);

  // k16 steps per stage.  The next stage's loads go out over the first kLoadSteps of them: early
  // enough to land before the stage ends, spread enough not to stall the MFMA stream (measured
  // best at two steps for BK 64).
  constexpr int NP = BK / 16;
  constexpr int kLoadSteps = NP < 2 ? NP : 2;
  constexpr int LA = OA::kLoads / WAVES, LB = OB::kLoads / WAVES;
  // Stages wholly inside K use offsets computed once plus a scalar offset for the stage's first k
  // (no vector work per load); a ragged last stage checks k per load.
  uint32_t voa[LA], vob[LB];
  OA::template prep<WAVES>(voa, lane, wave, m0, g.M, g.lda);
  OB::template prep<WAVES>(vob, lane, wave, n0, g.N, g.ldb);
  // Part `part` of `nparts` of one stage's loads (parts split the per-thread loads evenly).
  auto issue_part = [&](int kt, int slot, auto part, auto nparts) {
    constexpr int P = decltype(part)::value, Q = decltype(nparts)::value;
    constexpr int A0 = P * LA / Q, A1 = (P + 1) * LA / Q;
    constexpr int B0 = P * LB / Q, B1 = (P + 1) * LB / Q;
    if constexpr (A1 > A0 || B1 > B0) {
      char* base = smem + slot * kStage;
      const int k0 = kt * BK;
      if (k0 + BK <= g.K) {
        load_pre<WAVES, A0, A1>(ra, base, wave, voa, uint32_t(A_KM ? int64_t(k0) * 2 : int64_t(k0) * g.lda * 2));
        load_pre<WAVES, B0, B1>(rb, base + OA::kBytes, wave, vob, uint32_t(B_KM ? int64_t(k0) * 2 : int64_t(k0) * g.ldb * 2));
      } else {
        OA::template load<WAVES, A0, A1>(ra, base, lane, wave, m0, g.M, k0, g.K, g.lda);
        OB::template load<WAVES, B0, B1>(rb, base + OA::kBytes, lane, wave, n0, g.N, k0, g.K, g.ldb);
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

  // prologue: S-1 stages in flight (stages past the end load zeros: uniform wait counts)
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue_part(kt0 + (s < nk ? s : nk), s, ic<0>{}, ic<1>{});

  constexpr int kDs = TM * (A_KM ? 1 : 2) + TN * (B_KM ? 1 : 2);   // LDS reads per k16 step
  // Interleave the MFMAs of a k16 step with the LDS reads issued before them.
  auto interleave = [&]() {
#pragma unroll
    for (int q = 0; q < TM * TN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < kDs) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (kDs > TM * TN) __builtin_amdgcn_sched_group_barrier(0x100, kDs - TM * TN, 0);
  };

  for (int it = 0; it < nk; ++it) {
    wait_vmcnt<(S - 2) * kLoadsPerThread>();
    __syncthreads();
    const int nxt = it + S - 1;
    const int kt_next = kt0 + (nxt < nk ? nxt : nk), slot_next = nxt % S;
    const char* la = smem + (it % S) * kStage;
    const char* lb = la + OA::kBytes;
    // fragments double-buffered in registers: the reads for k16 step ks+1 are in flight while
    // the MFMAs of step ks issue
    bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = OA::frag(la, wm * WM + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = OB::frag(lb, wn * WN + j * 32, 0, lane);
    static_for<NP>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      constexpr int cur = ks & 1;
      if constexpr (ks < kLoadSteps) issue_part(kt_next, slot_next, ksc, ic<kLoadSteps>{});
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
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
      if constexpr (SCHED == 1 && ks + 1 < NP) interleave();
    });
  }
  wait_vmcnt<0>();

  __syncthreads();    // every wave is past its last operand read: the ring becomes epilogue space
  store_tile<WM, WN, TM, TN, ACC>(g, acc, smem, m0 + wm * WM, n0 + wn * WN, split, lane, wave);
}

template <int BM, int BN, int BK, int S, int WGM, int WGN, bool A_KM, bool B_KM, bool ACC, int SCHED = 0, int OCC = 1>
int launch_cfg(hipStream_t st, Gemm2Args g) {
  using OA = typename OpSel<A_KM, BM, BK>::T;
  using OB = typename OpSel<B_KM, BN, BK>::T;
  constexpr int ring = S * (OA::kBytes + OB::kBytes);
  constexpr int epi = WGM * WGN * EpiOf<BM / WGM, BN / WGN, ACC>::kBytes;
  constexpr int lds = ring > epi ? ring : epi;
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
  static const int t[kGemm2Configs][2] = {
      {256, 256}, {256, 256}, {128, 128}, {256, 128}, {128, 256}, {256, 256}, {256, 256},
      {256, 256}, {256, 256}, {256, 256}, {256, 256}, {256, 256}, {256, 128}, {128, 256},
      {256, 128}};
  *bm = t[cfg][0];
  *bn = t[cfg][1];
}
