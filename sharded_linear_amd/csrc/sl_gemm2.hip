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
// lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4) and, in the default fixed-order
// configurations, v_mfma_f32_16x16x32_bf16 (operand lane l: row/column l%16, k = 8*(l/16)+0..7;
// result lane l holds column l%16, rows 4*(l/16) + r).  Both take the B fragment first, so each
// accumulator block holds C^T and a lane owns one output row with four consecutive columns per
// register quad (the epilogue in sl_epi.h relies on that).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "sl_gemm2.h"
#include "sl_device.h"
#include "sl_epi.h"

namespace sl2 {


// ---- K-major operand: LDS [R rows][BK] bf16 -----------------------------------------------
template <int R, int BK, int SW = 0>
struct KMaj {
  static constexpr int kRowBytes = BK * 2;
  static constexpr int kCPR = BK / 8;                  // 16-byte chunks per row
  static constexpr int kBytes = R * kRowBytes;
  static constexpr int kLoads = kBytes / 1024;         // wave-loads of 1 KiB per stage
  static_assert(BK == 32 || BK == 64, "row swizzles are defined for BK 32 and 64");
  // XOR swizzle of 16-byte chunks by row, chosen by measurement: a wave's ds_read_b128 of one
  // fragment (32 rows, two chunks) runs at the rate of linear addresses -- full LDS rate with 8
  // waves per CU -- with these, while the 64-byte-row alternative ((r >> 1) ^ (r >> 3)) & 3,
  // conflict-free on paper for 8 and 16 consecutive lanes, ran 1.7x slower.
  // SW 1 serves the 16x16x32 fragment read (16 rows, four chunks) at BK 64: a ds_read_b128 pairs
  // lanes 0-7 with 16-23 (rows r with chunks c, c+1), so the four same-parity rows of an 8-row
  // block need distinct swizzles in bits {1,2} and in bits {0,2}, and rows r, r+8 distinct ones;
  // {0,3,5,6} by bits 1-2 of r, complemented for rows 8-15, meets all three and measured at the
  // linear rate.
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (SW == 1) {
      static_assert(BK == 64, "16x16 swizzle is defined for BK 64");
      return ((0x6530 >> (4 * ((r >> 1) & 3))) & 7) ^ (((r >> 3) & 1) * 7);
    } else if constexpr (BK == 64) {
      return (r & 7) ^ ((r >> 3) & 1);
    } else {
      return (r ^ (r >> 2)) & 3;
    }
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
  // (the compiler-scheduled kernels; the fixed-order ones compute offsets once, see kmaj_frag_off)
  __device__ static __forceinline__ bf16x8 frag(const char* lds, int r0, int ks, int lane) {
    const int r = r0 + (lane & 31);
    const int c = ks * 2 + (lane >> 5);
    const uint4 v = *reinterpret_cast<const uint4*>(lds + r * kRowBytes + ((c ^ swz(r)) << 4));
    return __builtin_bit_cast(bf16x8, v);
  }
};

// ---- MN-major operand: LDS [BK rows (k)][R] bf16 -------------------------------------------
template <int R, int BK, int SW = 0>
struct MNMaj {
  static constexpr int kRowBytes = R * 2;
  static constexpr int kCPR = R / 8;
  static constexpr int kBytes = BK * kRowBytes;
  static constexpr int kLoads = kBytes / 1024;
  static_assert(kRowBytes % 128 == 0, "rows must span whole bank windows");
  // XOR swizzle of 16-byte chunks by k row: for the 4 rows x 16 free indices read by each
  // 16-lane group of ds_read_b64_tr_b16 (and the 4 x 32 read by 32 lanes), the 32-byte chunk
  // pairs are pair ^ {0, 5, 2, 7}, distinct within 128- and 256-byte bank windows.
  // SW 1 serves the 16x16x32 fragment read, whose 32 lanes read k rows kb..kb+3 and kb+8..kb+11
  // of the same 16 free indices: those rows also flip the low pair bit ({1, 4, 3, 6}), so the
  // eight 32-byte pieces fill a 256-byte window.  Bit 3 of k is constant over a fragment's rows,
  // so its k32 steps and second read stay immediates.
  __device__ static __forceinline__ int swz(int k) {
    if constexpr (SW == 1) return (((k & 3) ^ ((k & 1) << 2)) ^ ((k >> 3) & 1)) << 1;
    else return ((k & 3) ^ ((k & 1) << 2)) << 1;
  }

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

template <bool KM, int R, int BK, int SW = 0>
struct OpSel { using T = KMaj<R, BK, SW>; };
template <int R, int BK, int SW>
struct OpSel<false, R, BK, SW> { using T = MNMaj<R, BK, SW>; };

// Workgroup -> macro-tile: blocks are dealt round-robin to the XCDs, so the block id is first
// remapped to make each XCD's blocks a contiguous run of tile ids; tile ids then walk groups of
// GR tile rows column by column, so the tiles one XCD runs at a time share A and B panels in its
// L2.  The fixed-order kernels take GR = 4 (an XCD's 32 tiles then span 4 tile rows and 8
// columns): against 8 it measured 3.6 % faster on the dgrad of the Llama-3.2-1B MLP shard and
// 0.3-1.5 % on the other products there and on the 7B layer shard; 2 and 16 were slower.
template <int BM, int BN, int GR = 8>
__device__ __forceinline__ void tile_origin(const Gemm2Args& g, int& m0, int& n0) {
  const int ntiles = g.tiles_m * g.tiles_n;
  const int t = xcd_remap(blockIdx.x, ntiles);
  const int group = t / (GR * g.tiles_n);
  const int first_m = group * GR;
  const int gsz = min(g.tiles_m - first_m, GR);
  const int tm = first_m + (t % (GR * g.tiles_n)) % gsz;
  const int tn = (t % (GR * g.tiles_n)) / gsz;
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

// ---- kernels with a fixed issue order ------------------------------------------------------------
// WGM x WGN waves (4 or 8), each computing a WM x WN part of a 256 x BN tile with TM x TN
// accumulator blocks, so an MFMA step (k16 for 32x32 blocks, k32 for 16x16) is TM*TN MFMAs against
// TM + TN fragment reads.  The LDS ring holds S stages of BK k; the loads of stage s + S go out
// right after the barrier that ends the reads of stage s, so every load has S - 1 stages of MFMA
// work to land.  Each step interleaves its MFMAs with the fragment reads of the next step and,
// where due, the HBM->LDS loads; sched_barrier fences keep exactly that order.  The stage barrier
// sits before a stage's last step: that step's fragments are already in registers, so its MFMAs
// cover the first reads of the next stage issued just after the barrier, and no wave starts a
// stage waiting on LDS.
//
// Barrier B(s+1), before the last step of stage s, certifies (i) every wave's loads of stage s + 1
// have landed (each wave waits for its own with vmcnt first) and (ii) every wave has read all of
// stage s (its last-step fragments were waited for), so its slot can take stage s + S.
//
// MF selects the matrix instruction: 32 for v_mfma_f32_32x32x16_bf16 (k16 steps, 32x32 blocks),
// 16 for v_mfma_f32_16x16x32_bf16 (k32 steps, 16x16 blocks).  Both run at the same rate per clock,
// but the 16x16 form draws less power, so the part holds a higher clock under it.
template <bool A_KM, bool B_KM, bool ACC, int S, int WGM, int WGN, int BK_, int BN_ = 256, int MF = 32>
struct G4 {
  static constexpr int BM = 256, BN = BN_, BK = BK_, WAVES = WGM * WGN, WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / MF, TN = WN / MF;
  static constexpr int KS = 512 / MF;                   // k per MFMA step
  using OA = typename OpSel<A_KM, BM, BK, MF == 16 ? 1 : 0>::T;
  using OB = typename OpSel<B_KM, BN, BK, MF == 16 ? 1 : 0>::T;
  static constexpr int kStage = OA::kBytes + OB::kBytes;
  static constexpr int LA = OA::kLoads / WAVES, LB = OB::kLoads / WAVES, LPS = LA + LB;
  static constexpr int kRing = S * kStage;
  static constexpr int kEpi = WAVES * EpiOf<WM, WN, ACC>::kBytes;
  static constexpr int kLds = kRing > kEpi ? kRing : kEpi;
  static_assert(OA::kLoads % WAVES == 0 && OB::kLoads % WAVES == 0, "loads per wave");
  static_assert(S >= 2 && kLds <= 160 * 1024, "ring");
};

// Per-lane LDS byte offset of the first fragment (32 rows from r0) of a K-major operand for k16
// step ks, relative to the operand's base in a stage.  The row swizzle repeats every 32 rows, so
// the other fragments add immediates; steps change the swizzled chunk and need their own offset.
template <class O>
__device__ __forceinline__ uint32_t kmaj_frag_off(int r0, int ks, int lane) {
  const int r = r0 + (lane & 31), c = ks * 2 + (lane >> 5);
  return uint32_t(r * O::kRowBytes + ((c ^ O::swz(r)) << 4));
}
// Same for an MN-major operand's first transposing read (k rows kb..kb+3 of step 0).  The chunk
// swizzle of these rows depends on k % 4 only, so steps (16 rows) and the second read (4 rows
// further) are immediates; fragments differ in their swizzled chunk and need their own offsets.
template <class O>
__device__ __forceinline__ uint32_t mnmaj_frag_off(int f0, int lane) {
  const int g = lane >> 4, s = lane & 15, j = s >> 2, q = s & 3;
  const int f = f0 + 16 * (g & 1) + 4 * q;
  const int k = 8 * (g >> 1) + j;
  return uint32_t(k * O::kRowBytes + (((f >> 3) ^ O::swz(k)) << 4) + ((f & 7) << 1));
}

// The 16x16x32 forms: a fragment is 16 rows (or free indices) x 32 k, lane l holding row l%16
// and k 8(l/16) .. 8(l/16)+7.  K-major: the swizzle repeats every 16 rows, so fragments add
// immediates and each k32 step has its own offset.  MN-major: the four 16-lane groups read k
// rows 8g .. 8g+3 (and 8g+4 .. 8g+7 in the second read) of the same 16 free indices.
template <class O>
__device__ __forceinline__ uint32_t kmaj_frag_off16(int r0, int ks, int lane) {
  const int r = r0 + (lane & 15), c = ks * 4 + (lane >> 4);
  return uint32_t(r * O::kRowBytes + ((c ^ O::swz(r)) << 4));
}
template <class O>
__device__ __forceinline__ uint32_t mnmaj_frag_off16(int f0, int lane) {
  const int g = lane >> 4, s = lane & 15, j = s >> 2, q = s & 3;
  const int f = f0 + 4 * q;
  const int k = 8 * g + j;
  return uint32_t(k * O::kRowBytes + (((f >> 3) ^ O::swz(k)) << 4) + ((f & 7) << 1));
}

template <int OFF>
__device__ __forceinline__ bf16x8 lds_rd128(uint32_t addr) {
  const auto* p = reinterpret_cast<const __attribute__((address_space(3))) uint4*>(addr + OFF);
  return __builtin_bit_cast(bf16x8, *p);
}
template <int OFF0, int OFF1>
__device__ __forceinline__ bf16x8 lds_rd_tr(uint32_t addr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(addr + OFF0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(addr + OFF1));
  const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int N>
__device__ __forceinline__ void asm_wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" : : "i"(N) : "memory"); }

template <bool A_KM, bool B_KM, bool ACC, int S, int WGM, int WGN, int BK_, int BN_, int MF>
__global__ void __launch_bounds__(WGM * WGN * 64, 1) gemm4(Gemm2Args g) {
  using P = G4<A_KM, B_KM, ACC, S, WGM, WGN, BK_, BN_, MF>;
  constexpr int KS = P::KS;
  using AccT = std::conditional_t<MF == 32, f32x16, f32x4v>;
  constexpr int NACC = MF == 32 ? 16 : 4;
  using OA = typename P::OA;
  using OB = typename P::OB;
  constexpr int BK = P::BK, WAVES = P::WAVES, WM = P::WM, WN = P::WN, TM = P::TM, TN = P::TN;
  constexpr int LA = P::LA, LB = P::LB, LPS = P::LPS, kStage = P::kStage;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  int m0, n0;
  tile_origin<P::BM, P::BN, 4>(g, m0, n0);
  const int split = blockIdx.z;
  const int nkt = (g.K + BK - 1) / BK;
  const int kt0 = split * g.kt_per_split;
  const int nk = min(nkt, kt0 + g.kt_per_split) - kt0;
  // The k tiles are walked from a starting point that depends on the XCD (blocks are dealt to
  // the XCDs round-robin): stage j of this split (0 <= j < nk) is k tile kmap(j), a rotation by
  // (3x mod 8) eighths of the split on XCD x (measured 1 % ahead of x eighths).  Without it every
  // workgroup of the chip loads the same k column of its rows at the same time; with rows a power
  // of two apart in HBM (K = 2048 or 8192 bf16), those loads pile onto the same memory channels.
  // The workgroups of one XCD keep one phase, so the operand panels they share in that XCD's L2
  // are still loaded once.  Each tile keeps one fixed k order, so results stay deterministic.
  const int rot = ((((int(blockIdx.x) % kXCD) * 3) % kXCD) * nk) / kXCD;
  auto kmap = [&](int j) { const int x = j + rot; return kt0 + (x >= nk ? x - nk : x); };

  const i32x4 ra = rsrc(g.a, g.a_bytes), rb = rsrc(g.b, g.b_bytes);
  // load offsets relative to a stage's first k; the ragged last stage (K % 32 != 0) uses a copy
  // with the lanes past K sent out of range
  uint32_t voa[LA], vob[LB], vra[LA], vrb[LB];
  OA::template prep<WAVES>(voa, lane, wave, m0, g.M, g.lda);
  OB::template prep<WAVES>(vob, lane, wave, n0, g.N, g.ldb);
  {
    const int kr = g.K - (nkt - 1) * BK;          // k extent of the last stage
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      const int p = (it * WAVES + wave) * 64 + lane;
      const int kk = A_KM ? ((p % OA::kCPR) ^ OA::swz(p / OA::kCPR)) * 8 : p / OA::kCPR;
      vra[it] = kk < kr ? voa[it] : kOOB;
    }
#pragma unroll
    for (int it = 0; it < LB; ++it) {
      const int p = (it * WAVES + wave) * 64 + lane;
      const int kk = B_KM ? ((p % OB::kCPR) ^ OB::swz(p / OB::kCPR)) * 8 : p / OB::kCPR;
      vrb[it] = kk < kr ? vob[it] : kOOB;
    }
  }
  const uint32_t ka_step = A_KM ? BK * 2 : uint32_t(BK * g.lda * 2);
  const uint32_t kb_step = B_KM ? BK * 2 : uint32_t(BK * g.ldb * 2);
  const uint32_t lds0 = lds_addr(smem);

  // fragment read offsets (per lane), K-major: one per MFMA step; MN-major: one per fragment
  constexpr int NPS = BK / KS;
  uint32_t ofa[A_KM ? NPS : TM], ofb[B_KM ? NPS : TN];
  auto kfo_a = [&](int ks) { return MF == 32 ? kmaj_frag_off<OA>(wm * WM, ks, lane) : kmaj_frag_off16<OA>(wm * WM, ks, lane); };
  auto kfo_b = [&](int ks) { return MF == 32 ? kmaj_frag_off<OB>(wn * WN, ks, lane) : kmaj_frag_off16<OB>(wn * WN, ks, lane); };
  auto mfo_a = [&](int f0) { return MF == 32 ? mnmaj_frag_off<OA>(f0, lane) : mnmaj_frag_off16<OA>(f0, lane); };
  auto mfo_b = [&](int f0) { return MF == 32 ? mnmaj_frag_off<OB>(f0, lane) : mnmaj_frag_off16<OB>(f0, lane); };
  if constexpr (A_KM)
#pragma unroll
    for (int ks = 0; ks < NPS; ++ks) ofa[ks] = kfo_a(ks);
  else
#pragma unroll
    for (int i = 0; i < TM; ++i) ofa[i] = mfo_a(wm * WM + MF * i);
  if constexpr (B_KM)
#pragma unroll
    for (int ks = 0; ks < NPS; ++ks) ofb[ks] = OA::kBytes + kfo_b(ks);
  else
#pragma unroll
    for (int j = 0; j < TN; ++j) ofb[j] = OA::kBytes + mfo_b(wn * WN + MF * j);

  AccT acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.f;
  bf16x8 fa[2][TM], fb[2][TN];

  // fragment i (A) or j (B) of MFMA step ks from the stage at LDS byte `base`
  auto read_a = [&](bf16x8& d, uint32_t base, auto ic_i, auto ic_ks) {
    constexpr int i = decltype(ic_i)::value, ks = decltype(ic_ks)::value;
    if constexpr (A_KM) d = lds_rd128<i * MF * OA::kRowBytes>(base + ofa[ks]);
    else d = lds_rd_tr<ks * KS * OA::kRowBytes, (ks * KS + 4) * OA::kRowBytes>(base + ofa[i]);
  };
  auto read_b = [&](bf16x8& d, uint32_t base, auto ic_j, auto ic_ks) {
    constexpr int j = decltype(ic_j)::value, ks = decltype(ic_ks)::value;
    if constexpr (B_KM) d = lds_rd128<j * MF * OB::kRowBytes>(base + ofb[ks]);
    else d = lds_rd_tr<ks * KS * OB::kRowBytes, (ks * KS + 4) * OB::kRowBytes>(base + ofb[j]);
  };
  // wave-load `l` (A: l < LA, then B) of the stage at k tile kt into LDS slot `slot`
  auto load_one = [&](auto ic_l, int kt, int slot, bool ragged) {
    constexpr int l = decltype(ic_l)::value;
    const uint32_t base = lds0 + slot * kStage;
    if constexpr (l < LA) {
      lds_dma16s(ra, base + (l * WAVES + wave) * 1024, ragged ? vra[l] : voa[l], uint32_t(kt) * ka_step);
    } else {
      constexpr int lb = l - LA;
      lds_dma16s(rb, base + OA::kBytes + (lb * WAVES + wave) * 1024, ragged ? vrb[lb] : vob[lb], uint32_t(kt) * kb_step);
    }
  };
  // Memory operation m of a step: m < NR reads fragment piece m into buffer NX; after that the
  // loads [L0, L0 + LPS/2) (or all LPS when ONE) of stage kt into slot `slot` (when `loads`).
  // ONE (the 16x16 kernels): a stage's loads all go out in the step right after the barrier that
  // frees its slot.  Under the 16x16 instruction the part clocks higher, a stage takes less time,
  // and loads issued a step later than that no longer land before the barrier that waits for them.
  constexpr bool ONE = MF == 16;
  constexpr int NR = TM + TN, LH = LPS / 2;
  static_assert(ONE || LPS % 2 == 0, "loads split over two steps");
  auto memop = [&](auto ic_m, auto ic_nx, auto ic_ks, auto ic_l0, uint32_t rbase, bool loads, int kt, int slot,
                   bool ragged) {
    constexpr int m = decltype(ic_m)::value, nx = decltype(ic_nx)::value, l0 = decltype(ic_l0)::value;
    if constexpr (m < NR) {
      if constexpr (m < TM) read_a(fa[nx][m], rbase, ic<m>{}, ic_ks);
      else read_b(fb[nx][m - TM], rbase, ic<m - TM>{}, ic_ks);
    } else {
      if (loads) load_one(ic<l0 + m - NR>{}, kt, slot, ragged);
    }
  };
  // One MFMA step: TM x TN MFMAs on buffer CUR with NM memory operations among them.  The
  // fragment reads go out over the first three quarters of the MFMAs, so they have landed when
  // the step ends (the stage barrier waits for them); the loads are spread evenly over the whole
  // step, one every NQ/NL MFMAs, which keeps the texture-address queue from filling.
  auto step = [&](auto ic_cur, auto ic_nm, auto&& mem) {
    constexpr int cur = decltype(ic_cur)::value, NM = decltype(ic_nm)::value;
    // MFMAs row by row over the A fragments, the B fragments in serpentine order (odd rows run j
    // backwards), so that every MFMA shares an operand with the one before it: the part is held
    // at its power limit, and fewer operand changes measured 0.3-0.6 % faster per launch on every
    // product.
    static_for<TM * TN>([&](auto qc) {
      constexpr int q = decltype(qc)::value, i = q / TN, j = (i & 1) ? TN - 1 - q % TN : q % TN;
      if constexpr (MF == 32)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
      constexpr int NQ = TM * TN, NRD = NR < NM ? NR : NM, NL = NM - NRD;
      constexpr int RQ = NQ * 3 / 4 > 0 ? NQ * 3 / 4 : 1;
      constexpr int rlo = q < RQ ? q * NRD / RQ : NRD, rhi = q < RQ ? (q + 1) * NRD / RQ : NRD;
      static_for<rhi - rlo>([&](auto mc) { mem(ic<rlo + decltype(mc)::value>{}); });
      constexpr int llo = NL ? (2 * q * NL + NQ) / (2 * NQ) : 0, lhi = NL ? (2 * (q + 1) * NL + NQ) / (2 * NQ) : 0;
      static_for<lhi - llo>([&](auto mc) { mem(ic<NRD + llo + decltype(mc)::value>{}); });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  {
    // Prologue: stages 0..S-2 and the first half of stage S-1, or all S stages when ONE (the host
    // launches this kernel only when every split has at least S stages).  From then on the loads of
    // stage x are issued in the last step of stage x - S (just after the barrier that frees its
    // slot): all of them when ONE, else the first half there and the second in the first step of
    // stage x - S + 1.  Either way, at barrier B(s+1) the loads issued after stage s + 1's are the
    // S - 2 whole stages s + 2 .. s + S - 1.
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bool rag = kmap(s) == nkt - 1;
      if (ONE || s < S - 1) static_for<LPS>([&](auto lc) { load_one(lc, kmap(s), s, rag); });
      else static_for<LH>([&](auto lc) { load_one(lc, kmap(s), s, rag); });
    }
    // stage 0 is complete once at most the later prologue stages' loads (S - 1 of them, the last
    // one only half issued unless ONE) are outstanding
    asm_wait_vm<ONE ? LPS * (S - 1) : LPS * (S - 2) + LH>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    static_for<TM>([&](auto ic_i) { read_a(fa[0][decltype(ic_i)::value], lds0, ic_i, ic<0>{}); });
    static_for<TN>([&](auto ic_j) { read_b(fb[0][decltype(ic_j)::value], lds0, ic_j, ic<0>{}); });
    __builtin_amdgcn_sched_barrier(0);

    // Stage s: steps 0 .. NPS-2, each on buffer t % 2 and reading step t + 1 into the other (the
    // first also issues the second half of stage s + S - 1); barrier; the last step on buffer 1
    // (NPS is even), reading the next stage's step 0 into buffer 0 and issuing the first half of
    // stage s + S into s's slot.  At the barrier the loads issued after the last one of stage
    // s + 1 are the S - 2 whole stages s + 2 .. s + S - 1.
    constexpr int NPS_ = BK / KS;
    static_assert(NPS_ % 2 == 0, "steps per stage");
    auto stage = [&](int s, auto ic_vm, auto ic_la, auto ic_lb, auto ic_last) {
      constexpr int VM = decltype(ic_vm)::value;
      constexpr bool LDA = decltype(ic_la)::value, LDB = decltype(ic_lb)::value, LAST = decltype(ic_last)::value;
      const int slot = s % S;
      const uint32_t cur = lds0 + slot * kStage;
      static_for<NPS_ - 1>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr bool ld = !ONE && LDA && t == 0;
        const int kt = kmap(s + S - 1), lslot = (s + S - 1) % S;
        const bool rag = kt == nkt - 1;
        step(ic<t % 2>{}, ic<ld ? NR + LH : NR>{},
             [&](auto ic_m) { memop(ic_m, ic<(t + 1) % 2>{}, ic<t + 1>{}, ic<LH>{}, cur, ld, kt, lslot, rag); });
      });
      if constexpr (!LAST) {
        asm_wait_vm<VM>();
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t nxt = lds0 + ((s + 1) % S) * kStage;
        const int kt = kmap(s + S);
        const bool rag = kt == nkt - 1;
        step(ic<1>{}, ic<LDB ? NR + (ONE ? LPS : LH) : NR>{},
             [&](auto ic_m) { memop(ic_m, ic<0>{}, ic<0>{}, ic<0>{}, nxt, LDB, kt, slot, rag); });
      } else {
        step(ic<1>{}, ic<0>{}, [&](auto) {});
      }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    for (int s = 0; s < nk - S; ++s) stage(s, ic<LPS * (S - 2)>{}, T_{}, T_{}, F_{});
    // The last S stages issue no new stages (the first still completes stage nk - 1); stage
    // nk-S+j waits for stage nk-S+j+1, after which S-2-j whole stages remain outstanding.
    static_for<S>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j == S - 1) stage(nk - S + j, ic<0>{}, std::bool_constant<j == 0>{}, F_{}, T_{});
      else stage(nk - S + j, ic<(S - 2 - j) * LPS>{}, std::bool_constant<j == 0>{}, F_{}, F_{});
    });
  }
  asm_wait_vm<0>();
  __syncthreads();    // every wave is past its last operand read: the ring becomes epilogue space
  if constexpr (MF == 32) store_tile<WM, WN, TM, TN, ACC>(g, acc, smem, m0 + wm * WM, n0 + wn * WN, split, lane, wave);
  else store_tile16<WM, WN, TM, TN, ACC>(g, acc, smem, m0 + wm * WM, n0 + wn * WN, split, lane, wave);
}

template <int BM, int BN, int BK, int S, int WGM, int WGN, bool A_KM, bool B_KM, bool ACC, int SCHED = 0, int OCC = 1>
int launch_cfg(hipStream_t st, Gemm2Args g) {
  using OA = typename OpSel<A_KM, BM, BK>::T;
  using OB = typename OpSel<B_KM, BN, BK>::T;
  constexpr int ring = S * (OA::kBytes + OB::kBytes);
  constexpr int epi = WGM * WGN * EpiOf<BM / WGM, BN / WGN, ACC>::kBytes;
  constexpr int lds = ring > epi ? ring : epi;
  auto kfn = gemm2<BM, BN, BK, S, WGM, WGN, A_KM, B_KM, ACC, SCHED, OCC>;
  static std::atomic<uint64_t> attr{0};
  if (smem_attr_once(reinterpret_cast<const void*>(kfn), lds, attr)) return -5;
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + BN - 1) / BN;
  hipLaunchKernelGGL(kfn, dim3(g.tiles_m * g.tiles_n, 1, g.splits), dim3(WGM * WGN * 64), lds, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int S, int WGM, int WGN, bool A_KM, bool B_KM, bool ACC, int BK = 32, int BN = 256, int MF = 32>
int launch_g4(hipStream_t st, Gemm2Args g) {
  using P = G4<A_KM, B_KM, ACC, S, WGM, WGN, BK, BN, MF>;
  auto kfn = gemm4<A_KM, B_KM, ACC, S, WGM, WGN, BK, BN, MF>;
  static std::atomic<uint64_t> attr{0};
  if (smem_attr_once(reinterpret_cast<const void*>(kfn), P::kLds, attr)) return -5;
  // every split needs at least S stages of 32 k: the prologue fills the whole ring (the planner
  // gives shorter products to another configuration)
  const int nkt = (g.K + P::BK - 1) / P::BK;
  const int last = nkt - (g.splits - 1) * g.kt_per_split;
  if (g.kt_per_split < S || last < S) return -1;
  g.tiles_m = (g.M + P::BM - 1) / P::BM;
  g.tiles_n = (g.N + P::BN - 1) / P::BN;
  hipLaunchKernelGGL(kfn, dim3(g.tiles_m * g.tiles_n, 1, g.splits), dim3(P::WAVES * 64), P::kLds, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// 256x192 tiles exist for the forward only: an MN-major operand 192 wide has 24 chunks per LDS row,
// beyond what the transposing-read swizzle keeps inside a row.
template <bool A_KM, bool B_KM, bool ACC>
int launch_g4_192(hipStream_t st, Gemm2Args g) {
  if constexpr (A_KM && B_KM && !ACC) return launch_g4<2, 2, 4, A_KM, B_KM, ACC, 64, 192, 16>(st, g);
  else return -1;
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
//  15: 256x256, BK 32, 4 stages, 4 waves (128x128 wave tiles), fixed issue order        LDS 128 KiB
//  16: 256x256, BK 32, 4 stages, 8 waves 2x4 (128x64 wave tiles), fixed issue order     LDS 128 KiB
//  17: 256x256, BK 64, 2 stages, 8 waves 2x4 (128x64 wave tiles), fixed issue order     LDS 128 KiB
//  18: 256x256, BK 64, 2 stages, 4 waves (128x128 wave tiles), fixed issue order        LDS 128 KiB
//  19: 256x128, BK 64, 3 stages, 4 waves (128x64 wave tiles), fixed issue order         LDS 144 KiB
//  20: 256x128, BK 32, 4 stages, 4 waves (128x64 wave tiles), fixed issue order         LDS  96 KiB
//  21-23: as 17-19 with v_mfma_f32_16x16x32_bf16 (16x16 blocks, k32 steps)
//  24: 256x128, BK 64, 3 stages, 8 waves 4x2 (64x64 wave tiles), fixed issue order, 16x16x32  LDS 144 KiB
//  25: 256x192, BK 64, 2 stages, 8 waves 2x4 (128x48 wave tiles), fixed issue order, 16x16x32, forward
//      only                                                                                   LDS 112 KiB
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
    case 15: return sl2::launch_g4<4, 2, 2, AK, BKM, ACC>(st, g);                                  \
    case 16: return sl2::launch_g4<4, 2, 4, AK, BKM, ACC>(st, g);                                  \
    case 17: return sl2::launch_g4<2, 2, 4, AK, BKM, ACC, 64>(st, g);                              \
    case 18: return sl2::launch_g4<2, 2, 2, AK, BKM, ACC, 64>(st, g);                              \
    case 19: return sl2::launch_g4<3, 2, 2, AK, BKM, ACC, 64, 128>(st, g);                         \
    case 20: return sl2::launch_g4<4, 2, 2, AK, BKM, ACC, 32, 128>(st, g);                         \
    case 21: return sl2::launch_g4<2, 2, 4, AK, BKM, ACC, 64, 256, 16>(st, g);                     \
    case 22: return sl2::launch_g4<2, 2, 2, AK, BKM, ACC, 64, 256, 16>(st, g);                     \
    case 23: return sl2::launch_g4<3, 2, 2, AK, BKM, ACC, 64, 128, 16>(st, g);                     \
    case 24: return sl2::launch_g4<3, 4, 2, AK, BKM, ACC, 64, 128, 16>(st, g);                     \
    case 25: return sl2::launch_g4_192<AK, BKM, ACC>(st, g);                                       \
    default: return -1;                                                                            \
  }

// SL2_PART splits the instantiations over separate compilations of this file (the build runs
// them in parallel): 1 = fwd and the shared tables, 2 = dgrad, 3 = wgrad; unset = all.
#if !defined(SL2_PART) || SL2_PART == 1
int gemm2_fwd(hipStream_t st, Gemm2Args g) { SL2_DISPATCH(true, true, false) }
#endif
#if !defined(SL2_PART) || SL2_PART == 2
int gemm2_dgrad(hipStream_t st, Gemm2Args g) { SL2_DISPATCH(true, false, false) }
#endif
#if !defined(SL2_PART) || SL2_PART == 3
int gemm2_wgrad(hipStream_t st, Gemm2Args g) { SL2_DISPATCH(false, false, true) }
#endif

#if !defined(SL2_PART) || SL2_PART == 1

int gemm2_min_stages(int cfg) {
  return cfg == 15 || cfg == 16 || cfg == 20 ? 4 : cfg == 17 || cfg == 18 || cfg == 21 || cfg == 22 || cfg == 25 ? 2
         : cfg == 19 || cfg == 23 || cfg == 24 ? 3 : 1;
}

void gemm2_tile(int cfg, int* bm, int* bn, int* bk) {
  *bk = (cfg == 0 || cfg == 7 || cfg == 8 || (cfg >= 12 && cfg <= 16) || cfg == 20) ? 32 : 64;
  static const int t[kGemm2Configs][2] = {
      {256, 256}, {256, 256}, {128, 128}, {256, 128}, {128, 256}, {256, 256}, {256, 256},
      {256, 256}, {256, 256}, {256, 256}, {256, 256}, {256, 256}, {256, 128}, {128, 256},
      {256, 128}, {256, 256}, {256, 256}, {256, 256}, {256, 256}, {256, 128}, {256, 128},
      {256, 256}, {256, 256}, {256, 128}, {256, 128}, {256, 192}};
  *bm = t[cfg][0];
  *bn = t[cfg][1];
}
#endif
