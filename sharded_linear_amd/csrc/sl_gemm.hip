// GEMM kernels of one tensor-parallel rank's linear step, written for gfx950 (CDNA4, MI355X).
//
// The three products of llm-infra-atlas, "01 · ColumnParallelLinear / RowParallelLinear and the
// core autograd", sections 4.1-4.2:
//   fwd    Y[T,out]        = X[T,in] . W[out,in]^T        M=T   N=out K=in
//   dgrad  dX[T,in]        = dY[T,out] . W[out,in]        M=T   N=in  K=out
//   wgrad  main_grad[out,in] += dY[T,out]^T . X[T,in]     M=out N=in  K=T   (fp32, in place)
// All three are one kernel template: C[m][n] (+)= sum_k A(m,k) B(n,k).  An operand is stored
// either with k contiguous ("K-major": X and W in fwd, dY in dgrad) or with m/n contiguous
// ("MN-major": W in dgrad, dY and X in wgrad).  Both kinds are staged through LDS in one
// layout -- rows of 64 k values, 16-byte chunks XOR-swizzled against bank conflicts -- so the
// MFMA loop is shared; MN-major tiles are transposed in registers (8x8 blocks of bf16) on their
// way from HBM into LDS.
//
// Matrix cores: v_mfma_f32_32x32x16_bf16.  Lane l supplies row (l % 32) of its A block and
// column (l % 32) of its B block with eight consecutive k values (k offset 8*(l/32)); the
// 32x32 fp32 result leaves lane l holding column l % 32, rows 8*(r/4) + 4*(l/32) + r%4 for
// r = 0..15.
//
// MXFP8 operands (NVIDIA Megatron-Core guide "Generalized Tensor Parallelism", section 1.3:
// E4M3 data, one E8M0 scale per 32 elements) are dequantised exactly to bf16 as they are moved
// into LDS, then take the same MFMA path.
//
// Split-K for the weight gradient is deterministic and needs no cross-block synchronisation:
// each split writes its fp32 partial into its own plane of the workspace, and a second kernel
// on the same stream adds the planes in split order and performs the single read-modify-write
// of main_grad.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "sharded_linear.h"
#include "sl_device.h"
#include "sl_gemm2.h"
#include "sl_gemm_f8.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;           // k extent of one LDS stage
constexpr int kCH = kBK / 8;      // 16-byte chunks per LDS row
constexpr int kXCD = 8;           // accelerator complex dies; workgroups are dealt round-robin

enum class Elem { BF16, MXFP8 };
enum class Epi { StoreBF16, AccumF32 };

struct Operand {
  const void* p;        // bf16 storage, or E4M3 codes for MXFP8
  const uint8_t* s;     // E8M0 scales (MXFP8 only), row-major [rows of storage][ld / 32]
  int64_t ld;           // elements between consecutive storage rows
  int rows;             // extent of the free (m or n) index
};

struct Args {
  Operand a, b;
  void* c;
  int64_t ldc;
  int M, N, K;
  int tiles_m, tiles_n;
  int splits, kt_per_split;
  float* ws;            // split-K partial planes [splits][M][N]
  float alpha = 1.0f;   // bf16 results are alpha * (A . B^T), scaled in fp32 before rounding
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Eight E4M3 codes (one 8-byte chunk) with their block scale -> eight bf16 in a 16-byte chunk.
__device__ __forceinline__ uint4 dequant8(uint2 q, uint32_t s) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t src = i < 2 ? q.x : q.y;
    const int sh = (i & 1) * 16;
    w[i] = sl2::e4m3_to_bf16((src >> sh) & 0xFFu, s) | (sl2::e4m3_to_bf16((src >> (sh + 8)) & 0xFFu, s) << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Element loader: the 8 consecutive elements of storage row `srow` starting at column `col`
// (a multiple of 8), as a 16-byte chunk of bf16.
template <Elem E>
struct Chunk;

template <>
struct Chunk<Elem::BF16> {
  uint4 v;
  __device__ __forceinline__ void load(const Operand& op, int64_t srow, int64_t col) {
    v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(op.p) + srow * op.ld + col);
  }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ uint4 get() const { return v; }
};

template <>
struct Chunk<Elem::MXFP8> {
  uint2 q;
  uint32_t s;
  __device__ __forceinline__ void load(const Operand& op, int64_t srow, int64_t col) {
    q = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(op.p) + srow * op.ld + col);
    s = op.s[srow * (op.ld / 32) + col / 32];
  }
  __device__ __forceinline__ void zero() { q = make_uint2(0, 0); s = 127; }
  __device__ __forceinline__ uint4 get() const { return dequant8(q, s); }
};

// K-major operand tile: R rows (free index) x kBK k; storage row = free index, k contiguous.
template <int R, int NT, Elem E>
struct KMajTile {
  static constexpr int kPasses = R * kCH / NT;
  static_assert(kPasses * NT == R * kCH, "tile/thread mismatch");
  Chunk<E> ch[kPasses];

  __device__ __forceinline__ void load(const Operand& op, int row0, int k0, int K, int tid) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int r = p * (NT / kCH) + tid / kCH, c = tid % kCH;
      const int gr = row0 + r, k = k0 + c * 8;
      if (gr < op.rows && k < K) ch[p].load(op, gr, k); else ch[p].zero();
    }
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int r = p * (NT / kCH) + tid / kCH, c = tid % kCH;
      lds[r * kCH + (c ^ swz(r))] = ch[p].get();
    }
  }
};

// MN-major operand tile: storage row = k, free index contiguous.  Each thread moves blocks of
// KB k rows x 8 consecutive free indices (KB = 8, or 4 when the tile has too few 8x8 blocks for
// one per thread) and transposes them so that LDS again holds rows of consecutive k.
template <int R, int NT, Elem E>
struct MNMajTile {
  static constexpr int KB = (R / 8) * (kBK / 8) >= NT ? 8 : 4;
  static constexpr int kBlocks = (R / 8) * (kBK / KB);
  static constexpr int kPer = kBlocks / NT;
  static_assert(kPer >= 1 && kPer * NT == kBlocks, "tile/thread mismatch");
  Chunk<E> ch[kPer][KB];

  __device__ __forceinline__ void load(const Operand& op, int row0, int k0, int K, int tid) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int q = p * NT + tid, rb = q % (R / 8), kb = q / (R / 8);
      const int gr = row0 + rb * 8;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int k = k0 + kb * KB + j;
        if (gr < op.rows && k < K) ch[p][j].load(op, k, gr); else ch[p][j].zero();
      }
    }
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int q = p * NT + tid, rb = q % (R / 8), kb = q / (R / 8);
      uint32_t in[KB][4];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const uint4 v = ch[p][j].get();
        in[j][0] = v.x; in[j][1] = v.y; in[j][2] = v.z; in[j][3] = v.w;
      }
      // in[j] holds free indices 8rb..8rb+7 at k = KB*kb + j (two bf16 per word, even index low)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t o[KB / 2];
#pragma unroll
        for (int w = 0; w < KB / 2; ++w) {
          const uint32_t lo = in[2 * w][i >> 1], hi = in[2 * w + 1][i >> 1];
          o[w] = (i & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        const int r = rb * 8 + i;
        if constexpr (KB == 8) {
          lds[r * kCH + (kb ^ swz(r))] = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
          uint2* l2 = reinterpret_cast<uint2*>(lds);
          l2[(r * kCH + ((kb >> 1) ^ swz(r))) * 2 + (kb & 1)] = make_uint2(o[0], o[1]);
        }
      }
    }
  }
};

template <bool KMAJ, int R, int NT, Elem E>
struct TileSel { using T = KMajTile<R, NT, E>; };
template <int R, int NT, Elem E>
struct TileSel<false, R, NT, E> { using T = MNMajTile<R, NT, E>; };

// Deal workgroups so that each XCD works on a contiguous stretch of the tile order (tiles
// that share operand panels then share that XCD's L2).  Hardware hands block b to XCD b % 8.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int per = n / kXCD, rem = n % kXCD, x = b % kXCD;
  return x * per + (x < rem ? x : rem) + b / kXCD;
}

template <int BM, int BN, int WGM, int WGN, bool A_KMAJ, bool B_KMAJ, Elem EA, Elem EB, Epi EPI>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_kernel(Args args) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;        // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;          // 32x32 MFMA blocks per wave
  using TileA = typename TileSel<A_KMAJ, BM, NT, EA>::T;
  using TileB = typename TileSel<B_KMAJ, BN, NT, EB>::T;

  __shared__ uint4 lds_a[2][BM * kCH];
  __shared__ uint4 lds_b[2][BN * kCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // tile coordinates: XCD-aware dealing, then groups of 8 tile rows walked column-major
  const int ntiles = args.tiles_m * args.tiles_n;
  const int t = xcd_remap(blockIdx.x, ntiles);
  const int group = t / (8 * args.tiles_n);
  const int first_m = group * 8;
  const int gsz = min(args.tiles_m - first_m, 8);
  const int tm = first_m + (t % (8 * args.tiles_n)) % gsz;
  const int tn = (t % (8 * args.tiles_n)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int split = blockIdx.z;
  const int nkt = (args.K + kBK - 1) / kBK;
  const int kt_begin = split * args.kt_per_split;
  const int kt_end = min(nkt, kt_begin + args.kt_per_split);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  TileA ta;
  TileB tb;
  if (kt_begin < kt_end) {
    ta.load(args.a, m0, kt_begin * kBK, args.K, tid);
    tb.load(args.b, n0, kt_begin * kBK, args.K, tid);
    ta.store(lds_a[0], tid);
    tb.store(lds_b[0], tid);
  }
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = (kt - kt_begin) & 1;
    const bool more = kt + 1 < kt_end;
    if (more) {
      ta.load(args.a, m0, (kt + 1) * kBK, args.K, tid);
      tb.load(args.b, n0, (kt + 1) * kBK, args.K, tid);
    }
    const uint4* la = lds_a[cur];
    const uint4* lb = lds_b[cur];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 32 + (lane & 31);
        const uint4 v = la[r * kCH + (c ^ swz(r))];
        fa[i] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WN + j * 32 + (lane & 31);
        const uint4 v = lb[r * kCH + (c ^ swz(r))];
        fb[j] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      ta.store(lds_a[cur ^ 1], tid);
      tb.store(lds_b[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------------------
  const int row_in_blk = 4 * (lane >> 5);
  const int col_in_blk = lane & 31;
  if constexpr (EPI == Epi::StoreBF16) {
    __bf16* C = static_cast<__bf16*>(args.c);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + col_in_blk;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + row_in_blk + (r & 3);
          if (m < args.M && n < args.N) C[int64_t(m) * args.ldc + n] = static_cast<__bf16>(acc[i][j][r] * args.alpha);
        }
      }
  } else {
    // Unsplit: the single fp32 read-modify-write of main_grad.  Split-K: this split's partial
    // goes to its own plane ws[split][M][N]; splitk_reduce adds the planes into main_grad.
    const bool direct = args.splits == 1;
    float* C = direct ? static_cast<float*>(args.c) : args.ws + int64_t(split) * args.M * args.N;
    const int64_t ldc = direct ? args.ldc : args.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + col_in_blk;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + row_in_blk + (r & 3);
          if (m < args.M && n < args.N) {
            float* p = C + int64_t(m) * ldc + n;
            *p = direct ? *p + acc[i][j][r] : acc[i][j][r];
          }
        }
      }
  }
}

// main_grad[m][n] += sum over splits s (in order) of ws[s][m][n]; n counted in float4 (N % 4 == 0).
__global__ void splitk_reduce(float* C, int64_t ldc, const float* ws, int M, int N, int splits) {
  const int64_t n4 = N / 4, total = int64_t(M) * n4, plane = int64_t(M) * n4;
  const float4* w = reinterpret_cast<const float4*>(ws);
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < splits; ++sp) {
      const float4 v = w[sp * plane + i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    float4* p = reinterpret_cast<float4*>(C + (i / n4) * ldc) + (i % n4);
    float4 c = *p;
    c.x += s.x; c.y += s.y; c.z += s.z; c.w += s.w;
    *p = c;
  }
}

__global__ void fill_zero_f32(float4* p, int64_t n4, float* tail, int ntail) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (blockIdx.x == 0 && int(threadIdx.x) < ntail) tail[threadIdx.x] = 0.f;
}

// ---- host side -------------------------------------------------------------------------------

constexpr int64_t kMaxExtent = int64_t(1) << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(int64_t T, int64_t in, int64_t out, int64_t mult) {
  if (T < 0 || in < 0 || out < 0) return SL_EINVAL;
  if (T >= kMaxExtent || in >= kMaxExtent || out >= kMaxExtent) return SL_ESHAPE;
  if (in % mult || out % mult) return SL_ESHAPE;
  // element offsets of every operand must fit the kernels' 64-bit row arithmetic and the
  // 32-bit tile indices
  return SL_OK;
}

// ---- launch planning ------------------------------------------------------------------------
// bf16 operands go through the direct-to-LDS kernels (sl_gemm2.hip) whenever every operand's
// byte extent fits their 31-bit buffer offsets; MXFP8 operands (dequantised on the way into
// LDS) and larger operands use the register-staged kernels above.

enum class Kind { Fwd, Dgrad, Wgrad };

struct Plan {
  bool v2;          // direct-to-LDS kernel family
  int cfg;          // its tile configuration
  int bm, bn, bk;   // macro-tile
  int splits, kps;  // split-K (weight gradient only)
};

constexpr int64_t kMaxDmaBytes = 0x7FFFFFF0LL - 16;

int64_t ntiles(int64_t M, int64_t N, int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); }

// Tuning overrides, set through sl_set_tuning (-1: the built-in choice).  Process-wide and read
// with relaxed loads: a query and the calls it sizes see the same values unless the caller
// changes them in between.
std::atomic<int> g_tune[SL_TUNE_COUNT] = {{-1}, {-1}, {-1}, {-1}, {-1}};

int config_override(Kind k) {
  return g_tune[k == Kind::Fwd ? SL_TUNE_FWD_CONFIG : k == Kind::Dgrad ? SL_TUNE_DGRAD_CONFIG : SL_TUNE_WGRAD_CONFIG]
      .load(std::memory_order_relaxed);
}

int splits_override() {
  const int v = g_tune[SL_TUNE_SPLITK].load(std::memory_order_relaxed);
  return v > 0 ? v : 0;
}

// Tile configuration for a forward / dgrad GEMM: each candidate's time is estimated as the number
// of rounds of workgroups over the 256 CUs times one round's work (tile area x workgroups per CU)
// over the candidate's measured efficiency relative to the 8-wave 256x256 kernel.  The weight
// gradient always takes 256x256 tiles and fills the chip by splitting K instead.  The forward also
// considers the fixed-order 256x192 kernel (cfg 25).
int pick_config(Kind kind, int64_t M, int64_t N) {
  struct Cand { int cfg, bm, bn, occ; double eff; };
  static const Cand cand[] = {{10, 256, 256, 1, 1.0}, {12, 256, 128, 2, 0.85}, {13, 128, 256, 2, 0.85},
                              {3, 256, 128, 1, 0.78}, {4, 128, 256, 1, 0.78}, {2, 128, 128, 1, 0.6},
                              {kGemm2FwdOnlyConfig, 256, 192, 1, 0.92}};
  int best = 10;
  double best_t = 0.0;
  for (const Cand& c : cand) {
    if (c.cfg == kGemm2FwdOnlyConfig && kind != Kind::Fwd) continue;
    const int64_t rounds = (ntiles(M, N, c.bm, c.bn) + 256 * c.occ - 1) / (256 * c.occ);
    const double t = double(rounds) * double(c.bm * c.bn * c.occ) / c.eff;
    if (best_t == 0.0 || t < best_t) { best = c.cfg; best_t = t; }
  }
  return best;
}

Plan make_plan_cfg(Kind kind, bool mxfp8, int64_t M, int64_t N, int64_t K, int64_t a_bytes, int64_t b_bytes,
                   int cfg) {
  Plan p{};
  p.v2 = !mxfp8 && a_bytes <= kMaxDmaBytes && b_bytes <= kMaxDmaBytes;
  if (p.v2) {
    p.cfg = cfg;
    gemm2_tile(cfg, &p.bm, &p.bn, &p.bk);
  } else {
    const bool big = ntiles(M, N, 256, 256) >= 200;
    p.bm = p.bn = big ? 256 : 128;
    p.bk = kBK;
  }
  // split-K for the weight gradient: fill ~256 CUs with output tiles, keep >= 8 k stages per split
  const int64_t tiles = ntiles(M, N, p.bm, p.bn);
  const int64_t nkt = (K + p.bk - 1) / p.bk;
  int64_t s = 1;
  if (kind == Kind::Wgrad && tiles < 200) s = (256 + tiles / 2) / tiles;
  const int64_t min_stages = p.bk == 32 ? 16 : 8;
  if (s > nkt / min_stages) s = nkt / min_stages;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  if (kind == Kind::Wgrad && splits_override()) s = splits_override();
  int64_t per = (nkt + s - 1) / s;
  if (per < 1) per = 1;
  p.kps = int(per);
  p.splits = int(nkt == 0 ? 1 : (nkt + per - 1) / per);
  return p;
}

Plan make_plan(Kind kind, bool mxfp8, int64_t M, int64_t N, int64_t K, int64_t a_bytes, int64_t b_bytes) {
  int cfg = config_override(kind);
  if (cfg < 0) {
    cfg = kind == Kind::Wgrad ? 10 : pick_config(kind, M, N);
    // 256x256 tiles: the fixed-order 8-wave kernel on the 16x16x32 instruction (2 stages of 64 k)
    // for all three products.  Against the 32x32x16 kernels (fwd: 8 waves, 2 x 64 k; dgrad and
    // wgrad: 4 waves, 4 x 32 k) it measured 2-9 % ahead on the forward and up to 18 % on the
    // weight gradients of short-K shapes: the part holds a higher clock under the 16x16 form.
    if (cfg == 10) cfg = 21;
    // A weight gradient whose 256x256 tiles cover about half of the 256 CUs, but whose 256x128
    // tiles make one full round, runs those unsplit on the 32x32x16 fixed-order kernel (cfg 20):
    // ahead of two K splits plus the reduce on the 1B MLP shard's down projection (main_grad
    // [2048, 4096] over 8192 tokens), by 5 % and, against later forms of cfg 21, 0.4-0.6 %.
    if (kind == Kind::Wgrad && cfg == 21) {
      const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256), t128 = ((M + 255) / 256) * ((N + 127) / 128);
      if (t256 <= 144 && t128 >= 240 && t128 <= 288) cfg = 20;
    }
    // 256x128 tiles (shapes whose 256x256 tile count leaves CUs idle): the fixed-order 8-wave
    // 16x16x32 kernel with a 3-stage ring of 64 k (64x64 wave tiles), measured 7 % ahead of the
    // 4-wave 32x32x16 one (cfg 19) and 27 % ahead of the compiler-scheduled one on dgrad
    if (cfg == 3 && kind != Kind::Wgrad) cfg = 24;
  }
  Plan p = make_plan_cfg(kind, mxfp8, M, N, K, a_bytes, b_bytes, cfg);
  // configurations that prefill a deep ring need that many k stages in every split
  if (p.v2) {
    const int64_t nkt = (K + p.bk - 1) / p.bk;
    const int64_t last = nkt - int64_t(p.splits - 1) * p.kps;
    const int need = gemm2_min_stages(p.cfg);
    if (p.kps < need || last < need) p = make_plan_cfg(kind, mxfp8, M, N, K, a_bytes, b_bytes, 10);
  }
  return p;
}

// Workspace = split-K partial planes [splits][M][N] fp32; written before it is read within one
// call, so its initial contents never matter.
size_t plan_ws_bytes(const Plan& p, int64_t M, int64_t N) {
  if (p.splits <= 1) return 0;
  return size_t(int64_t(p.splits) * M * N * 4);
}

// weight-gradient GEMM: M = out, N = in, K = T; A = dY [T, out], B = X [T, in] (bf16 or MXFP8)
size_t wgrad_ws_bytes(int64_t T, int64_t in, int64_t out) {
  if (T <= 0 || in <= 0 || out <= 0) return 0;
  return plan_ws_bytes(make_plan(Kind::Wgrad, false, out, in, T, T * out * 2, T * in * 2), out, in);
}

template <int BM, int BN, bool A_KMAJ, bool B_KMAJ, Elem EA, Elem EB, Epi EPI>
int launch(hipStream_t st, Args& a) {
  a.tiles_m = int((a.M + BM - 1) / BM);
  a.tiles_n = int((a.N + BN - 1) / BN);
  dim3 grid(a.tiles_m * a.tiles_n, 1, a.splits);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, 2, 2, A_KMAJ, B_KMAJ, EA, EB, EPI>), grid, dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? SL_OK : SL_EHIP;
}

template <bool A_KMAJ, bool B_KMAJ, Elem EA, Elem EB, Epi EPI>
int run_v1(hipStream_t st, Args& a, const Plan& p) {
  if (p.bm == 256) return launch<256, 256, A_KMAJ, B_KMAJ, EA, EB, EPI>(st, a);
  return launch<128, 128, A_KMAJ, B_KMAJ, EA, EB, EPI>(st, a);
}

// ---- whole rounds plus a tail on smaller tiles -----------------------------------------------
// A product whose 256x256 tiles make whole rounds of the 256 CUs plus a partial last round runs in
// two launches: a region of whole rounds of 256x256 tiles (all of M and a prefix of N, or a prefix
// of M and all of N), then the rest of the output on 256x128 tiles, which covers the tail in about
// half a round.  Each output element is still computed by one workgroup with one k order, so the
// result is the same as the single launch's up to that order and stays deterministic.  Only
// unsplit products on the default 256x256 configuration are split; a forced configuration or split
// count keeps one launch.
struct Region {
  int64_t m_off, n_off, M, N;
  Plan p;
};

// relative throughput of the 256x128 tail configurations against the 256x256 one on the same work
constexpr double kTailEff[3] = {0.85, 0.85, 0.82};   // fwd, dgrad, wgrad

int plan_regions(Kind kind, const Plan& p, int64_t M, int64_t N, int64_t K, int64_t a_bytes, int64_t b_bytes,
                 Region out[2]) {
  out[0] = {0, 0, M, N, p};
  if (!p.v2 || p.cfg != 21 || p.splits != 1 || config_override(kind) >= 0 || splits_override()) return 1;
  const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256, tiles = tm * tn;
  if (tiles < 256 || tiles % 256 == 0) return 1;
  const int tail_cfg = kind == Kind::Wgrad ? 20 : 24;
  const double eff = kTailEff[int(kind)];
  auto rounds = [](int64_t t) { return double((t + 255) / 256); };
  double best = 0.95 * rounds(tiles);
  int n = 1;
  // along N: the first n1 tile columns (tm x n1 a multiple of 256), the remaining columns on 256x128
  for (int64_t n1 = tn - 1; n1 >= 1; --n1) {
    if ((tm * n1) % 256) continue;
    const int64_t N2 = N - n1 * 256;
    const double cost = rounds(tm * n1) + 0.5 / eff * rounds(tm * ((N2 + 127) / 128));
    if (cost < best) {
      best = cost;
      out[0] = {0, 0, M, n1 * 256, p};
      out[1] = {0, n1 * 256, M, N2, make_plan_cfg(kind, false, M, N2, K, a_bytes, b_bytes, tail_cfg)};
      n = 2;
    }
    break;
  }
  // along M: the first m1 tile rows, the remaining rows on 256x128
  for (int64_t m1 = tm - 1; m1 >= 1; --m1) {
    if ((m1 * tn) % 256) continue;
    const int64_t M2 = M - m1 * 256;
    const double cost = rounds(m1 * tn) + 0.5 / eff * rounds(((M2 + 255) / 256) * ((N + 127) / 128));
    if (cost < best) {
      best = cost;
      out[0] = {0, 0, m1 * 256, N, p};
      out[1] = {m1 * 256, 0, M2, N, make_plan_cfg(kind, false, M2, N, K, a_bytes, b_bytes, tail_cfg)};
      n = 2;
    }
    break;
  }
  if (n == 2) {
    // the tail region runs unsplit like the first; its configuration prefills a 3- or 4-stage ring,
    // so it needs that many k stages
    Plan& t = out[1].p;
    t.splits = 1;
    t.kps = int((K + t.bk - 1) / t.bk);
    if (!t.v2 || t.kps < gemm2_min_stages(tail_cfg)) {
      out[0] = {0, 0, M, N, p};
      n = 1;
    }
  }
  return n;
}

int run_v2(hipStream_t st, Kind kind, const Args& a, const Plan& p, int64_t a_bytes, int64_t b_bytes);

// Launch a product through plan_regions: each region is the same product on sub-views of the
// operands (a K-major operand is offset by whole rows, an MN-major one by columns) and of C.
int run_v2_regions(hipStream_t st, Kind kind, const Args& a, const Plan& p, int64_t a_bytes, int64_t b_bytes) {
  Region r[2];
  const int n = plan_regions(kind, p, a.M, a.N, a.K, a_bytes, b_bytes, r);
  if (n == 1) return run_v2(st, kind, a, p, a_bytes, b_bytes);
  const bool a_kmaj = kind != Kind::Wgrad, b_kmaj = kind == Kind::Fwd;
  const int64_t cbytes = kind == Kind::Wgrad ? 4 : 2;
  for (int i = 0; i < n; ++i) {
    Args s = a;
    const int64_t ao = (a_kmaj ? r[i].m_off * a.a.ld : r[i].m_off) * 2;
    const int64_t bo = (b_kmaj ? r[i].n_off * a.b.ld : r[i].n_off) * 2;
    s.a.p = static_cast<const char*>(a.a.p) + ao;
    s.b.p = static_cast<const char*>(a.b.p) + bo;
    s.c = static_cast<char*>(a.c) + (r[i].m_off * a.ldc + r[i].n_off) * cbytes;
    s.M = int(r[i].M);
    s.N = int(r[i].N);
    s.a.rows = int(r[i].M);
    s.b.rows = int(r[i].N);
    s.splits = 1;
    s.kt_per_split = r[i].p.kps;
    const int st_ = run_v2(st, kind, s, r[i].p, a_bytes - ao, b_bytes - bo);
    if (st_) return st_;
  }
  return SL_OK;
}

int run_v2(hipStream_t st, Kind kind, const Args& a, const Plan& p, int64_t a_bytes, int64_t b_bytes) {
  Gemm2Args g{};
  g.a = a.a.p; g.b = a.b.p; g.c = a.c;
  g.lda = a.a.ld; g.ldb = a.b.ld; g.ldc = a.ldc;
  g.a_bytes = uint32_t(a_bytes); g.b_bytes = uint32_t(b_bytes);
  g.M = a.M; g.N = a.N; g.K = a.K;
  g.splits = a.splits; g.kt_per_split = a.kt_per_split;
  g.ws = a.ws;
  g.cfg = p.cfg;
  g.alpha = a.alpha;
  const int r = kind == Kind::Fwd ? gemm2_fwd(st, g) : kind == Kind::Dgrad ? gemm2_dgrad(st, g) : gemm2_wgrad(st, g);
  return r == 0 ? SL_OK : SL_EHIP;
}

int bind_workspace(Args& a, const Plan& p, int64_t M, int64_t N, void* ws, size_t ws_bytes) {
  a.splits = p.splits;
  a.kt_per_split = p.kps;
  if (p.splits > 1) {
    if (!ws || ws_bytes < plan_ws_bytes(p, M, N) || !aligned16(ws)) return SL_EWORKSPACE;
    a.ws = static_cast<float*>(ws);
  }
  return SL_OK;
}

// Second half of a split-K weight gradient: main_grad += the partial planes, in split order.
int reduce_splits(hipStream_t st, const Args& a) {
  if (a.splits <= 1) return SL_OK;
  const int64_t n4 = int64_t(a.M) * (a.N / 4);
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(splitk_reduce, dim3(unsigned(blocks)), dim3(256), 0, st, static_cast<float*>(a.c), a.ldc,
                     static_cast<const float*>(a.ws), a.M, a.N, a.splits);
  return hipGetLastError() == hipSuccess ? SL_OK : SL_EHIP;
}

Args base_args(int64_t M, int64_t N, int64_t K, const Plan& p) {
  Args a{};
  a.M = int(M); a.N = int(N); a.K = int(K);
  a.splits = 1;
  a.kt_per_split = int((K + p.bk - 1) / p.bk);
  return a;
}

// Y = alpha * (X . W^T) in bf16 (alpha = 1 for the plain product)
int linear_fwd(hipStream_t hs, const void* X, const void* W, float alpha, void* Y, int64_t T, int64_t in,
               int64_t out) {
  int st = check_dims(T, in, out, 8);
  if (st) return st;
  if (T == 0 || out == 0) return SL_OK;
  if (!Y || (in > 0 && (!X || !W))) return SL_EINVAL;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return SL_EALIGN;
  const Plan p = make_plan(Kind::Fwd, false, T, out, in, T * in * 2, out * in * 2);
  Args a = base_args(T, out, in, p);
  a.a = {X, nullptr, in, int(T)};
  a.b = {W, nullptr, in, int(out)};
  a.c = Y;
  a.ldc = out;
  a.alpha = alpha;
  if (p.v2) return run_v2_regions(hs, Kind::Fwd, a, p, T * in * 2, out * in * 2);
  return run_v1<true, true, Elem::BF16, Elem::BF16, Epi::StoreBF16>(hs, a, p);
}

// dX = alpha * (dY . W) in bf16
int linear_dgrad(hipStream_t hs, const void* dY, const void* W, float alpha, void* dX, int64_t T, int64_t in,
                 int64_t out) {
  int st = check_dims(T, in, out, 8);
  if (st) return st;
  if (T == 0 || in == 0) return SL_OK;
  if (!dX || (out > 0 && (!dY || !W))) return SL_EINVAL;
  if (!aligned16(dY) || !aligned16(W) || !aligned16(dX)) return SL_EALIGN;
  const Plan p = make_plan(Kind::Dgrad, false, T, in, out, T * out * 2, out * in * 2);
  Args a = base_args(T, in, out, p);
  a.a = {dY, nullptr, out, int(T)};
  a.b = {W, nullptr, in, int(in)};
  a.c = dX;
  a.ldc = in;
  a.alpha = alpha;
  if (p.v2) return run_v2_regions(hs, Kind::Dgrad, a, p, T * out * 2, out * in * 2);
  return run_v1<true, false, Elem::BF16, Elem::BF16, Epi::StoreBF16>(hs, a, p);
}

}  // namespace

extern "C" int sl_set_tuning(int32_t knob, int32_t value, int32_t* previous) {
  static const int hi[SL_TUNE_COUNT] = {kGemm2Configs - 1, kGemm2FwdOnlyConfig - 1, kGemm2FwdOnlyConfig - 1, 64, 2};
  static_assert(kGemm2FwdOnlyConfig == kGemm2Configs - 1, "the forward-only configuration comes last");
  static const int lo[SL_TUNE_COUNT] = {0, 0, 0, 1, 0};
  if (knob < 0 || knob >= SL_TUNE_COUNT) return SL_EINVAL;
  if (value != -1 && (value < lo[knob] || value > hi[knob])) return SL_EINVAL;
  const int old = g_tune[knob].exchange(value);
  if (previous) *previous = old;
  return SL_OK;
}

extern "C" int sl_grad_buffer_zero(void* stream, float* grad_data, int64_t numel) {
  if (numel < 0) return SL_EINVAL;
  if (numel == 0) return SL_OK;
  if (!grad_data) return SL_EINVAL;
  if (!aligned16(grad_data)) return SL_EALIGN;
  const int64_t n4 = numel / 4;
  const int ntail = int(numel - n4 * 4);
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_f32, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<float4*>(grad_data), n4, grad_data + n4 * 4, ntail);
  return hipGetLastError() == hipSuccess ? SL_OK : SL_EHIP;
}

extern "C" int sl_linear_fwd(void* stream, const void* X, const void* W, void* Y, int64_t T, int64_t in,
                             int64_t out) {
  return linear_fwd(static_cast<hipStream_t>(stream), X, W, 1.0f, Y, T, in, out);
}

extern "C" int sl_linear_dgrad(void* stream, const void* dY, const void* W, void* dX, int64_t T, int64_t in,
                               int64_t out) {
  return linear_dgrad(static_cast<hipStream_t>(stream), dY, W, 1.0f, dX, T, in, out);
}

// ---- NVFP4 weights ------------------------------------------------------------------------------
// The weight shard is stored as NVFP4 (NVIDIA Megatron-Core guide "Generalized Tensor
// Parallelism", section 1.3, native NVFP4 param): E2M1 codes, an E4M3 scale per 16 elements and
// one fp32 tensor scale.  Every E2M1 x E4M3 product is a bf16 value, so the materialised weight
// holds those products exactly and the tensor scale multiplies the fp32 accumulators before the
// bf16 rounding of the result; the products themselves run on the bf16 kernels.

extern "C" int sl_nvfp4_materialize(void* stream, const uint8_t* Wq, const uint8_t* Ws, void* Wm, int64_t rows,
                                    int64_t cols) {
  if (rows < 0 || cols < 0) return SL_EINVAL;
  if (cols % 16) return SL_ESHAPE;
  if (rows >= kMaxExtent || cols >= kMaxExtent) return SL_ESHAPE;
  if (rows == 0 || cols == 0) return SL_OK;
  if (!Wq || !Ws || !Wm) return SL_EINVAL;
  if (!aligned16(Wq) || !aligned16(Wm)) return SL_EALIGN;
  return nvfp4_expand(static_cast<hipStream_t>(stream), Wq, Ws, Wm, rows, cols) == 0 ? SL_OK : SL_EHIP;
}

extern "C" int sl_linear_fwd_nvfp4w(void* stream, const void* X, const void* Wm, float w_scale, void* Y,
                                    int64_t T, int64_t in, int64_t out) {
  if (!std::isfinite(w_scale)) return SL_EINVAL;
  if (in % 16) return SL_ESHAPE;
  return linear_fwd(static_cast<hipStream_t>(stream), X, Wm, w_scale, Y, T, in, out);
}

extern "C" int sl_linear_dgrad_nvfp4w(void* stream, const void* dY, const void* Wm, float w_scale, void* dX,
                                      int64_t T, int64_t in, int64_t out) {
  if (!std::isfinite(w_scale)) return SL_EINVAL;
  if (in % 16) return SL_ESHAPE;
  return linear_dgrad(static_cast<hipStream_t>(stream), dY, Wm, w_scale, dX, T, in, out);
}

extern "C" size_t sl_wgrad_workspace_bytes(int64_t T, int64_t in, int64_t out) {
  if (T < 0 || in < 0 || out < 0) return 0;
  return wgrad_ws_bytes(T, in, out);
}

extern "C" int sl_linear_wgrad_accum(void* stream, const void* X, const void* dY, float* main_grad, int64_t T,
                                     int64_t in, int64_t out, void* workspace, size_t workspace_bytes) {
  int st = check_dims(T, in, out, 8);
  if (st) return st;
  if (T == 0 || in == 0 || out == 0) return SL_OK;
  if (!X || !dY || !main_grad) return SL_EINVAL;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(main_grad)) return SL_EALIGN;
  const Plan p = make_plan(Kind::Wgrad, false, out, in, T, T * out * 2, T * in * 2);
  Args a = base_args(out, in, T, p);
  a.a = {dY, nullptr, out, int(out)};
  a.b = {X, nullptr, in, int(in)};
  a.c = main_grad;
  a.ldc = in;
  st = bind_workspace(a, p, out, in, workspace, workspace_bytes);
  if (st) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = p.v2 ? run_v2_regions(hs, Kind::Wgrad, a, p, T * out * 2, T * in * 2)
            : run_v1<false, false, Elem::BF16, Elem::BF16, Epi::AccumF32>(hs, a, p);
  return st ? st : reduce_splits(hs, a);
}

// ---- the weight gradient without allocation --------------------------------------------------
// For callers that cannot allocate: the split-K partial planes live in a file-scope device array
// instead of a caller workspace.  Each GPU holds its own copy from module load until the process
// ends; host code reaches it only through the address hipGetSymbolAddress returns on that device
// (the array's name in host code is a host-side stand-in, not a device address).

constexpr size_t kNoAllocScratchBytes = size_t(SL_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// This device's `scratch`, resolved once per device with that device current (the stream must
// belong to the current device).  Two threads racing on the first call both store the same
// address.
int device_scratch(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SL_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SL_EINVAL;
  hipDevice_t sdev = -1;
  if (hipStreamGetDevice(st, &sdev) != hipSuccess) return SL_EHIP;
  if (sdev != dev) return SL_EINVAL;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SL_EHIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SL_OK;
}

}  // namespace

extern "C" int sl_linear_wgrad_accum_noalloc(void* stream, const void* X, const void* dY, float* main_grad,
                                             int64_t T, int64_t in, int64_t out) {
  int st = check_dims(T, in, out, 8);
  if (st) return st;
  if (T == 0 || in == 0 || out == 0) return SL_OK;
  if (!X || !dY || !main_grad) return SL_EINVAL;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(main_grad)) return SL_EALIGN;
  const size_t need = wgrad_ws_bytes(T, in, out);
  if (need > kNoAllocScratchBytes) return SL_EWORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need) {
    st = device_scratch(hs, &ws);
    if (st) return st;
  }
  return sl_linear_wgrad_accum(stream, X, dY, main_grad, T, in, out, ws, need ? kNoAllocScratchBytes : 0);
}

// ---- MXFP8 operand entry points -----------------------------------------------------------
// The native paths need 128 | in (whole 4-block scale dwords per stage) and dword-aligned scale
// rows; other shapes take the register-staged kernels, which dequantise in registers.

namespace {

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Block-scaled fp8 forward configuration: 256x256 tiles (8 waves) when they fill the chip, else
// 128x128.  The SL_TUNE_F8_CONFIG knob forces configuration n (0: 256x256, 1: 128x128, 2: 256x128).
int f8_config_override() { return g_tune[SL_TUNE_F8_CONFIG].load(std::memory_order_relaxed); }

int f8_config(int64_t T, int64_t out) {
  const int cfg = f8_config_override();
  if (cfg >= 0) return cfg;
  return ntiles(T, out, 256, 256) >= 200 ? 0 : 1;
}

bool f8_native(int64_t T, int64_t in, int64_t out, const void* Xs, const void* Ws) {
  return in % 128 == 0 && aligned4(Xs) && aligned4(Ws) && T * in <= kMaxDmaBytes && out * in <= kMaxDmaBytes;
}

// Dequantised operand (bf16) at the front of an MXFP8 workspace, then the bf16 split-K planes.
int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

bool mx_bf16_path(int64_t rows, int64_t in, int64_t other_bytes) {
  return in % 32 == 0 && rows * in * 2 <= kMaxDmaBytes && other_bytes <= kMaxDmaBytes;
}

}  // namespace

extern "C" int sl_mxfp8_dequantize(void* stream, const uint8_t* q, const uint8_t* s, void* out, int64_t rows,
                                   int64_t cols) {
  if (rows < 0 || cols < 0) return SL_EINVAL;
  if (cols % 32) return SL_ESHAPE;
  if (rows >= kMaxExtent || cols >= kMaxExtent) return SL_ESHAPE;
  if (rows == 0 || cols == 0) return SL_OK;
  if (!q || !s || !out) return SL_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return SL_EALIGN;
  return mx_dequant(static_cast<hipStream_t>(stream), q, s, out, rows, cols) == 0 ? SL_OK : SL_EHIP;
}

extern "C" size_t sl_mxfp8_workspace_bytes(int64_t T, int64_t in, int64_t out) {
  if (T <= 0 || in <= 0 || out <= 0 || in % 32) return 0;
  size_t need = 0;
  // dgrad: W [out, in] dequantised
  if (mx_bf16_path(out, in, T * out * 2)) need = size_t(round256(out * in * 2));
  // wgrad: X [T, in] dequantised, plus the bf16 plan's split planes
  if (mx_bf16_path(T, in, T * out * 2)) {
    const Plan p = make_plan(Kind::Wgrad, false, out, in, T, T * out * 2, T * in * 2);
    const size_t w = size_t(round256(T * in * 2)) + plan_ws_bytes(p, out, in);
    if (w > need) need = w;
  } else {
    const Plan p = make_plan(Kind::Wgrad, true, out, in, T, T * out * 2, T * in);
    const size_t w = plan_ws_bytes(p, out, in);
    if (w > need) need = w;
  }
  return need;
}

extern "C" int sl_linear_fwd_mxfp8(void* stream, const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                                   const uint8_t* Ws, void* Y, int64_t T, int64_t in, int64_t out) {
  int st = check_dims(T, in, out, 8);
  if (st) return st;
  if (in % 32) return SL_ESHAPE;
  if (T == 0 || out == 0) return SL_OK;
  if (!Y || (in > 0 && (!Xq || !Xs || !Wq || !Ws))) return SL_EINVAL;
  if (!aligned16(Xq) || !aligned16(Wq) || !aligned16(Y)) return SL_EALIGN;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (in > 0 && f8_native(T, in, out, Xs, Ws)) {
    F8Args g{};
    g.a = Xq; g.b = Wq; g.sa = Xs; g.sb = Ws; g.c = Y;
    g.lda = in; g.ldb = in; g.ldc = out;
    g.a_bytes = uint32_t(T * in); g.b_bytes = uint32_t(out * in);
    g.sa_bytes = uint32_t(T * (in / 32)); g.sb_bytes = uint32_t(out * (in / 32));
    g.M = int(T); g.N = int(out); g.K = int(in);
    g.cfg = f8_config(T, out);
    return f8_fwd(hs, g) == 0 ? SL_OK : SL_EHIP;
  }
  const Plan p = make_plan(Kind::Fwd, true, T, out, in, T * in, out * in);
  Args a = base_args(T, out, in, p);
  a.a = {Xq, Xs, in, int(T)};
  a.b = {Wq, Ws, in, int(out)};
  a.c = Y;
  a.ldc = out;
  return run_v1<true, true, Elem::MXFP8, Elem::MXFP8, Epi::StoreBF16>(hs, a, p);
}

extern "C" int sl_linear_dgrad_mxfp8w(void* stream, const void* dY, const uint8_t* Wq, const uint8_t* Ws,
                                      void* dX, int64_t T, int64_t in, int64_t out, void* workspace,
                                      size_t workspace_bytes) {
  int st = check_dims(T, in, out, 8);
  if (st) return st;
  if (in % 32) return SL_ESHAPE;
  if (T == 0 || in == 0) return SL_OK;
  if (!dX || (out > 0 && (!dY || !Wq || !Ws))) return SL_EINVAL;
  if (!aligned16(dY) || !aligned16(Wq) || !aligned16(dX)) return SL_EALIGN;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (out > 0 && mx_bf16_path(out, in, T * out * 2)) {
    if (!workspace || !aligned16(workspace) || workspace_bytes < size_t(round256(out * in * 2))) return SL_EWORKSPACE;
    if (mx_dequant(hs, Wq, Ws, workspace, out, in)) return SL_EHIP;
    return sl_linear_dgrad(stream, dY, workspace, dX, T, in, out);
  }
  const Plan p = make_plan(Kind::Dgrad, true, T, in, out, T * out * 2, out * in);
  Args a = base_args(T, in, out, p);
  a.a = {dY, nullptr, out, int(T)};
  a.b = {Wq, Ws, in, int(in)};
  a.c = dX;
  a.ldc = in;
  return run_v1<true, false, Elem::BF16, Elem::MXFP8, Epi::StoreBF16>(hs, a, p);
}

extern "C" int sl_linear_wgrad_accum_mxfp8x(void* stream, const uint8_t* Xq, const uint8_t* Xs, const void* dY,
                                            float* main_grad, int64_t T, int64_t in, int64_t out, void* workspace,
                                            size_t workspace_bytes) {
  int st = check_dims(T, in, out, 8);
  if (st) return st;
  if (in % 32) return SL_ESHAPE;
  if (T == 0 || in == 0 || out == 0) return SL_OK;
  if (!Xq || !Xs || !dY || !main_grad) return SL_EINVAL;
  if (!aligned16(Xq) || !aligned16(dY) || !aligned16(main_grad)) return SL_EALIGN;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (mx_bf16_path(T, in, T * out * 2)) {
    // the whole workspace (dequantised X, then the bf16 plan's split planes) is checked before
    // the first launch
    const int64_t xb = round256(T * in * 2);
    const Plan p = make_plan(Kind::Wgrad, false, out, in, T, T * out * 2, T * in * 2);
    if (!workspace || !aligned16(workspace) || workspace_bytes < size_t(xb) + plan_ws_bytes(p, out, in))
      return SL_EWORKSPACE;
    if (mx_dequant(hs, Xq, Xs, workspace, T, in)) return SL_EHIP;
    return sl_linear_wgrad_accum(stream, workspace, dY, main_grad, T, in, out, static_cast<char*>(workspace) + xb,
                                 workspace_bytes - size_t(xb));
  }
  const Plan p = make_plan(Kind::Wgrad, true, out, in, T, T * out * 2, T * in);
  Args a = base_args(out, in, T, p);
  a.a = {dY, nullptr, out, int(out)};
  a.b = {Xq, Xs, in, int(in)};
  a.c = main_grad;
  a.ldc = in;
  st = bind_workspace(a, p, out, in, workspace, workspace_bytes);
  if (st) return st;
  st = run_v1<false, false, Elem::BF16, Elem::MXFP8, Epi::AccumF32>(hs, a, p);
  return st ? st : reduce_splits(hs, a);
}

// ---- all-MXFP8 step: quantisation and the both-MXFP8 dgrad / wgrad --------------------------

namespace {

// Tiles and split-K of the fp8 weight gradient (128-k stages).  256x256 tiles by default; where
// they fill only about half the chip but 256x128 tiles fill it once, those run unsplit (no partial
// planes, no reduce).  Otherwise split K to fill ~256 CUs with output tiles, keeping at least 8
// stages per split and at most 16 splits.  The SL_TUNE_F8_CONFIG knob forces the tile configuration.
F8Args f8_wgrad_plan(int64_t T, int64_t in, int64_t out) {
  F8Args g{};
  g.M = int(out); g.N = int(in); g.K = int(T);
  const int64_t t256 = ntiles(out, in, 256, 256), t128 = ntiles(out, in, 256, 128);
  const int forced = f8_config_override();
  g.cfg = forced >= 0 ? forced : (t256 <= 144 && t128 >= 240 && t128 <= 288) ? 2 : 0;
  const int64_t tiles = g.cfg == 0 ? t256 : g.cfg == 2 ? t128 : ntiles(out, in, 128, 128), nkt = T / 128;
  int64_t s = tiles < 200 ? (256 + tiles / 2) / tiles : 1;
  if (s > nkt / 8) s = nkt / 8;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  const int64_t per = (nkt + s - 1) / s;
  g.kt_per_split = int(per);
  g.splits = int((nkt + per - 1) / per);
  return g;
}

bool f8_extents_ok(int64_t a_bytes, int64_t b_bytes) { return a_bytes <= kMaxDmaBytes && b_bytes <= kMaxDmaBytes; }

}  // namespace

extern "C" int sl_mxfp8_quantize(void* stream, const void* x, int64_t rows, int64_t cols, uint8_t* q_rows,
                                 uint8_t* s_rows, uint8_t* q_cols, uint8_t* s_cols) {
  if (rows < 0 || cols < 0) return SL_EINVAL;
  if (rows >= kMaxExtent || cols >= kMaxExtent) return SL_ESHAPE;
  if (!q_rows != !s_rows || !q_cols != !s_cols) return SL_EINVAL;
  if ((q_rows && cols % 32) || (q_cols && (rows % 32 || cols % 8))) return SL_ESHAPE;
  if (rows == 0 || cols == 0 || (!q_rows && !q_cols)) return SL_OK;
  if (!x) return SL_EINVAL;
  if (!aligned16(x) || (q_rows && !aligned16(q_rows)) || (q_cols && !aligned16(q_cols))) return SL_EALIGN;
  return mx_quantize(static_cast<hipStream_t>(stream), x, rows, cols, q_rows, s_rows, q_cols, s_cols) == 0 ? SL_OK
                                                                                                        : SL_EHIP;
}

extern "C" int sl_linear_dgrad_mxfp8(void* stream, const uint8_t* dYq, const uint8_t* dYs, const uint8_t* WqT,
                                     const uint8_t* WsT, void* dX, int64_t T, int64_t in, int64_t out) {
  int st = check_dims(T, in, out, 8);
  if (st) return st;
  if (out % 128) return SL_ESHAPE;
  if (T == 0 || in == 0) return SL_OK;
  if (!dX || (out > 0 && (!dYq || !dYs || !WqT || !WsT))) return SL_EINVAL;
  if (!aligned16(dX) || (out > 0 && (!aligned16(dYq) || !aligned16(WqT) || !aligned4(dYs) || !aligned4(WsT))))
    return SL_EALIGN;
  if (!f8_extents_ok(T * out, in * out)) return SL_ESHAPE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  F8Args g{};   // out == 0: the kernel runs no k stage and stores zeros
  g.a = dYq; g.b = WqT; g.sa = dYs; g.sb = WsT; g.c = dX;
  g.lda = out; g.ldb = out; g.ldc = in;
  g.a_bytes = uint32_t(T * out); g.b_bytes = uint32_t(in * out);
  g.sa_bytes = uint32_t(T * (out / 32)); g.sb_bytes = uint32_t(in * (out / 32));
  g.M = int(T); g.N = int(in); g.K = int(out);
  g.cfg = f8_config(T, in);
  return f8_fwd(hs, g) == 0 ? SL_OK : SL_EHIP;
}

extern "C" size_t sl_mxfp8_wgrad_workspace_bytes(int64_t T, int64_t in, int64_t out) {
  if (T <= 0 || in <= 0 || out <= 0 || T % 128) return 0;
  const F8Args g = f8_wgrad_plan(T, in, out);
  return g.splits > 1 ? size_t(int64_t(g.splits) * out * in * 4) : 0;
}

extern "C" int sl_linear_wgrad_accum_mxfp8(void* stream, const uint8_t* dYqT, const uint8_t* dYsT, const uint8_t* XqT,
                                           const uint8_t* XsT, float* main_grad, int64_t T, int64_t in, int64_t out,
                                           void* workspace, size_t workspace_bytes) {
  int st = check_dims(T, in, out, 8);
  if (st) return st;
  if (T % 128) return SL_ESHAPE;
  if (T == 0 || in == 0 || out == 0) return SL_OK;
  if (!dYqT || !dYsT || !XqT || !XsT || !main_grad) return SL_EINVAL;
  if (!aligned16(dYqT) || !aligned16(XqT) || !aligned16(main_grad) || !aligned4(dYsT) || !aligned4(XsT))
    return SL_EALIGN;
  if (!f8_extents_ok(out * T, in * T)) return SL_ESHAPE;
  F8Args g = f8_wgrad_plan(T, in, out);
  if (g.splits > 1) {
    if (!workspace || !aligned16(workspace) || workspace_bytes < sl_mxfp8_wgrad_workspace_bytes(T, in, out))
      return SL_EWORKSPACE;
    g.ws = static_cast<float*>(workspace);
  }
  g.a = dYqT; g.b = XqT; g.sa = dYsT; g.sb = XsT; g.c = main_grad;
  g.lda = T; g.ldb = T; g.ldc = in;
  g.a_bytes = uint32_t(out * T); g.b_bytes = uint32_t(in * T);
  g.sa_bytes = uint32_t(out * (T / 32)); g.sb_bytes = uint32_t(in * (T / 32));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (f8_accum(hs, g)) return SL_EHIP;
  if (g.splits <= 1) return SL_OK;
  Args a{};
  a.M = g.M; a.N = g.N; a.c = main_grad; a.ldc = in; a.splits = g.splits; a.ws = g.ws;
  return reduce_splits(hs, a);
}
