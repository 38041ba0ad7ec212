// Device helpers shared by the direct-to-LDS kernels (internal).
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <type_traits>

namespace sl2 {

// Host: hipFuncSetAttribute(MaxDynamicSharedMemorySize) of one kernel, once per device.  `done`
// (one per kernel) holds a bit per device id; ids of 64 and above set the attribute at every
// launch.  Two threads that race on the first launch both set the same value, which is harmless.
inline int smem_attr_once(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -5;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return 0;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return -5;
  if (bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return 0;
}

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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kXCD = 8;
constexpr uint32_t kOOB = 0x7FFFFFF0u;        // offset past every operand extent: loads return zeros
constexpr int kRsrcWord3 = 0x00020000;        // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int per = n / kXCD, rem = n % kXCD, x = b % kXCD;
  return x * per + (x < rem ? x : rem) + b / kXCD;
}

// s_waitcnt with vmcnt <= N and the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt unconstrained: this wave's LDS reads are complete.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Raw buffer descriptor over one operand (gfx9 layout: base, stride 0, num_records = byte
// extent, format word).  Offsets outside the extent -- including kOOB, above every extent the
// host admits -- read zeros instead of touching memory.
__device__ __forceinline__ i32x4 rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = int(uint32_t(a));
  r[1] = int(uint32_t(a >> 32) & 0xFFFFu);
  r[2] = int(bytes);
  r[3] = kRsrcWord3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// One 16-byte-per-lane HBM->LDS load: lane i writes LDS [lds + 16 i, +16).  Issued as inline
// assembly so that the compiler does not guard every later LDS read with a full vmcnt wait;
// the kernel orders these loads itself with wait_vmcnt<>() and a barrier.  gfx9 parts need one
// wait state between a scalar write of M0 and an LDS DMA that reads it; the compiler cannot see
// the DMA inside the assembly, so the s_nop provides it.
__device__ __forceinline__ void lds_dma16(i32x4 rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}

// As lds_dma16, with a wave-uniform byte offset `soff` added to the address.  Lanes whose voff
// lies past the descriptor's extent still read zeros, and in-range lanes must stay in range
// with soff added (the caller only uses it that way), so the result does not depend on whether
// the range check includes soff.
__device__ __forceinline__ void lds_dma16s(i32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds) : "memory");
}

// One 4-byte-per-lane HBM->LDS load: lane i writes LDS [lds + 4 i, +4).
__device__ __forceinline__ void lds_dma4(i32x4 rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" : : "v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}

// E4M3FN code times 2^(s - 127) as bf16 bits.  Value = sig * 2^(max(e,1) - 10) with
// sig = 8 + m for normals (e > 0) and sig = m for subnormals; exact whenever the result is a
// normal bf16 (the caller's contract); NaN codes or the NaN scale give a quiet NaN.
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t code, uint32_t s) {
  const uint32_t sign = (code & 0x80u) << 8;
  const uint32_t e = (code >> 3) & 0xFu, m = code & 0x7u;
  if ((code & 0x7Fu) == 0x7Fu || s == 0xFFu) return sign | 0x7FC0u;
  if ((code & 0x7Fu) == 0) return sign;
  int exp;
  uint32_t mant;
  if (e) {
    exp = int(e) + int(s) - 7;
    mant = m << 4;
  } else {
    const int p = 31 - __builtin_clz(m);            // leading bit of the subnormal field
    exp = p + int(s) - 9;
    mant = ((m << (3 - p)) & 0x7u) << 4;
  }
  if (exp <= 0) return sign;                        // outside the contract: flush
  if (exp >= 255) return sign | 0x7F80u;
  return sign | (uint32_t(exp) << 7) | mant;
}

}  // namespace sl2
