// K/V tiles through LDS for the attention kernels (block attention and
// multi-block attention): direct-to-LDS loads, their waits, the row swizzles
// that keep the fragment reads free of bank conflicts, and a bare barrier.
#pragma once

#include "common.h"

namespace fdl {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane HBM -> LDS: lane l's 16 bytes land at LDS address
// lds + 16 l (lds is wave-uniform; it goes to M0).  Issued from inline
// assembly so that the compiler does not see an LDS write in flight: it would
// otherwise wait for every outstanding load (vmcnt(0)) before each LDS read,
// including the loads of later tiles into other stages.  The kernel waits for
// its loads itself (wait_vm) before the barrier that precedes the reads.
// Nothing else in the kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const void* src, void* lds) {
  const uint32_t l = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(l) : "memory", "m0");
}
// The same from a base address that must be wave-uniform (it is taken from
// the first active lane into SGPRs) and a 32-bit per-lane byte offset.
__device__ __forceinline__ void load_lds16_s(const void* sbase, uint32_t voff, void* lds) {
  const uint32_t l = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));
  const uint64_t p = reinterpret_cast<uint64_t>(sbase);
  // (readfirstlane returns int: widen through uint32_t, not by sign extension)
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(p))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(p >> 32))));
  const uint64_t ps = (uint64_t(hi) << 32) | uint64_t(lo);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(ps), "s"(l) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_barrier with the compiler kept from moving memory accesses across it
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// a ? x : y on pointer values (a conditional over two pointer variables
// would select between their addresses and keep them in scratch memory)
__device__ __forceinline__ const bf16_t* pick(bool a, const bf16_t* x, const bf16_t* y) {
  const uintptr_t ux = reinterpret_cast<uintptr_t>(x), uy = reinterpret_cast<uintptr_t>(y);
  return reinterpret_cast<const bf16_t*>(a ? ux : uy);
}

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((((N >> 4) & 3) << 14) | (0xF << 8) | (7 << 4) | (N & 15));
}

// Physical chunk = logical chunk ^ swizzle(row).  K (fragment reads: 32 rows
// at one logical chunk) spreads consecutive rows over distinct chunks; V
// (transposing reads: 4 consecutive rows x 4 chunks) spreads each group of
// four rows over distinct 4-chunk groups.  d = 64: a row is half of the 64
// banks, so rows 2m and 2m + 1 already differ in bank half.
template <int DH>
__device__ __forceinline__ int swz_k(int row) { return DH == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int DH>
__device__ __forceinline__ int swz_v(int row) { return DH == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }

}  // namespace fdl
