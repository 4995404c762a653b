// Shared device helpers for the gfx950 kernels of libfdl.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fdl.h"

namespace fdl {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Round-to-nearest-even float -> bfloat16 (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

// Two floats -> two bfloat16 (round to nearest even) in one 32-bit word, low
// half first; gfx950 converts in hardware (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-byte global load / store through the vector memory path.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Non-temporal 16-byte load for data read exactly once (streamed weights).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 mfma16x16x32_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x4_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Combination with the lane 32 apart without an LDS round trip:
// v_permlane32_swap hands both lanes of a pair {v[l & 31], v[(l & 31) + 32]}
// (checked on gfx950), so both get the same max / sum, in the same order.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// (max, sum of exp(l - max), lowest argmax) of a run of logits: the partial
// form of the softmax confidence of one row.
struct Red {
  float m, s;
  int i;
};

// merge two partials; equal maxima keep the lower index
__device__ __forceinline__ Red combine(Red a, Red b) {
  Red r;
  r.m = fmaxf(a.m, b.m);
  const float ta = a.s > 0.f ? a.s * exp2f((a.m - r.m) * kLog2e) : 0.f;
  const float tb = b.s > 0.f ? b.s * exp2f((b.m - r.m) * kLog2e) : 0.f;
  r.s = ta + tb;
  r.i = (b.m > a.m || (b.m == a.m && b.i < a.i)) ? b.i : a.i;
  return r;
}

__device__ __forceinline__ void push(Red& r, float x, int v) {
  if (x > r.m) {
    r.s = r.s * exp2f((r.m - x) * kLog2e) + 1.f;
    r.m = x;
    r.i = v;
  } else {
    r.s += exp2f((x - r.m) * kLog2e);
  }
}

// Device-side gate of the decode loop: a launch whose gate word reads 0 does no
// work (every thread returns before its first barrier).  A null gate: always run.
__device__ __forceinline__ bool gate_closed(const int32_t* gate) { return gate != nullptr && *gate == 0; }

__device__ __forceinline__ f32x4 pack_red(Red r) { return f32x4{r.m, r.s, __int_as_float(r.i), 0.f}; }
__device__ __forceinline__ Red unpack_red(f32x4 p) { return Red{p[0], p[1], __float_as_int(p[2])}; }
__device__ __forceinline__ Red red_empty() { return Red{-INFINITY, 0.f, 0x7fffffff}; }
__device__ __forceinline__ Red shfl_xor_red(Red r, int o) {
  return Red{__shfl_xor(r.m, o, kWave), __shfl_xor(r.s, o, kWave), __shfl_xor(r.i, o, kWave)};
}

}  // namespace fdl

// Host-side launch helpers (defined in abi.hip).
namespace fdl {
int dtype_size(int dtype);
int check_launch();
}  // namespace fdl
