// ep_common.h -- shared device helpers of the gfx950 dispatch / combine kernels.
//
// Wave64 throughout: every kernel is written for 64-lane wavefronts (CDNA4),
// rows move as 16-byte vectors (global_load/store_dwordx4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

// 16-byte vector as a clang ext-vector so the non-temporal builtins accept it.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Device error word: one per device, sticky until ep_device_error() reads it.
__device__ unsigned int g_device_error;

constexpr unsigned kErrBadExpert = 1u;   // EP_DEVERR_BAD_EXPERT
constexpr unsigned kErrSplits = 2u;      // EP_DEVERR_SPLITS
constexpr unsigned kErrPlanStall = 4u;   // the plan's look-back gave up waiting
constexpr unsigned kErrBadRow = 8u;      // a position outside the row capacity

__device__ __forceinline__ void raise_device_error(unsigned bits) {
  __hip_atomic_fetch_or(&g_device_error, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave-uniform copy of a value held identically by all active lanes.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Lanes strictly below this one.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Largest of the 64 lanes' values, in every lane (all lanes active).  Within
// each row of 16 lanes by DPP (swap neighbours, swap pairs, mirror halves of
// 8, mirror the row: after each step a lane holds the maximum over 2, 4, 8,
// 16 lanes), then the four rows' maxima through v_readlane.  Each step is
// one VALU operation instead of a round trip through LDS.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// bf16 <-> fp32.  bf16 is the upper half of a binary32; the narrowing rounds
// to nearest, ties to even, keeping NaNs quiet.
__device__ __forceinline__ float bf16lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace ep
