// Device-side helpers shared by the Mesa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mesa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Every CG loop counts r.r and p.(A p) below the smallest normal float as
// zero: the recursive residual of a system solved to rounding keeps shrinking
// and can underflow, and a reciprocal of such a value is not finite.
constexpr float kCgZero = 0x1p-126f;

// D = 16x16x32 bf16 MFMA, fp32 accumulate.  Lane l supplies A[l%16][8(l/16)..+7],
// B[8(l/16)..+7][l%16] and receives D[4(l/16)..+3][l%16].
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = 16x16x4 fp32 MFMA.  Lane l supplies A[l%16][l/16], B[l/16][l%16] and
// receives D[4(l/16)..+3][l%16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return static_cast<__bf16>(x); }

__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

// Sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane groups of a
// wave).  Every participating lane receives the bitwise-identical result.
// Uses the gfx950 cross-row swaps: permlane16_swap(v, v) yields, in every
// lane, {value of the even 16-lane row, value of the odd row} of its row
// pair; permlane32_swap(v, v) yields {value of lanes 0-31, value of lanes
// 32-63} for the same lane position.  Both sums are formed in the same order
// in every lane.
__device__ __forceinline__ float sum_lane_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over all 64 lanes without LDS traffic: DPP pairings inside each 16-lane
// row (quad xor 1, quad xor 2, half-row mirror, row mirror -- each pairs lanes
// symmetrically, so both partners form the same sum), then the cross-row
// swaps of sum_lane_groups.  Every lane receives the bitwise-identical result.
#define MESA_DPP_ADD(v, ctrl) \
  ((v) + __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(v), (ctrl), 0xF, 0xF, false)))
// Sum over each aligned group of N consecutive lanes (N = 2, 4, ..., 64).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group of 2^k lanes, k >= 1");
  v = MESA_DPP_ADD(v, 0xB1);                          // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (N >= 4) v = MESA_DPP_ADD(v, 0x4E);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) v = MESA_DPP_ADD(v, 0x141);   // row_half_mirror: quad 0 <-> quad 1, quad 2 <-> quad 3
  if constexpr (N >= 16) v = MESA_DPP_ADD(v, 0x140);  // row_mirror: half-row 0 <-> half-row 1
  if constexpr (N >= 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  if constexpr (N == 64) {
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// Load 4 consecutive input elements (fp32 or bf16 storage) as fp32.
template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* base, size_t idx) {
  if constexpr (BF16) {
    const u16x4 u = *reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(base) + idx);
    return f32x4{bf16_to_f32(u[0]), bf16_to_f32(u[1]), bf16_to_f32(u[2]), bf16_to_f32(u[3])};
  } else {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
  } else {
    return static_cast<const float*>(base)[idx];
  }
}

}  // namespace mesa
