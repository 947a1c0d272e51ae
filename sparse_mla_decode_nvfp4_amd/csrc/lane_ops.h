// Cross-lane steps shared by the decode kernels whose QK product leaves a
// lane (n, g) of a wave with heads n and 16 + n of a 32-head group (two
// 16x16 output blocks): per-head maxima and sums over the four 16-lane rows.
// gfx950.
#pragma once

#include "device_common.h"

namespace nvfp4 {

// V tile swizzle of the 32-head kernels (rows of 16-byte chunks, one row
// per token): chunk j of row t lives at chunk j ^ vswz_p(t), within its
// 256-byte segment.  Row writes of 16 lanes and the transposed reads of the
// PV operands are then free of bank conflicts.
__device__ __forceinline__ int vswz_p(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

// Lane-row swaps (VALU): permlane16_swap(a, b) exchanges the odd 16-lane
// rows of a with the even rows of b; permlane32_swap(a, b) exchanges the
// upper 32 lanes of a with the lower 32 of b.

// max(a, b) as one v_max_f32: written as an instruction because the
// compiler otherwise canonicalises both lane-swapped operands first (two
// extra VALU ops per use).  Scores are finite or -inf, never NaN.
__device__ __forceinline__ float fmax_p(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Per-head maximum (max_blocks) or sum (sum_blocks) over the four 16-lane
// rows: x0, x1 hold this lane's block-0 and block-1 values (heads n and
// 16+n); both totals come back in every lane.  The first, two-source swap
// reduces the two blocks together (even rows then carry block 0, odd rows
// block 1); the last swap hands each lane both totals.
__device__ __forceinline__ void max_blocks(float& x0, float& x1) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  const float t = fmax_p(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  const float u = fmax_p(__uint_as_float(b[0]), __uint_as_float(b[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(u), false, false);
  x0 = __uint_as_float(c[0]);
  x1 = __uint_as_float(c[1]);
}
__device__ __forceinline__ void sum_blocks(float& x0, float& x1) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  const float t = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  const float u = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(u), false, false);
  x0 = __uint_as_float(c[0]);
  x1 = __uint_as_float(c[1]);
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

}  // namespace nvfp4
