// LSE-weighted merge of split-KV partial results for one (row, head) and four
// consecutive output dims, shared by the standalone combine kernel and the
// decode kernel's in-kernel merge.  For partials (O_i, LSE_i) over disjoint
// index subsets (O_i sink-free, normalised within its subset, LSE_i natural
// log, -inf for an empty subset):
//   LSE = ln sum_i exp(LSE_i),  O = sum_i exp(LSE_i - LSE) O_i / (1 + exp(sink - LSE)),
// and an all-empty row gives O = 0, LSE = -inf.
#pragma once

#include <math.h>

#include "device_common.h"

namespace nvfp4 {

// o_part [splits][stride rows*heads][512] fp32, lse_part [splits][stride];
// rh = row*heads + head; writes out[rh][dv0..dv0+3] (bf16) and, for dv0 == 0,
// lse[rh].
__device__ __forceinline__ void combine_chunk4(const float* o_part, const float* lse_part,
                                               int splits, int64_t stride, int64_t rh, int dv0,
                                               const float* sink_h, uint16_t* out, float* lse) {
  float m = -INFINITY;
  for (int s = 0; s < splits; s++) m = fmaxf(m, lse_part[s * stride + rh]);
  uint16_t* orow = out + rh * kVDim + dv0;
  if (m == -INFINITY) {
    *reinterpret_cast<u32x2*>(orow) = u32x2{0u, 0u};
    if (dv0 == 0) lse[rh] = -INFINITY;
    return;
  }
  float tot = 0.f;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int s = 0; s < splits; s++) {
    const float ls = lse_part[s * stride + rh];
    const float w = (ls == -INFINITY) ? 0.f : expf(ls - m);
    tot += w;
    const f32x4 v = *reinterpret_cast<const f32x4*>(o_part + (s * stride + rh) * kVDim + dv0);
    a0 += w * v.x;
    a1 += w * v.y;
    a2 += w * v.z;
    a3 += w * v.w;
  }
  const float lse_v = m + logf(tot);
  float inv = 1.0f / tot;
  if (sink_h != nullptr) inv /= (1.0f + expf(*sink_h - lse_v));
  const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(a0 * inv)) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(a1 * inv)) << 16);
  const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(a2 * inv)) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(a3 * inv)) << 16);
  *reinterpret_cast<u32x2*>(orow) = u32x2{lo, hi};
  if (dv0 == 0) lse[rh] = lse_v;
}

}  // namespace nvfp4
