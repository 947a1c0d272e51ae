// Split-KV combine, gfx950: LSE-weighted merge of partial decode results over
// disjoint index subsets, with the per-head attention sink applied once at the
// end.  For partial results (O_i, LSE_i) (O_i sink-free and normalised within
// its subset, LSE_i = ln of its softmax denominator):
//   LSE = ln sum_i exp(LSE_i),  O = sum_i exp(LSE_i - LSE) O_i / (1 + exp(sink - LSE)).
// An all-empty row (every LSE_i = -inf) gives O = 0, LSE = -inf.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

// One 128-thread block per (row, head); thread t owns dv 4t .. 4t+3.
__global__ void __launch_bounds__(128)
combine_kernel(const float* __restrict__ o_part, const float* __restrict__ lse_part,
               int32_t splits, int64_t rows, int32_t h_q, const float* __restrict__ sink,
               uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int64_t rh = blockIdx.x;                  // row * h_q + h
  const int h = (int)(rh % h_q);
  const int64_t stride = rows * (int64_t)h_q;     // elements between splits (per head row)
  float m = -INFINITY;
  for (int s = 0; s < splits; s++) m = fmaxf(m, lse_part[s * stride + rh]);
  const int t = threadIdx.x;
  uint16_t* orow = out + rh * kVDim + 4 * t;
  if (m == -INFINITY) {
    *reinterpret_cast<u32x2*>(orow) = u32x2{0u, 0u};
    if (t == 0) lse[rh] = -INFINITY;
    return;
  }
  float tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; s++) {
    const float ls = lse_part[s * stride + rh];
    const float w = (ls == -INFINITY) ? 0.f : expf(ls - m);
    tot += w;
    const f32x4 v = *reinterpret_cast<const f32x4*>(o_part + (s * stride + rh) * kVDim + 4 * t);
    acc += w * v;
  }
  const float lse_v = m + logf(tot);
  float inv = 1.0f / tot;
  if (sink != nullptr) inv /= (1.0f + expf(sink[h] - lse_v));
  uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.x * inv)) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.y * inv)) << 16);
  uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.z * inv)) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.w * inv)) << 16);
  *reinterpret_cast<u32x2*>(orow) = u32x2{lo, hi};
  if (t == 0) lse[rh] = lse_v;
}

hipError_t launch_combine(const float* o_part, const float* lse_part, int32_t splits,
                          int64_t rows, int32_t h_q, const float* sink, uint16_t* out,
                          float* lse, hipStream_t stream) {
  const int64_t blocks = rows * (int64_t)h_q;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)blocks), dim3(128), 0, stream, o_part,
                     lse_part, splits, rows, h_q, sink, out, lse);
  return hipGetLastError();
}

}  // namespace nvfp4
