// Split-KV combine, gfx950: LSE-weighted merge of partial decode results over
// disjoint index subsets, with the per-head attention sink applied once at the
// end.  For partial results (O_i, LSE_i) (O_i sink-free and normalised within
// its subset, LSE_i = ln of its softmax denominator):
//   LSE = ln sum_i exp(LSE_i),  O = sum_i exp(LSE_i - LSE) O_i / (1 + exp(sink - LSE)).
// An all-empty row (every LSE_i = -inf) gives O = 0, LSE = -inf.
#include <math.h>

#include "combine_math.h"
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
  combine_chunk4(o_part, lse_part, splits, rows * (int64_t)h_q, rh, 4 * threadIdx.x,
                 sink != nullptr ? sink + h : nullptr, out, lse);
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
