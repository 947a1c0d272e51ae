// Split-KV combine, gfx950: LSE-weighted merge of partial decode results over
// disjoint index subsets, with the per-head attention sink applied once at the
// end.  For partial results (O_i, LSE_i) (O_i sink-free and normalised within
// its subset, LSE_i = ln of its softmax denominator):
//   LSE = ln sum_i exp(LSE_i),  O = sum_i exp(LSE_i - LSE) O_i / (1 + exp(sink - LSE)).
// An all-empty row (every LSE_i = -inf) gives O = 0, LSE = -inf; a NaN LSE_i
// gives a NaN row.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

namespace {

typedef _Float16 f16x8c __attribute__((ext_vector_type(8)));

// Eight consecutive partial values as fp32.
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const f16x8c a = *reinterpret_cast<const f16x8c*>(p);
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = (float)a[i];
}

constexpr int kWavesC = 4;

}  // namespace

// One wave per (row, head); lane l owns output dims 8l .. 8l+7.  Splits are
// read four at a time (their LSEs and partials in flight together) and merged
// against a running maximum of the LSEs, rescaling when it rises.  T is the
// partial type: fp32 for the standalone export and the 16-head decode, fp16
// for the 32-head decode's own partials.
//
// Workgroups are dealt to the 8 XCDs round-robin by blockIdx.  The decode
// kernels run every workgroup of row r on XCD r % 8 when the row count is a
// multiple of 8, and with xcd_rows the blocks of row r go there too.  The
// partials are not found in that XCD's L2 after the launch boundary, though:
// by rocprofv3 FETCH_SIZE the combine fetches all of them from beyond L2.
template <typename T>
__global__ void __launch_bounds__(64 * kWavesC)
combine_kernel(const T* __restrict__ o_part, const float* __restrict__ lse_part,
               int32_t splits, int64_t rh_total, int32_t h_q, int32_t xcd_rows,
               const float* __restrict__ sink, uint16_t* __restrict__ out,
               float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t rh;
  if (xcd_rows) {
    const int64_t bpr = h_q / kWavesC;               // blocks per row
    const int64_t i = blockIdx.x >> 3;
    const int64_t row = (blockIdx.x & 7) + 8 * (i / bpr);
    rh = row * h_q + kWavesC * (i % bpr) + w;
  } else {
    rh = (int64_t)blockIdx.x * kWavesC + w;
  }
  if (rh >= rh_total) return;
  const int dv0 = 8 * lane;
  uint16_t* orow = out + rh * kVDim + dv0;
  // running maximum of the LSEs with rescaling, so each group's LSE and
  // partial loads are issued together
  float m = -INFINITY, tot = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // a NaN partial LSE (a decode workgroup that marked its result as failed)
  // makes the merged row NaN rather than being skipped by the maxima
  bool nan_seen = false;
  for (int s0 = 0; s0 < splits; s0 += 4) {
    float ls[4];
    float v[4][8];
    // the four loads go out unconditionally (a load under a branch would
    // wait for the one before it): past the last split they re-read it and
    // its weight is zero
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int s = min(s0 + u, splits - 1);
      ls[u] = lse_part[s * rh_total + rh];
      load8(o_part + (s * rh_total + rh) * kVDim + dv0, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) ls[u] = s0 + u < splits ? ls[u] : -INFINITY;
    nan_seen |= (ls[0] != ls[0]) | (ls[1] != ls[1]) | (ls[2] != ls[2]) | (ls[3] != ls[3]);
    // (while every LSE so far is -inf, mn = m = -inf and every weight below
    // is zero: no skip, whose branch would hold the loads above behind the
    // LSE loads)
    const float mn = fmaxf(m, fmaxf(fmaxf(ls[0], ls[1]), fmaxf(ls[2], ls[3])));
    if (mn != m) {
      const float sc = (m == -INFINITY) ? 0.f : expf(m - mn);
      tot *= sc;
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] *= sc;
      m = mn;
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const float w = (ls[u] == -INFINITY) ? 0.f : expf(ls[u] - m);
      tot += w;
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] = __builtin_fmaf(w, v[u][i], acc[i]);
    }
  }
  if (nan_seen) {
    const float qnan = __builtin_nanf("");
    const uint32_t nb = 0x7FC07FC0u;               // two bf16 quiet NaNs
    reinterpret_cast<u32x2*>(orow)[0] = u32x2{nb, nb};
    reinterpret_cast<u32x2*>(orow)[1] = u32x2{nb, nb};
    if (lane == 0) lse[rh] = qnan;
    return;
  }
  if (m == -INFINITY) {
    reinterpret_cast<u32x2*>(orow)[0] = u32x2{0u, 0u};
    reinterpret_cast<u32x2*>(orow)[1] = u32x2{0u, 0u};
    if (lane == 0) lse[rh] = -INFINITY;
    return;
  }
  const float lse_v = m + logf(tot);
  float inv = 1.0f / tot;
  if (sink != nullptr) inv /= (1.0f + expf(sink[rh % h_q] - lse_v));
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; i++)
    b[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[2 * i] * inv)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[2 * i + 1] * inv)) << 16);
  reinterpret_cast<u32x2*>(orow)[0] = u32x2{b[0], b[1]};
  reinterpret_cast<u32x2*>(orow)[1] = u32x2{b[2], b[3]};
  if (lane == 0) lse[rh] = lse_v;
}

template <typename T>
static hipError_t launch_combine_t(const T* o_part, const float* lse_part, int32_t splits,
                                   int64_t rows, int32_t h_q, const float* sink, uint16_t* out,
                                   float* lse, hipStream_t stream) {
  const int64_t rh_total = rows * (int64_t)h_q;
  if (rh_total == 0) return hipSuccess;
  const int64_t blocks = (rh_total + kWavesC - 1) / kWavesC;
  // XCD-matched placement needs whole rows per block and rows in eights
  const int32_t xcd_rows = (rows % 8 == 0 && h_q % kWavesC == 0) ? 1 : 0;
  hipLaunchKernelGGL(combine_kernel<T>, dim3((uint32_t)blocks), dim3(64 * kWavesC), 0, stream,
                     o_part, lse_part, splits, rh_total, h_q, xcd_rows, sink, out, lse);
  return hipGetLastError();
}

hipError_t launch_combine(const float* o_part, const float* lse_part, int32_t splits,
                          int64_t rows, int32_t h_q, const float* sink, uint16_t* out,
                          float* lse, hipStream_t stream) {
  return launch_combine_t(o_part, lse_part, splits, rows, h_q, sink, out, lse, stream);
}

hipError_t launch_combine_f16(const uint16_t* o_part, const float* lse_part, int32_t splits,
                              int64_t rows, int32_t h_q, const float* sink, uint16_t* out,
                              float* lse, hipStream_t stream) {
  return launch_combine_t(o_part, lse_part, splits, rows, h_q, sink, out, lse, stream);
}

}  // namespace nvfp4
