// Sparse MLA decode over 352-byte NVFP4 records, gfx950.
//
// What it computes (FlashMLA PR #18 "W4A16 DSA: NVFP4 KV cache format for
// SM100 sparse decode", PR description): for each query row and head, gather
// the top-k token records by slot id (negative = invalid), dequantize them to
// bf16 (NoPE = e2m1 * block scale, RoPE = e4m3), S = scale * Q K^T over the
// 576 dims with bf16 MFMA and fp32 accumulation, softmax with an optional
// per-head sink, O = P V over the 512 NoPE dims, also as bf16 MFMA.
//
// Kernel organisation ("token-stream" kernel, 16 heads per workgroup):
//   * a workgroup owns one query row, one group of 16 heads and one split of
//     the top-k list; its NW waves take 16-token blocks round-robin, each with
//     its own online-softmax state and O accumulator, merged through LDS at
//     the end;
//   * a lane loads the bytes of one token it needs straight from HBM (the
//     permuted scale layout makes a lane's 8 block scales one 8-byte load),
//     dequantizes them into the QK MFMA's A operand registers (K never visits
//     LDS), and stores the NoPE half into a wave-private LDS tile that the PV
//     MFMA reads back transposed (ds_read_b64_tr_b16);
//   * S^T = K Q^T is computed so P lands in the PV MFMA's A-operand layout
//     without any data movement;
//   * P is split into bf16 hi + lo parts (two PV MFMAs), keeping all
//     contractions bf16 while bounding the P rounding error far below the
//     output tolerance;
//   * the running max is only raised (and O rescaled) when a new block
//     exceeds it by more than 2^8, so rescales are rare.
#include <math.h>

#include "combine_math.h"
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

namespace {

constexpr int kVRow = kVDim + 8;            // padded LDS row (bf16 elements)
constexpr float kLazyThreshold = 8.0f;      // log2 units

__device__ __forceinline__ float wave_shfl_xor(float v, int m) { return __shfl_xor(v, m); }

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

struct RawTok {          // the bytes one lane needs of one token record
  u32x2 nope[8];         // blocks 4c+g, c = 0..7
  u32x2 scale;           // scale bytes 8g .. 8g+7  (= blocks 4c+g)
  u32x4 rope;            // RoPE elements 16g .. 16g+15
};

__device__ __forceinline__ void load_tok(RawTok& t, const uint8_t* rec, int g, bool valid) {
  if (valid) {
#pragma unroll
    for (int c = 0; c < 8; c++) t.nope[c] = *reinterpret_cast<const u32x2*>(rec + 32 * c + 8 * g);
    t.scale = *reinterpret_cast<const u32x2*>(rec + kScaleOffset + 8 * g);
    t.rope = *reinterpret_cast<const u32x4*>(rec + kRopeOffset + 16 * g);
  } else {
#pragma unroll
    for (int c = 0; c < 8; c++) t.nope[c] = u32x2{0u, 0u};
    t.scale = u32x2{0u, 0u};
    t.rope = u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace

// Token-stream decode kernel.  Grid: rows * (h_q/16) * splits workgroups of
// 64*NW threads.  Lane l: g = l/16 (lane group), n = l%16.
//   QK (16x16x32): A = K[token n][k-chunk g], B = Q^T[k-chunk g][head n],
//   C = S^T[token 4g+r][head n].  K-step ks < 16 covers NoPE dims
//   16*(4c+g) + 8*(ks&1) + [0,8) with c = ks/2 for lane group g; ks 16, 17
//   cover RoPE dims 16g + 8*(ks-16) + [0,8).  Q is laid out to match.
//   PV (16x16x16): A = P[head n][token 4g+i], B = V[token 4g+i][dv 16nb+n],
//   C = O[head 4g+r][dv 16nb+n].
template <int NW, bool kSplitP>
__global__ void __launch_bounds__(64 * NW)
decode_stream16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vtile[NW][16][kVRow];
  __shared__ float red_m[NW][16];
  __shared__ float red_l[NW][16];
  __shared__ float sh_ms[16];
  __shared__ float sh_lt[16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;

  const int hgroups = a.h_q >> 4;
  int bid = blockIdx.x;
  const int split = bid % a.splits;
  bid /= a.splits;
  const int hg = bid % hgroups;
  const int row = bid / hgroups;
  const int h0 = hg * 16;

  // token range of this split, in whole 16-token blocks
  const int nblk_total = (a.topk + 15) >> 4;
  const int blk_per_split = (nblk_total + a.splits - 1) / a.splits;
  const int blk0 = split * blk_per_split;
  const int blk1 = min(nblk_total, blk0 + blk_per_split);

  // ---- Q^T operand registers (head n, k-chunk g)
  bf16x8 qB[18];
  {
    const uint16_t* qrow = a.q + ((size_t)row * a.h_q + h0 + n) * kQkDim;
#pragma unroll
    for (int ks = 0; ks < 16; ks++) {
      const int d = 16 * (4 * (ks >> 1) + g) + 8 * (ks & 1);
      qB[ks] = *reinterpret_cast<const bf16x8*>(qrow + d);
    }
#pragma unroll
    for (int ks = 16; ks < 18; ks++) {
      const int d = kNopeDim + 16 * g + 8 * (ks - 16);
      qB[ks] = *reinterpret_cast<const bf16x8*>(qrow + d);
    }
  }

  f32x4 acc_o[32];
#pragma unroll
  for (int nb = 0; nb < 32; nb++) acc_o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_use = -INFINITY;   // running max (log2 units) of head n
  float l_part = 0.f;        // this lane's share of the softmax denominator

  const int32_t* idx_row = a.indices + (size_t)row * a.topk;
  uint16_t* vt = &vtile[wave][0][0];

  // prefetch the first block
  int jb = blk0 + wave;
  RawTok cur;
  int32_t cur_idx = -1;
  {
    const int p = jb * 16 + n;
    if (jb < blk1 && p < a.topk) cur_idx = idx_row[p];
    const bool valid = cur_idx >= 0 && (int64_t)cur_idx < a.num_slots;
    load_tok(cur, a.cache + (valid ? a.pa.offset((uint32_t)cur_idx) : 0), g, valid);
  }

  for (; jb < blk1; jb += NW) {
    const bool cur_valid = cur_idx >= 0 && (int64_t)cur_idx < a.num_slots;
    // ---- prefetch the next block of this wave
    RawTok nxt;
    int32_t nxt_idx = -1;
    {
      const int jn = jb + NW;
      const int p = jn * 16 + n;
      if (jn < blk1 && p < a.topk) nxt_idx = idx_row[p];
      const bool valid = nxt_idx >= 0 && (int64_t)nxt_idx < a.num_slots;
      load_tok(nxt, a.cache + (valid ? a.pa.offset((uint32_t)nxt_idx) : 0), g, valid);
    }
    const uint64_t vmask = __ballot(cur_valid);

    // ---- dequantize into K operand registers; NoPE also into the V tile
    const f32x2 s01 = e4m3x2_to_f32<0>(cur.scale.x);
    const f32x2 s23 = e4m3x2_to_f32<1>(cur.scale.x);
    const f32x2 s45 = e4m3x2_to_f32<0>(cur.scale.y);
    const f32x2 s67 = e4m3x2_to_f32<1>(cur.scale.y);
    const float sc[8] = {s01.x, s01.y, s23.x, s23.y, s45.x, s45.y, s67.x, s67.y};
    u32x4 kA[18];
#pragma unroll
    for (int c = 0; c < 8; c++) {
      uint32_t o[4];
      dequant8(cur.nope[c].x, sc[c], o);
      kA[2 * c] = u32x4{o[0], o[1], o[2], o[3]};
      dequant8(cur.nope[c].y, sc[c], o);
      kA[2 * c + 1] = u32x4{o[0], o[1], o[2], o[3]};
    }
    kA[16] = u32x4{e4m3x2_to_bf16x2<0>(cur.rope.x), e4m3x2_to_bf16x2<1>(cur.rope.x),
                   e4m3x2_to_bf16x2<0>(cur.rope.y), e4m3x2_to_bf16x2<1>(cur.rope.y)};
    kA[17] = u32x4{e4m3x2_to_bf16x2<0>(cur.rope.z), e4m3x2_to_bf16x2<1>(cur.rope.z),
                   e4m3x2_to_bf16x2<0>(cur.rope.w), e4m3x2_to_bf16x2<1>(cur.rope.w)};

    // previous block's transposed reads are done before the tile is rewritten
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ks = 0; ks < 16; ks++) {
      const int d = 16 * (4 * (ks >> 1) + g) + 8 * (ks & 1);
      *reinterpret_cast<u32x4*>(vt + n * kVRow + d) = kA[ks];
    }

    // ---- S^T = K Q^T
    f32x4 s_acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ks++)
      s_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kA[ks]), qB[ks],
                                                      s_acc, 0, 0, 0);

    // ---- online softmax for head n over tokens 4g+r
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; r++)
      s[r] = ((vmask >> (4 * g + r)) & 1ull) ? s_acc[r] * a.scale_log2 : -INFINITY;
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    bm = fmaxf(bm, wave_shfl_xor(bm, 16));
    bm = fmaxf(bm, wave_shfl_xor(bm, 32));
    const bool need = bm > m_use + kLazyThreshold;
    if (__any(need)) {
      const float m_new = need ? bm : m_use;
      const float alpha = (m_new == m_use) ? 1.0f : exp2f(m_use - m_new);
      l_part *= alpha;
      m_use = m_new;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; r++) ar[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int nb = 0; nb < 32; nb++)
#pragma unroll
        for (int r = 0; r < 4; r++) acc_o[nb][r] *= ar[r];
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; r++) p[r] = (s[r] == -INFINITY) ? 0.0f : exp2f(s[r] - m_use);
    l_part += (p[0] + p[1]) + (p[2] + p[3]);
    i16x4 p_hi, p_lo;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const uint16_t h = bf16_rne(p[r]);
      p_hi[r] = (short)h;
      if (kSplitP) p_lo[r] = (short)bf16_rne(p[r] - bf16_to_f32(h));
    }

    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // ---- O += P V   (B operand via transposed LDS reads)
    {
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const uint16_t* vb = vt + (4 * g + (n >> 2)) * kVRow + 4 * (n & 3);
#pragma unroll
      for (int nb = 0; nb < 32; nb++) {
        const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + 16 * nb));
        acc_o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_hi, b, acc_o[nb], 0, 0, 0);
        if (kSplitP)
          acc_o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_lo, b, acc_o[nb], 0, 0, 0);
      }
    }

    cur = nxt;
    cur_idx = nxt_idx;
  }

  // ---- merge the NW waves' partial states
  float l_tot = l_part;
  l_tot += wave_shfl_xor(l_tot, 16);
  l_tot += wave_shfl_xor(l_tot, 32);
  if (g == 0) {
    red_m[wave][n] = m_use;
    red_l[wave][n] = l_tot;
  }
  __syncthreads();
  if (threadIdx.x < 16) {              // per-head max and denominator over waves
    const int h = threadIdx.x;
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; w++) ms = fmaxf(ms, red_m[w][h]);
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      const float mw = red_m[w][h];
      lt += (mw == -INFINITY) ? 0.f : exp2f(mw - ms) * red_l[w][h];
    }
    sh_ms[h] = ms;
    sh_lt[h] = lt;
  }
  __syncthreads();
  float wfac[4];                       // this wave's weight for O rows 4g+r
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const float mw = red_m[wave][4 * g + r];
    wfac[r] = (mw == -INFINITY) ? 0.f : exp2f(mw - sh_ms[4 * g + r]);
  }
  // the V tiles are reused as the reduction buffer: [NW][16 heads][256 dv] fp32
  float* redbuf = reinterpret_cast<float*>(&vtile[0][0][0]);
  static_assert(sizeof(vtile) >= NW * 16 * 256 * sizeof(float), "reduction buffer too small");
  const size_t orow_base = ((size_t)row * a.h_q + h0);
  const size_t part_base = ((size_t)split * a.rows + row) * a.h_q + h0;
  for (int half = 0; half < 2; half++) {
    __syncthreads();
#pragma unroll
    for (int nbh = 0; nbh < 16; nbh++) {
      const int nb = half * 16 + nbh;
#pragma unroll
      for (int r = 0; r < 4; r++)
        redbuf[(wave * 16 + 4 * g + r) * 256 + 16 * nbh + n] = acc_o[nb][r] * wfac[r];
    }
    __syncthreads();
    for (int e2 = threadIdx.x; e2 < 16 * 128; e2 += 64 * NW) {
      const int h = e2 >> 7;
      const int dv2 = (e2 & 127) * 2;
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int w = 0; w < NW; w++) {
        v0 += redbuf[(w * 16 + h) * 256 + dv2];
        v1 += redbuf[(w * 16 + h) * 256 + dv2 + 1];
      }
      const float ms = sh_ms[h];
      const float lt = sh_lt[h];
      const int dv = half * 256 + dv2;
      if (a.splits == 1) {
        float denom = lt;
        if (a.sink != nullptr && lt > 0.f)
          denom += exp2f(a.sink[h0 + h] * 1.4426950408889634f - ms);
        const float inv = lt > 0.f ? 1.0f / denom : 0.f;
        const uint32_t pk = (uint32_t)bf16_rne(v0 * inv) | ((uint32_t)bf16_rne(v1 * inv) << 16);
        *reinterpret_cast<uint32_t*>(a.out + (orow_base + h) * kVDim + dv) = pk;
      } else {
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        *reinterpret_cast<f32x2*>(a.o_part + (part_base + h) * kVDim + dv) =
            f32x2{v0 * inv, v1 * inv};
      }
    }
  }
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    const float lt = sh_lt[h];
    const float lse = lt > 0.f ? (sh_ms[h] + log2f(lt)) * 0.6931471805599453f : -INFINITY;
    if (a.splits == 1) a.lse[orow_base + h] = lse;
    else a.lse_part[part_base + h] = lse;
  }
  if (a.splits == 1) return;

  // ---- split-KV: the last split of this (row, head group) to finish merges
  // all splits' partials.  Release the partials device-wide, count, and let
  // the last arrival acquire them; it resets the counter for the next call.
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  uint32_t* counter = a.counters + (size_t)row * hgroups + hg;
  if (threadIdx.x == 0) s_last = (atomicAdd(counter, 1u) == (uint32_t)(a.splits - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int64_t rh0 = (int64_t)row * a.h_q + h0;
  const int64_t part_stride = (int64_t)a.rows * a.h_q;
  for (int e = threadIdx.x; e < 16 * (kVDim / 4); e += 64 * NW) {
    const int h = e / (kVDim / 4);
    combine_chunk4(a.o_part, a.lse_part, a.splits, part_stride, rh0 + h, 4 * (e % (kVDim / 4)),
                   a.sink != nullptr ? a.sink + h0 + h : nullptr, a.out, a.lse);
  }
  if (threadIdx.x == 0) *counter = 0u;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int grid = a.rows * (a.h_q / 16) * a.splits;
  constexpr int NW = 4;
  hipLaunchKernelGGL((decode_stream16_kernel<NW, true>), dim3(grid), dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
