// Sparse MLA decode over 352-byte NVFP4 records, gfx950.
//
// What it computes (FlashMLA PR #18 "W4A16 DSA: NVFP4 KV cache format for
// SM100 sparse decode", PR description): for each query row and head, gather
// the top-k token records by slot id (negative = invalid), dequantize them to
// bf16 (NoPE = e2m1 * block scale, RoPE = e4m3), S = scale * Q K^T over the
// 576 dims with bf16 MFMA and fp32 accumulation, softmax with an optional
// per-head sink, O = P V over the 512 NoPE dims, also as bf16 MFMA.
//
// Kernel organisation ("tile" kernel, 16 heads per workgroup, 4 waves):
//   * a workgroup owns one query row, one group of 16 heads and one split of
//     the top-k list, and walks it in 64-token tiles; wave w loads and
//     dequantizes tokens [16w, 16w+16) of each tile;
//   * a lane loads the bytes of one token it needs straight from HBM (the
//     permuted scale layout makes a lane's 8 block scales one 8-byte load),
//     dequantizes them into the QK MFMA's A operand registers (K never visits
//     LDS) and writes the NoPE half to the shared V tile;
//   * S^T = K Q^T per wave; the per-head tile maximum is exchanged through
//     LDS so every wave applies the same running max; P (bf16 hi + lo parts)
//     goes to a shared P tile;
//   * wave w accumulates O[16 heads, dv 128w .. 128w+127] over all 64 tokens
//     of the tile (V read back with ds_read_b64_tr_b16), so the O accumulator
//     is 32 registers per lane and two workgroups fit per CU;
//   * indices are prefetched two tiles ahead and token bytes one tile ahead;
//   * the running max is only raised (and O rescaled) when a tile exceeds it
//     by more than 2^8, so rescales are rare;
//   * P is split into bf16 hi + lo parts (two PV MFMAs): every contraction
//     stays bf16 while P's rounding error stays far below the tolerance.
// With several splits, the last split of a (row, head group) to finish merges
// the partial results (LSE-weighted) inside the same launch.
#include <math.h>

#include "combine_math.h"
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

namespace {

constexpr int kWaves = 4;
constexpr int kTile = 16 * kWaves;          // tokens per tile
constexpr int kVRow = kVDim + 8;            // padded LDS row of the V tile (bf16)
constexpr int kPRow = kTile + 8;            // padded LDS row of the P tile (bf16)
constexpr float kLazyThreshold = 8.0f;      // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m); }

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// Two fp32 -> packed bf16 (round to nearest even), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Workgroup barrier ordering LDS accesses only.  __syncthreads() also
// fences global memory, which makes every wave wait for its outstanding
// global loads -- the token bytes prefetched for the next tile -- at each
// barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 2^x with the hardware approximation (no denormal range reduction: inputs
// here are softmax exponents <= 8, and results below 2^-126 are negligible
// weights that may flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct RawTok {          // the bytes one lane needs of one token record
  u32x2 nope[8];         // NoPE blocks 4c+g, c = 0..7
  u32x2 scale;           // scale bytes 8g .. 8g+7 (= blocks 4c+g)
  u32x4 rope;            // RoPE elements 16g .. 16g+15
};

// Unconditional loads (uniform control flow keeps the prefetch in flight:
// after a divergent load the compiler can only wait for every outstanding
// load).  Invalid tokens read record 0, which always exists; their scale
// bytes are zeroed when consumed (see scale_or_zero), so their NoPE values
// are exact zeros and cannot carry NaN into P V, and their scores are masked.
__device__ __forceinline__ void load_tok(RawTok& t, const uint8_t* rec, int g) {
#pragma unroll
  for (int c = 0; c < 8; c++) t.nope[c] = *reinterpret_cast<const u32x2*>(rec + 32 * c + 8 * g);
  t.scale = *reinterpret_cast<const u32x2*>(rec + kScaleOffset + 8 * g);
  t.rope = *reinterpret_cast<const u32x4*>(rec + kRopeOffset + 16 * g);
}

__device__ __forceinline__ int32_t load_idx(const int32_t* idx_row, int p, int t1) {
  const int32_t v = idx_row[min(p, max(t1 - 1, 0))];   // in bounds: topk >= 1
  return p < t1 ? v : -1;
}

__device__ __forceinline__ bool idx_valid(int32_t idx, int64_t num_slots) {
  return idx >= 0 && (int64_t)idx < num_slots;
}

__device__ __forceinline__ const uint8_t* rec_ptr(const DecodeArgs& a, int32_t idx) {
  return a.cache + (idx_valid(idx, a.num_slots) ? a.pa.offset((uint32_t)idx) : 0);
}

}  // namespace

// Lane l of wave w: g = l/16 (lane group), n = l%16.
//   QK (16x16x32): A = K[token 16w+n][k-chunk g], B = Q^T[k-chunk g][head n],
//   C = S^T[token 16w+4g+r][head n].  K-step ks < 16 covers NoPE dims
//   16*(4c+g) + 8*(ks&1) + [0,8) with c = ks/2 for lane group g (so a lane's
//   blocks are {4c+g}, whose scales are the contiguous bytes 8g..8g+7);
//   ks 16, 17 cover RoPE dims 16g + 8*(ks-16) + [0,8).  Q is laid out to match.
//   PV (16x16x32): A = P[head n][token 32ks+8g+i], B = V[token 32ks+8g+i][dv],
//   C = O[head 4g+r][dv 128w + 16nb + n].
template <bool kSplitP>
__global__ void __launch_bounds__(64 * kWaves, 2)
decode_tile16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vtile[kTile][kVRow];
  __shared__ __attribute__((aligned(16))) uint16_t ptile_hi[16][kPRow];
  __shared__ __attribute__((aligned(16))) uint16_t ptile_lo[16][kPRow];
  __shared__ float tmax[kWaves][16];
  __shared__ float lsum[kWaves][16];
  __shared__ int s_last;

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

  // token range of this split, in whole tiles
  const int ntiles_total = (a.topk + kTile - 1) / kTile;
  const int tiles_per_split = (ntiles_total + a.splits - 1) / a.splits;
  const int tile0 = split * tiles_per_split;
  const int tile1 = min(ntiles_total, tile0 + tiles_per_split);
  const int t_end = min(a.topk, tile1 * kTile);       // first token past the split
  const int32_t* idx_row = a.indices + (size_t)row * a.topk;
  const int my_tok = 16 * wave + n;                    // this lane's token within a tile

  // ---- Q^T operand registers (head n, k-chunk g)
  bf16x8 qB[18];
  {
    const uint16_t* qrow = a.q + ((size_t)row * a.h_q + h0 + n) * kQkDim;
#pragma unroll
    for (int ks = 0; ks < 16; ks++)
      qB[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * (4 * (ks >> 1) + g) + 8 * (ks & 1));
#pragma unroll
    for (int ks = 16; ks < 18; ks++)
      qB[ks] = *reinterpret_cast<const bf16x8*>(qrow + kNopeDim + 16 * g + 8 * (ks - 16));
  }

  f32x4 acc_o[8];
#pragma unroll
  for (int nb = 0; nb < 8; nb++) acc_o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running max (log2 units) of head n (for P) and of heads 4g+r (O rows);
  // every wave derives them from the same LDS values, so they agree
  float m_n = -INFINITY;
  float m_r[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float l_part = 0.f;          // this lane's share of head n's denominator

  // ---- prologue: indices of tiles 0 and 1, token bytes of tile 0
  int tile = tile0;
  int32_t idx_cur = load_idx(idx_row, tile * kTile + my_tok, t_end);
  int32_t idx_nxt = load_idx(idx_row, (tile + 1) * kTile + my_tok, t_end);
  RawTok cur;
  load_tok(cur, rec_ptr(a, idx_cur), g);

  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  // One tile step.  `cur` holds this lane's bytes of tile t, `nxt` receives
  // tile t+1's; the loop below alternates the two buffers so the prefetched
  // bytes are never copied.
  auto step = [&](RawTok& cur, RawTok& nxt, int t) {
    // ---- prefetch: indices two tiles ahead, token bytes one tile ahead
    const int32_t idx_nn = load_idx(idx_row, (t + 2) * kTile + my_tok, t_end);
    load_tok(nxt, rec_ptr(a, idx_nxt), g);
    const bool cur_valid = idx_valid(idx_cur, a.num_slots);
    const uint64_t vmask = __ballot(cur_valid);

    // ---- dequantize this wave's 16 tokens into K operand registers
    const uint32_t scx = cur_valid ? cur.scale.x : 0u;
    const uint32_t scy = cur_valid ? cur.scale.y : 0u;
    const f32x2 s01 = e4m3x2_to_f32<0>(scx);
    const f32x2 s23 = e4m3x2_to_f32<1>(scx);
    const f32x2 s45 = e4m3x2_to_f32<0>(scy);
    const f32x2 s67 = e4m3x2_to_f32<1>(scy);
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

    // all waves are done reading the previous tile's V and P
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < 16; ks++)
      *reinterpret_cast<u32x4*>(&vtile[my_tok][16 * (4 * (ks >> 1) + g) + 8 * (ks & 1)]) = kA[ks];

    // ---- S^T = K Q^T for this wave's tokens
    f32x4 s_acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ks++)
      s_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kA[ks]), qB[ks],
                                                      s_acc, 0, 0, 0);
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; r++)
      s[r] = ((vmask >> (4 * g + r)) & 1ull) ? s_acc[r] * a.scale_log2 : -INFINITY;
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    bm = fmaxf(bm, shfl_xor(bm, 16));
    bm = fmaxf(bm, shfl_xor(bm, 32));
    if (g == 0) tmax[wave][n] = bm;
    lds_barrier();                        // every wave's maxima posted

    // ---- running max update (same rule in every wave), lazy O rescale
    float tm_n = tmax[0][n];
#pragma unroll
    for (int w = 1; w < kWaves; w++) tm_n = fmaxf(tm_n, tmax[w][n]);
    if (tm_n > m_n + kLazyThreshold) {
      l_part *= fast_exp2(m_n - tm_n);    // m_n = -inf gives 0 (l_part is 0 then)
      m_n = tm_n;
    }
    bool any_rescale = false;
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      float tm = tmax[0][4 * g + r];
#pragma unroll
      for (int w = 1; w < kWaves; w++) tm = fmaxf(tm, tmax[w][4 * g + r]);
      alpha[r] = 1.0f;
      if (tm > m_r[r] + kLazyThreshold) {
        alpha[r] = fast_exp2(m_r[r] - tm);
        m_r[r] = tm;
        any_rescale = true;
      }
    }
    if (__any(any_rescale)) {
#pragma unroll
      for (int nb = 0; nb < 8; nb++)
#pragma unroll
        for (int r = 0; r < 4; r++) acc_o[nb][r] *= alpha[r];
    }

    // ---- P for this wave's tokens -> P tile (bf16 hi and lo parts)
    const float m_safe = (m_n == -INFINITY) ? 0.f : m_n;   // s = -inf -> p = 0
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; r++) p[r] = fast_exp2(s[r] - m_safe);
    l_part += (p[0] + p[1]) + (p[2] + p[3]);
    {
      const uint32_t hi01 = pack_bf16x2(p[0], p[1]);
      const uint32_t hi23 = pack_bf16x2(p[2], p[3]);
      const int col = 16 * wave + 4 * g;
      *reinterpret_cast<u32x2*>(&ptile_hi[n][col]) = u32x2{hi01, hi23};
      if (kSplitP) {
        const uint32_t lo01 = pack_bf16x2(p[0] - __uint_as_float(hi01 << 16),
                                          p[1] - __uint_as_float(hi01 & 0xFFFF0000u));
        const uint32_t lo23 = pack_bf16x2(p[2] - __uint_as_float(hi23 << 16),
                                          p[3] - __uint_as_float(hi23 & 0xFFFF0000u));
        *reinterpret_cast<u32x2*>(&ptile_lo[n][col]) = u32x2{lo01, lo23};
      }
    }
    lds_barrier();                        // P and V tiles complete

    // ---- O[:, 128w .. 128w+127] += P V over the tile's 64 tokens
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const int t8 = 32 * ks + 8 * g;
      const bf16x8 pa_hi = *reinterpret_cast<const bf16x8*>(&ptile_hi[n][t8]);
      bf16x8 pa_lo;
      if (kSplitP) pa_lo = *reinterpret_cast<const bf16x8*>(&ptile_lo[n][t8]);
      const uint16_t* vb0 = &vtile[t8 + (n >> 2)][128 * wave + 4 * (n & 3)];
      const uint16_t* vb1 = vb0 + 4 * kVRow;
#pragma unroll
      for (int nb = 0; nb < 8; nb++) {
        const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb0 + 16 * nb));
        const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb1 + 16 * nb));
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc_o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, bv, acc_o[nb], 0, 0, 0);
        if (kSplitP)
          acc_o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, bv, acc_o[nb], 0, 0, 0);
      }
    }
    idx_cur = idx_nxt;
    idx_nxt = idx_nn;
  };

  RawTok other;
  for (; tile + 1 < tile1; tile += 2) {
    step(cur, other, tile);
    step(other, cur, tile + 1);
  }
  if (tile < tile1) step(cur, other, tile);

  // ---- epilogue: denominators over lanes and waves, normalise, write
  float lt = l_part;
  lt += shfl_xor(lt, 16);
  lt += shfl_xor(lt, 32);
  __syncthreads();
  if (g == 0) lsum[wave][n] = lt;
  if (wave == 0 && g == 0) tmax[0][n] = m_n;      // the agreed running max of head n
  __syncthreads();
  const size_t orow = (size_t)row * a.h_q + h0;
  const size_t prow = ((size_t)split * a.rows + row) * a.h_q + h0;
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int h = 4 * g + r;
    const float l = lsum[0][h] + lsum[1][h] + lsum[2][h] + lsum[3][h];
    float denom = l;
    if (a.splits == 1 && a.sink != nullptr && l > 0.f)
      denom += exp2f(a.sink[h0 + h] * kLog2e - tmax[0][h]);
    inv[r] = l > 0.f ? 1.0f / denom : 0.f;
  }
#pragma unroll
  for (int nb = 0; nb < 8; nb++) {
    const int dv = 128 * wave + 16 * nb + n;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int h = 4 * g + r;
      const float v = acc_o[nb][r] * inv[r];
      if (a.splits == 1)
        a.out[(orow + h) * kVDim + dv] = (uint16_t)bf16_rne(v);
      else
        a.o_part[(prow + h) * kVDim + dv] = v;
    }
  }
  if (wave == 0 && g == 0) {
    const float l = lsum[0][n] + lsum[1][n] + lsum[2][n] + lsum[3][n];
    const float lse = l > 0.f ? (m_n + log2f(l)) * kLn2 : -INFINITY;
    if (a.splits == 1) a.lse[orow + n] = lse;
    else a.lse_part[prow + n] = lse;
  }
  if (a.splits == 1) return;

  // ---- split-KV: the last split of this (row, head group) to finish merges
  // all splits' partials.  Release the partials device-wide, count, and let
  // the last arrival acquire them; it resets the counter for the next call.
  // The workgroup barrier completes every wave's partial stores (to this
  // XCD's L2); one thread then releases them device-wide, counts, and on the
  // last arrival acquires the other splits' partials for the whole CU.
  __syncthreads();
  uint32_t* counter = a.counters + (size_t)row * hgroups + hg;
  if (threadIdx.x == 0) {
    __threadfence();
    const bool last = atomicAdd(counter, 1u) == (uint32_t)(a.splits - 1);
    if (last) __threadfence();
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  const int64_t rh0 = (int64_t)row * a.h_q + h0;
  const int64_t part_stride = (int64_t)a.rows * a.h_q;
  for (int e = threadIdx.x; e < 16 * (kVDim / 4); e += 64 * kWaves) {
    const int h = e / (kVDim / 4);
    combine_chunk4(a.o_part, a.lse_part, a.splits, part_stride, rh0 + h, 4 * (e % (kVDim / 4)),
                   a.sink != nullptr ? a.sink + h0 + h : nullptr, a.out, a.lse);
  }
  if (threadIdx.x == 0) *counter = 0u;
}

bool decode_uses_w32(int32_t h_q) { return h_q % 32 == 0; }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  if (decode_uses_w32(a.h_q)) return launch_decode_w32(a, stream);
  const int grid = a.rows * (a.h_q / 16) * a.splits;
  hipLaunchKernelGGL((decode_tile16_kernel<true>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
