// Sparse MLA decode for many heads (h_q a multiple of 64), gfx950.
//
// Same computation as decode.hip (FlashMLA PR #18 "W4A16 DSA: NVFP4 KV cache
// format for SM100 sparse decode", PR description: gather top-k NVFP4 token
// records, dequantize to bf16, S = scale * Q K^T over 576 dims, softmax with an
// optional per-head sink, O = P V over 512 dims, bf16 MFMA with fp32
// accumulation), organised for head counts where the matrix work dominates:
//
//   * a workgroup owns one query row, 64 heads and one split of the top-k
//     list; every token is dequantized once and shared by all 64 heads;
//   * the four waves produce 64-token tiles of dequantized bf16 K/V (576 dims
//     per token) into a double-buffered LDS tile: wave w loads and dequantizes
//     tokens [16w, 16w+16) of tile t+1 while all waves consume tile t, with one
//     barrier per tile;
//   * wave w owns heads [16w, 16w+16): QK (S^T = K Q^T, K read from LDS, Q^T
//     in registers), online softmax with no cross-wave exchange, and PV with P
//     taken straight from the S^T accumulators and V read back transposed
//     (ds_read_b64_tr_b16);
//   * the LDS tile is XOR-swizzled in 16-byte chunks (chunk j of row t lives
//     at chunk j ^ s(t mod 8)) so row writes, QK row reads and transposed PV
//     reads are free of bank conflicts;
//   * P is split into bf16 hi + lo parts (two PV MFMAs) and the running max
//     is raised lazily, as in decode.hip.
// With several splits, each writes its sink-free partial O and LSE and the
// combine kernel merges them.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

namespace {

constexpr int kWavesH = 4;
constexpr int kTileH = 64;                      // tokens per tile
constexpr int kRowBytes = kQkDim * 2;           // 1152 B per token row (72 chunks)
constexpr int kTileBytes = kTileH * kRowBytes;  // 72 KB
constexpr float kLazyH = 8.0f;
constexpr float kLog2eH = 1.4426950408889634f;
constexpr float kLn2H = 0.6931471805599453f;

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Swizzle of row t: chunk j of row t is stored at chunk j ^ swz(t).  swz
// only depends on t mod 8 and only changes the low 3 bits of j, so an access
// pattern needs a few per-lane base addresses plus compile-time offsets.
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// Byte offset, within a tile, of 16-byte chunk 8*hi8 + lo8 (lo8 < 8) of row t.
__device__ __forceinline__ uint32_t chunk_off(int t, int hi8, int lo8) {
  return (uint32_t)(t * kRowBytes + (hi8 << 7) + ((lo8 ^ swz(t)) << 4));
}

struct RawTokH {
  u32x2 nope[8];
  u32x2 scale;
  u32x4 rope;
};

__device__ __forceinline__ void load_tok_h(RawTokH& t, const uint8_t* rec, int g) {
#pragma unroll
  for (int c = 0; c < 8; c++) t.nope[c] = *reinterpret_cast<const u32x2*>(rec + 32 * c + 8 * g);
  t.scale = *reinterpret_cast<const u32x2*>(rec + kScaleOffset + 8 * g);
  t.rope = *reinterpret_cast<const u32x4*>(rec + kRopeOffset + 16 * g);
}

__device__ __forceinline__ void lds_barrier_h() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace

// Lane l of wave w: g = l/16, n = l%16.
//   Producer: lane (n, g) handles token 16w+n of a tile: NoPE blocks {4c+g}
//   (scale bytes 8g..8g+7 of the record, one 8-byte load), RoPE dims
//   16g..16g+15.
//   QK (16x16x32), token block j of the tile: A = K[token 16j+n][k-chunk g],
//   B = Q^T[k-chunk g][head 16w+n], C = S^T[token 16j+4g+r][head 16w+n].  The
//   k-steps use the same dim permutation as decode.hip.
//   PV (16x16x32), k-step ks: A = P[head n][k 8g+i] with k 8g+i standing for
//   token 32ks + 16(i/4) + 4g + (i%4) (exactly the S^T values this lane
//   holds), B = V[same tokens][dv 16nb+n], C = O[head 4g+r][dv 16nb+n].
template <bool kSplitP>
__global__ void __launch_bounds__(64 * kWavesH, 1)
decode_hsplit_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* tiles = smem;                                        // 2 x 72 KB
  uint32_t* vmask_lds = reinterpret_cast<uint32_t*>(smem + 2 * kTileBytes);   // [2][4]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;

  const int hgroups = a.h_q >> 6;
  int bid = blockIdx.x;
  const int split = bid % a.splits;
  bid /= a.splits;
  const int hg = bid % hgroups;
  const int row = bid / hgroups;
  const int hw0 = hg * 64 + 16 * wave;          // first head of this wave

  const int ntiles_total = (a.topk + kTileH - 1) / kTileH;
  const int tiles_per_split = (ntiles_total + a.splits - 1) / a.splits;
  const int tile0 = split * tiles_per_split;
  const int tile1 = min(ntiles_total, tile0 + tiles_per_split);
  const int t_end = min(a.topk, tile1 * kTileH);
  const int32_t* idx_row = a.indices + (size_t)row * a.topk;
  const int my_tok = 16 * wave + n;

  // ---- Q^T operand registers (head hw0+n, k-chunk g)
  bf16x8 qB[18];
  {
    const uint16_t* qrow = a.q + ((size_t)row * a.h_q + hw0 + n) * kQkDim;
#pragma unroll
    for (int ks = 0; ks < 16; ks++)
      qB[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * (4 * (ks >> 1) + g) + 8 * (ks & 1));
#pragma unroll
    for (int ks = 16; ks < 18; ks++)
      qB[ks] = *reinterpret_cast<const bf16x8*>(qrow + kNopeDim + 16 * g + 8 * (ks - 16));
  }

  f32x4 acc_o[32];
#pragma unroll
  for (int nb = 0; nb < 32; nb++) acc_o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_use = -INFINITY;     // running max (log2 units) of head hw0+n
  float l_part = 0.f;

  auto load_idx = [&](int p) -> int32_t {
    const int32_t v = idx_row[min(p, max(t_end - 1, 0))];
    return p < t_end ? v : -1;
  };
  auto valid = [&](int32_t idx) { return idx >= 0 && (int64_t)idx < a.num_slots; };
  auto rec_of = [&](int32_t idx) {
    return a.cache + (valid(idx) ? a.pa.offset((uint32_t)idx) : 0);
  };

  // Producer: dequantize this lane's token bytes into tile buffer `buf`.
  auto produce = [&](const RawTokH& raw, int32_t idx, int buf) {
    const bool v = valid(idx);
    const uint32_t scx = v ? raw.scale.x : 0u;
    const uint32_t scy = v ? raw.scale.y : 0u;
    const f32x2 s01 = e4m3x2_to_f32<0>(scx);
    const f32x2 s23 = e4m3x2_to_f32<1>(scx);
    const f32x2 s45 = e4m3x2_to_f32<0>(scy);
    const f32x2 s67 = e4m3x2_to_f32<1>(scy);
    const float sc[8] = {s01.x, s01.y, s23.x, s23.y, s45.x, s45.y, s67.x, s67.y};
    uint8_t* p0 = tiles + buf * kTileBytes + chunk_off(my_tok, 0, 2 * g);       // chunk 8c+2g
    uint8_t* p1 = tiles + buf * kTileBytes + chunk_off(my_tok, 0, 2 * g + 1);   // chunk 8c+2g+1
#pragma unroll
    for (int c = 0; c < 8; c++) {
      uint32_t o[4];
      dequant8(raw.nope[c].x, sc[c], o);
      *reinterpret_cast<u32x4*>(p0 + 128 * c) = u32x4{o[0], o[1], o[2], o[3]};
      dequant8(raw.nope[c].y, sc[c], o);
      *reinterpret_cast<u32x4*>(p1 + 128 * c) = u32x4{o[0], o[1], o[2], o[3]};
    }
    *reinterpret_cast<u32x4*>(p0 + 1024) =
        u32x4{e4m3x2_to_bf16x2<0>(raw.rope.x), e4m3x2_to_bf16x2<1>(raw.rope.x),
              e4m3x2_to_bf16x2<0>(raw.rope.y), e4m3x2_to_bf16x2<1>(raw.rope.y)};
    *reinterpret_cast<u32x4*>(p1 + 1024) =
        u32x4{e4m3x2_to_bf16x2<0>(raw.rope.z), e4m3x2_to_bf16x2<1>(raw.rope.z),
              e4m3x2_to_bf16x2<0>(raw.rope.w), e4m3x2_to_bf16x2<1>(raw.rope.w)};
    const uint64_t m = __ballot(v);
    if (lane == 0) vmask_lds[buf * 4 + wave] = (uint32_t)(m & 0xFFFFu);
  };

  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

  // Consumer: QK, softmax and PV of tile buffer `buf` for this wave's heads.
  auto consume = [&](int buf) {
    const uint8_t* tb = tiles + buf * kTileBytes;
    const uint64_t vm = (uint64_t)vmask_lds[buf * 4 + 0] | ((uint64_t)vmask_lds[buf * 4 + 1] << 16) |
                        ((uint64_t)vmask_lds[buf * 4 + 2] << 32) | ((uint64_t)vmask_lds[buf * 4 + 3] << 48);
    // S^T for the tile's 4 token blocks
    f32x4 sacc[4];
    // row 16j+n has the same swizzle as row n: two bases, the rest immediates
    const uint8_t* q0 = tb + chunk_off(n, 0, 2 * g);
    const uint8_t* q1 = tb + chunk_off(n, 0, 2 * g + 1);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ks++) {
        const uint8_t* base = (ks & 1) ? q1 : q0;
        const int off = 16 * kRowBytes * j + (ks < 16 ? 128 * (ks >> 1) : 1024);
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(base + off);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qB[ks], acc, 0, 0, 0);
      }
      sacc[j] = acc;
    }
    float s[16];
    float bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int t = 16 * j + 4 * g + r;
        const float v = ((vm >> t) & 1ull) ? sacc[j][r] * a.scale_log2 : -INFINITY;
        s[4 * j + r] = v;
        bm = fmaxf(bm, v);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const bool need = bm > m_use + kLazyH;
    if (__any(need)) {
      const float m_new = need ? bm : m_use;
      const float alpha = (m_new == m_use) ? 1.0f : __builtin_amdgcn_exp2f(m_use - m_new);
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
    const float m_safe = (m_use == -INFINITY) ? 0.f : m_use;
    float* p = s;                                  // P overwrites S in place
#pragma unroll
    for (int i = 0; i < 16; i++) {
      p[i] = __builtin_amdgcn_exp2f(s[i] - m_safe);
      l_part += p[i];
    }
    // V bases for the transposed reads: lane (i = n/4, c = n%4) reads row
    // 32ks + 16h + 4g + i (same swizzle for every ks, h), dims 16nb + 4c
    const uint8_t* vbase[4];
    {
      const int i = n >> 2, c = n & 3;
      const int r0 = 4 * g + i;
#pragma unroll
      for (int q = 0; q < 4; q++) vbase[q] = tb + chunk_off(r0, 0, 2 * q + (c >> 1)) + 8 * (c & 1);
    }
    // P operands, k-step ks: tokens 32ks + 16(i/4) + 4g + (i%4) = blocks 2ks, 2ks+1
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const float* pb = p + 8 * ks;               // p[4*(2ks) + r], p[4*(2ks+1) + r]
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        hi[q] = pack2(pb[2 * q], pb[2 * q + 1]);
        lo[q] = kSplitP ? pack2(pb[2 * q] - __uint_as_float(hi[q] << 16),
                                pb[2 * q + 1] - __uint_as_float(hi[q] & 0xFFFF0000u))
                        : 0u;
      }
      const bf16x8 pa_hi = __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
      const bf16x8 pa_lo = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
      // V rows for this lane's tr loads: 4 consecutive tokens starting at
      // 32ks + 16h + 4g, lane (i = n/4, c = n%4) addresses row +i, dims +4c
#pragma unroll
      for (int nb = 0; nb < 32; nb++) {
        // chunk 2nb + (c>>1) = 8*(nb>>2) + [2(nb&3) + (c>>1)]: four bases
        const uint8_t* a0 = vbase[nb & 3] + 36864 * ks + 128 * (nb >> 2);
        const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
        const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 16 * kRowBytes));
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc_o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, bv, acc_o[nb], 0, 0, 0);
        if (kSplitP)
          acc_o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, bv, acc_o[nb], 0, 0, 0);
      }
    }
  };

  // ---- pipeline: tile t+1 is produced while tile t is consumed.  One raw
  // buffer: right after tile t+1's bytes are dequantized into LDS, the same
  // registers start loading tile t+2's bytes, which then have the rest of
  // this step and the next step's consume phase to arrive.
  int32_t idx_p = load_idx(tile0 * kTileH + my_tok);     // index of the bytes in `raw`
  RawTokH raw;
  load_tok_h(raw, rec_of(idx_p), g);
  if (tile0 < tile1) {
    produce(raw, idx_p, 0);
    idx_p = load_idx((tile0 + 1) * kTileH + my_tok);
    load_tok_h(raw, rec_of(idx_p), g);
    lds_barrier_h();
    auto step = [&](int t, int cbuf) {
      if (t + 1 < tile1) {
        produce(raw, idx_p, cbuf ^ 1);
        idx_p = load_idx((t + 2) * kTileH + my_tok);
        load_tok_h(raw, rec_of(idx_p), g);
      }
      consume(cbuf);
      lds_barrier_h();
    };
    int t = tile0;
    for (; t + 1 < tile1; t += 2) {
      step(t, 0);
      step(t + 1, 1);
    }
    if (t < tile1) step(t, 0);
  }

  // ---- epilogue: this wave's 16 heads
  float lt = l_part;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  // rows of O are heads 4g+r: fetch their denominators and maxima
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const float l = __shfl(lt, 4 * g + r);
    const float m = __shfl(m_use, 4 * g + r);
    float denom = l;
    if (a.splits == 1 && a.sink != nullptr && l > 0.f)
      denom += __builtin_amdgcn_exp2f(a.sink[hw0 + 4 * g + r] * kLog2eH - m);
    inv[r] = l > 0.f ? 1.0f / denom : 0.f;
  }
  const size_t orow = (size_t)row * a.h_q + hw0;
  const size_t prow = ((size_t)split * a.rows + row) * a.h_q + hw0;
#pragma unroll
  for (int nb = 0; nb < 32; nb++) {
    const int dv = 16 * nb + n;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float v = acc_o[nb][r] * inv[r];
      if (a.splits == 1)
        a.out[(orow + 4 * g + r) * kVDim + dv] = __builtin_bit_cast(uint16_t, (__bf16)v);
      else
        a.o_part[(prow + 4 * g + r) * kVDim + dv] = v;
    }
  }
  if (g == 0) {
    const float lse = lt > 0.f ? (m_use + log2f(lt)) * kLn2H : -INFINITY;
    if (a.splits == 1) a.lse[orow + n] = lse;
    else a.lse_part[prow + n] = lse;
  }
}

size_t decode_hsplit_lds_bytes() { return 2 * kTileBytes + 2 * 4 * sizeof(uint32_t); }

hipError_t launch_decode_hsplit(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.rows * (a.h_q / 64) * a.splits;
  const size_t lds = decode_hsplit_lds_bytes();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_hsplit_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((decode_hsplit_kernel<true>), dim3(grid), dim3(64 * kWavesH), lds, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
