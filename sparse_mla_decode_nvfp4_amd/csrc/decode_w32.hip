// Sparse MLA decode for head counts that are multiples of 32, gfx950.
//
// Computes the decode of FlashMLA PR #18 ("W4A16 DSA: NVFP4 KV cache format
// for SM100 sparse decode", PR description): gather the top-k NVFP4 token
// records, dequantize, S = scale * Q K^T over 576 dims, softmax with an
// optional per-head sink, O = P V over 512 dims.  Organisation:
//
//   * a workgroup of four waves owns one (query row, 32-head group, split).
//     Waves 2p and 2p+1 form pair p; pair p takes every other 32-token chunk
//     of the split.  Within a pair, wave half hf owns half of the work:
//     NoPE blocks 16hf..16hf+15 plus RoPE dims 32hf..32hf+31 of the QK
//     contraction (288 dims) and output dims 256hf..256hf+255 of O;
//   * a wave gathers its half of each chunk's records straight into
//     registers, refilling each piece for the next chunk as soon as it has
//     been used (a chunk of lead time), and dequantizes them to fp16 MFMA
//     operands: every E2M1 x E4M3 product has at most 6 significant bits and
//     lies in [2^-10, 2688], so it is exact in fp16; the fp4 convert applies
//     the scale's power of two, one packed multiply applies its mantissa;
//   * partial S^T = K Q^T (32 tokens x 32 heads, 32x32x16 MFMAs) goes through
//     LDS to the other half of the pair; both halves add the two partials
//     (bit-identical sums), run the same online softmax and feed P, already in
//     the PV operand layout, to O += P V (32x32x16 MFMAs) on their own V half,
//     read transposed from a wave-private XOR-swizzled LDS tile;
//   * Q is converted to fp16 once per wave (kept in registers) with a
//     per-head power-of-two scale (the two halves agree on it through LDS),
//     folded into the softmax scale (exact for every bf16 element within 2^31
//     of its head's largest);
//   * P is rounded to fp16 for the PV product (relative error 2^-12); the
//     running max is raised lazily, only when a score exceeds it by more than
//     2^15 (so P stays in fp16 range and rescales of O are rare);
//   * the two pairs merge their states through LDS at the end, and each wave
//     writes a quarter of the output dims.
// Split partials (sink-free O normalised within the split, LSE) are merged by
// the combine kernel launched right after; all workgroups of a row share an
// XCD when the row count allows (the row's records stay in that XCD's L2).
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int kChunkP = 32;                        // tokens per chunk
constexpr int kVRowP = 256 * 2;                    // fp16 V half-row
constexpr int kVTileP = kChunkP * kVRowP;          // 16 KB per wave
constexpr int kXsBytes = 16 * 64 * 4;              // partial S^T of one wave: 4 KB
constexpr float kLazyP = 15.0f;                    // P = 2^(s - m_run) <= 2^15
constexpr float kLn2P = 0.6931471805599453f;
constexpr float kLog2eP = 1.4426950408889634f;

// This lane's share of one record: token tl of the chunk, half hf, lane half
// kg.  NoPE blocks s = 16hf + 2m + kg (m = 0..7, 8 bytes each), their scale
// bytes (blocks with m even sit in scale run kg, m odd in run 2+kg, at
// positions 4hf + m/2) and RoPE dims 32hf + 16kg .. +15.
struct RawP {
  u32x2 nope[8];
  uint32_t sc_even, sc_odd;
  u32x4 rope;
};

__device__ __forceinline__ u32x2 load_nope(const uint8_t* rec, int m, int hf, int kg) {
  return *reinterpret_cast<const u32x2*>(rec + 8 * (16 * hf + 2 * m + kg));
}
__device__ __forceinline__ void load_tail(RawP& r, const uint8_t* rec, int hf, int kg) {
  r.sc_even = *reinterpret_cast<const uint32_t*>(rec + kScaleOffset + 8 * kg + 4 * hf);
  r.sc_odd = *reinterpret_cast<const uint32_t*>(rec + kScaleOffset + 16 + 8 * kg + 4 * hf);
  r.rope = *reinterpret_cast<const u32x4*>(rec + kRopeOffset + 32 * hf + 16 * kg);
}
__device__ __forceinline__ void load_rawp(RawP& r, const uint8_t* rec, int hf, int kg) {
#pragma unroll
  for (int m = 0; m < 8; m++) r.nope[m] = load_nope(rec, m, hf, kg);
  load_tail(r, rec, hf, kg);
}

__device__ __forceinline__ void lds_sync_p() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t pack_f16p(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

// V tile swizzle: 16-byte chunk j of row t lives at chunk j ^ vswz_p(t).
__device__ __forceinline__ int vswz_p(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

// Row (token or head) of element r of a 32x32 accumulator in lane half kg.
__device__ __forceinline__ int acc_row(int r, int kg) { return 8 * (r >> 2) + 4 * kg + (r & 3); }

// Value of lane l ^ 32 combined with this lane's, through one VALU lane swap.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

}  // namespace

// Lane l: tl = l%32, kg = l/32.  With the 32x32x16 shapes a lane holds eight
// k-values of row/column tl; k-step j of half hf covers
//   j < 16: NoPE block 16hf + 2(j>>1) + kg, elements 8(j&1)..+7,
//   j = 16, 17: RoPE dims 32hf + 16kg + 8(j-16)..+7,
// for K (A operand, row = token tl) and Q^T (B operand, column = head tl).
// S^T accumulator: token acc_row(r, kg), head tl.  PV step p uses
// A = P[head tl][k] with k = 8kg + i standing for token 16p + 8(i>>2) + 4kg
// + (i&3) (exactly S^T element r = 8p + i of this lane), B = V[same
// tokens][dv 32nb + tl], C = O[head acc_row(r, kg)][dv 256hf + 32nb + tl].
__global__ void __launch_bounds__(256, 1) decode_w32_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_p[];
  lds_u8* const vt_all = (lds_u8*)smem_p;                      // 4 x 16 KB V tiles
  lds_u8* const xs_all = vt_all + 4 * kVTileP;                 // [2 bufs][4 waves] partial S^T
  lds_f32* const stat = (lds_f32*)(xs_all + 2 * 4 * kXsBytes); // [4 waves][2][32]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pr = wave >> 1;     // pair: token stream
  const int hf = wave & 1;      // half: dims / output dims
  const int tl = lane & 31;
  const int kg = lane >> 5;
  lds_u8* const vt = vt_all + wave * kVTileP;

  // ---- work unit: (row, 32-head group) x split.  Workgroups are dealt to
  // the 8 XCDs round-robin by blockIdx; when the row count allows, every
  // workgroup of a row (all head groups and splits) goes to XCD row % 8, so
  // the head groups share the row's gathered records in that XCD's L2 and
  // the split merge reads its partials from there.
  const int hgroups = a.h_q >> 5;
  int row, hgrp, split;
  {
    const int x = blockIdx.x;
    if ((a.rows & 7) == 0) {
      int y = x >> 3;
      split = y % a.splits;
      y /= a.splits;
      hgrp = y % hgroups;
      row = (y / hgroups) * 8 + (x & 7);
    } else {
      split = x % a.splits;
      const int unit = x / a.splits;
      row = unit / hgroups;
      hgrp = unit - row * hgroups;
    }
  }
  const int h0 = hgrp * 32;

  const int nchunks = (a.topk + kChunkP - 1) / kChunkP;
  const int cps = (nchunks + a.splits - 1) / a.splits;
  const int c_begin = split * cps;
  const int c_end = min(nchunks, c_begin + cps);
  const int span = max(c_end - c_begin, 0);
  const int my_n = (span + 1) >> 1;             // the same for both pairs
  const int32_t* idx_row = a.indices + (size_t)row * a.topk;

  // ---- Q^T operands (head h0 + tl, this half's dims) in fp16 with a
  // per-(head, half) power-of-two scale
  f16x8 qB[18];
  float qscale;   // softmax_scale * log2(e) * 2^p: undoes the Q scale
  {
    const uint16_t* qrow = a.q + ((size_t)row * a.h_q + h0 + tl) * kQkDim;
    u32x4 raw[18];
#pragma unroll
    for (int j = 0; j < 16; j++)
      raw[j] = *reinterpret_cast<const u32x4*>(qrow + 16 * (16 * hf + 2 * (j >> 1) + kg) + 8 * (j & 1));
#pragma unroll
    for (int j = 16; j < 18; j++)
      raw[j] = *reinterpret_cast<const u32x4*>(qrow + kNopeDim + 32 * hf + 16 * kg + 8 * (j - 16));
    uint32_t amax_bits = 0;
#pragma unroll
    for (int j = 0; j < 18; j++)
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const uint32_t x = raw[j][w];
        amax_bits = max(amax_bits, max((x << 16) & 0x7FFFFFFFu, x & 0x7FFF0000u));
      }
    amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 32));
    // both halves of a pair (and both pairs) hold the same heads: agree on
    // the head's largest magnitude through LDS
    __attribute__((address_space(3))) uint32_t* qmax = (__attribute__((address_space(3))) uint32_t*)stat;
    if (kg == 0) qmax[wave * 32 + tl] = amax_bits;
    lds_sync_p();
    amax_bits = max(qmax[(wave ^ 1) * 32 + tl], amax_bits);
    lds_sync_p();            // stat is reused later
    // largest magnitude's exponent e: scale by 2^-(e-14) so it lands in [2^14, 2^15)
    int e = (int)(amax_bits >> 23) - 127;
    if (amax_bits == 0 || amax_bits >= 0x7F800000u) e = 14;
    const int p = max(e - 14, -100);
    // a negative softmax scale flips Q's sign (exact) so the score scale is
    // positive and the max of the raw scores is the max of the scaled ones
    const float mul = a.scale_log2 < 0.f ? -__builtin_ldexpf(1.0f, -p) : __builtin_ldexpf(1.0f, -p);
    qscale = fabsf(a.scale_log2) * __builtin_ldexpf(1.0f, p);
#pragma unroll
    for (int j = 0; j < 18; j++) {
      f16x8 v;
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const uint32_t x = raw[j][w];
        v[2 * w] = (_Float16)(__uint_as_float(x << 16) * mul);
        v[2 * w + 1] = (_Float16)(__uint_as_float(x & 0xFFFF0000u) * mul);
      }
      qB[j] = v;
    }
  }

  f32x16 acc_o[8];
  float m_use = -INFINITY;      // running max (log2 units) of head tl
  float l_part = 0.f;

  auto valid = [&](int32_t idx) { return idx >= 0 && (int64_t)idx < a.num_slots; };
  // index of token tl of this pair's i-th chunk: the load is unconditional
  // (clamped in bounds) and chunk_ok marks the entries that exist (the odd
  // pair's last chunk, or positions past topk, do not); the two are combined
  // a chunk after the load, so no wait follows it
  auto load_idx = [&](int i) -> int32_t {
    const int ic = min(i, max(my_n - 1, 0));
    const int pos = (c_begin + pr + 2 * ic) * kChunkP + tl;
    return idx_row[min(pos, a.topk - 1)];
  };
  auto chunk_ok = [&](int i) -> bool {
    const int c = c_begin + pr + 2 * i;
    return i < my_n && c < c_end && c * kChunkP + tl < a.topk;
  };
  auto rec_of = [&](int32_t idx) {
    const uint32_t slot = valid(idx) ? (uint32_t)idx : 0u;
    return a.cache + a.pa.offset(slot);
  };

  // V tile write bases: k-step j (m = j>>1, h = j&1) of row tl goes to
  // wb[m&3][h] + 256*(m>>2)
  uint32_t wb[4][2];
  {
    const int sw = vswz_p(tl);
    const int sh = sw >> 2, sl = sw & 3;
#pragma unroll
    for (int mr = 0; mr < 4; mr++)
#pragma unroll
      for (int h = 0; h < 2; h++)
        wb[mr][h] = (uint32_t)(size_t)vt + (uint32_t)(tl * kVRowP + 64 * (mr ^ sh) + 16 * ((2 * kg + h) ^ sl));
  }
  // transposed-read bases: step p, group q, block nb at rb[q][nb&3] + 8192p + 256(nb>>2)
  uint32_t rb[2][4];
  {
    const int j16 = lane & 15, i = j16 >> 2, c = j16 & 3, gp = (lane >> 4) & 1;
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int lo = (2 * gp + (c >> 1)) ^ ((2 * q + kg) & 3);
#pragma unroll
      for (int u = 0; u < 4; u++)
        rb[q][u] = (uint32_t)(size_t)vt +
                   (uint32_t)((8 * q + 4 * kg + i) * kVRowP + 64 * (u ^ i) + 16 * lo + 8 * (c & 1));
    }
  }
  const int partner = wave ^ 1;

  // Chunk pos from `cur` (index cur_idx, -1 when absent or invalid), up to
  // the partial-S exchange; each raw piece is refilled with the next chunk's
  // bytes (raw index nxt_raw, loaded a chunk earlier) right after its last use.
  f32x16 sacc;
  uint64_t vmask = 0;
  auto pre = [&](RawP& cur, int32_t& cur_idx, int32_t& nxt_raw, int pos) {
    const int32_t nxt2_raw = load_idx(pos + 2);
    const bool v = valid(cur_idx);
    vmask = __ballot(v) & 0xFFFFFFFFull;
    const uint32_t se = v ? cur.sc_even : 0u;
    const uint32_t so = v ? cur.sc_odd : 0u;
    const int32_t nxt = chunk_ok(pos + 1) ? nxt_raw : -1;
    const uint8_t* const rec_next = rec_of(nxt);
    const u32x4 rope = cur.rope;
    load_tail(cur, rec_next, hf, kg);      // scales and RoPE of the next chunk
    // two accumulators (even / odd k-steps) halve the dependent MFMA chain
    f32x16 sacc1;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      sacc[r] = 0.f;
      sacc1[r] = 0.f;
    }
#pragma unroll
    for (int m = 0; m < 8; m++) {
      const uint32_t sw = (m & 1) ? so : se;
      const f32x2 s2 = ((m >> 2) & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(sw, true)
                                      : __builtin_amdgcn_cvt_pk_f32_fp8(sw, false);
      const float S = ((m >> 1) & 1) ? s2.y : s2.x;
      const float Fv = __uint_as_float((__float_as_uint(S) & 0x807FFFFFu) | 0x3F800000u);
      const f16x2 F = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(Fv, Fv));   // exact
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const uint32_t w = h ? cur.nope[m].y : cur.nope[m].x;
        const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, S, 0) * F;
        const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, S, 1) * F;
        const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, S, 2) * F;
        const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, S, 3) * F;
        const f16x8 k = f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
        *reinterpret_cast<lds_f16x8*>((lds_u8*)(size_t)wb[m & 3][h] + 256 * (m >> 2)) = k;
        if (h == 0) sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(k, qB[2 * m], sacc, 0, 0, 0);
        else sacc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k, qB[2 * m + 1], sacc1, 0, 0, 0);
      }
      cur.nope[m] = load_nope(rec_next, m, hf, kg);
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const f16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rope[2 * h], 1.0f, false);
      const f16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rope[2 * h], 1.0f, true);
      const f16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rope[2 * h + 1], 1.0f, false);
      const f16x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rope[2 * h + 1], 1.0f, true);
      const f16x8 k = f16x8{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
      if (h == 0) sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(k, qB[16], sacc, 0, 0, 0);
      else sacc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k, qB[17], sacc1, 0, 0, 0);
    }
    sacc += sacc1;
    cur_idx = nxt;
    nxt_raw = nxt2_raw;
    lds_u8* const xs = xs_all + (pos & 1) * 4 * kXsBytes;
#pragma unroll
    for (int e = 0; e < 4; e++)
      *reinterpret_cast<lds_f32x4*>(xs + wave * kXsBytes + (e * 64 + lane) * 16) =
          f32x4{sacc[4 * e], sacc[4 * e + 1], sacc[4 * e + 2], sacc[4 * e + 3]};
  };

  // After the exchange: full S^T, online softmax, O += P V.
  auto post = [&](int pos) {
    lds_u8* const xs = xs_all + (pos & 1) * 4 * kXsBytes;
    float s[16];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const f32x4 o4 = *reinterpret_cast<const lds_f32x4*>(xs + partner * kXsBytes + (e * 64 + lane) * 16);
      s[4 * e] = sacc[4 * e] + o4.x;
      s[4 * e + 1] = sacc[4 * e + 1] + o4.y;
      s[4 * e + 2] = sacc[4 * e + 2] + o4.z;
      s[4 * e + 3] = sacc[4 * e + 3] + o4.w;
    }
    // lane holds head tl, tokens acc_row(r, kg); invalid tokens -> -inf.
    // Token validity is uniform over each lane half, so the select condition
    // is a scalar lane mask.
    const uint32_t vm32 = (uint32_t)vmask;
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int t0 = acc_row(r, 0);
      const uint64_t keep = (((vm32 >> t0) & 1u) ? 0x00000000FFFFFFFFull : 0ull) |
                            (((vm32 >> (t0 + 4)) & 1u) ? 0xFFFFFFFF00000000ull : 0ull);
      s[r] = __builtin_amdgcn_inverse_ballot_w64(keep) ? s[r] * qscale : -INFINITY;
      bm = fmaxf(bm, s[r]);
    }
    bm = max_halves(bm);
    const bool need = bm > m_use + kLazyP;
    if (__any(need)) {
      const float m_new = need ? bm : m_use;
      const float alpha = (m_new == m_use) ? 1.0f : __builtin_amdgcn_exp2f(m_use - m_new);
      l_part *= alpha;
      m_use = m_new;
      float ar[16];
#pragma unroll
      for (int r = 0; r < 16; r++) ar[r] = __shfl(alpha, acc_row(r, kg));
      // the accumulators live in AGPRs; pin them there around this (rare)
      // block so their VGPR copies are made here and not on every chunk
#pragma unroll
      for (int nb = 0; nb < 8; nb++) {
        asm volatile("" : "+a"(acc_o[nb]));
#pragma unroll
        for (int r = 0; r < 16; r++) acc_o[nb][r] *= ar[r];
        asm volatile("" : "+a"(acc_o[nb]));
      }
    }
    const float ms = (m_use == -INFINITY) ? 0.f : m_use;
    uint32_t pd[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(s[r] - ms);
      const float p1 = __builtin_amdgcn_exp2f(s[r + 1] - ms);
      l_part += p0 + p1;
      pd[r >> 1] = pack_f16p(p0, p1);
    }
    // ---- O += P V on this half's output dims
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const f16x8 pA = __builtin_bit_cast(f16x8, u32x4{pd[4 * p], pd[4 * p + 1], pd[4 * p + 2], pd[4 * p + 3]});
#pragma unroll
      for (int nb = 0; nb < 8; nb++) {
        const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((lds_u8*)(size_t)rb[0][nb & 3] + 8192 * p + 256 * (nb >> 2)));
        const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((lds_u8*)(size_t)rb[1][nb & 3] + 8192 * p + 256 * (nb >> 2)));
        const f16x8 bv = __builtin_bit_cast(f16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc_o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pA, bv, acc_o[nb], 0, 0, 0);
      }
      // keep at most two blocks of V operands in flight ahead of the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int nb = 0; nb < 6; nb++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };

  // Every chunk passes exactly one barrier (the partial-S exchange) in every
  // wave: both pairs run the same number of chunks.
  {
    // zero the accumulators with an MFMA so they start out (and stay) in
    // the accumulator registers the PV MFMAs use
    const f16x8 z = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    f32x16 zc;
#pragma unroll
    for (int r = 0; r < 16; r++) zc[r] = 0.f;
#pragma unroll
    for (int nb = 0; nb < 8; nb++) acc_o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(z, z, zc, 0, 0, 0);
  }
  if (my_n > 0) {
    RawP buf;
    int32_t idx_cur = load_idx(0);
    int32_t idx_nxt = load_idx(1);
    idx_cur = chunk_ok(0) ? idx_cur : -1;
    load_rawp(buf, rec_of(idx_cur), hf, kg);
    for (int pos = 0; pos < my_n; pos++) {
      pre(buf, idx_cur, idx_nxt, pos);
      lds_sync_p();
      post(pos);
    }
  }

  // ---- merge the two pairs (same heads and output dims, disjoint tokens)
  l_part = sum_halves(l_part);
  if (kg == 0) {
    stat[(wave * 2 + 0) * 32 + tl] = m_use;
    stat[(wave * 2 + 1) * 32 + tl] = l_part;
  }
  lds_sync_p();
  const int other = wave ^ 2;         // same half, other pair
  float Mh, Lh, fown;
  {
    const float mo = stat[(other * 2 + 0) * 32 + tl];
    const float lo = stat[(other * 2 + 1) * 32 + tl];
    Mh = fmaxf(m_use, mo);
    const float fo = (mo == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mo - Mh);
    fown = (m_use == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_use - Mh);
    Lh = l_part * fown + lo * fo;
  }
  {
    float fr[16];
#pragma unroll
    for (int r = 0; r < 16; r++) fr[r] = __shfl(fown, acc_row(r, kg));
#pragma unroll
    for (int nb = 0; nb < 8; nb++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc_o[nb][r] *= fr[r];
  }
  // pair 0 keeps output blocks 0..3 of its half, pair 1 blocks 4..7; each
  // sends the other four through its V tile (64 floats per lane)
  auto send_recv = [&](auto kept_c, auto sent_c) {
    constexpr int kKept = decltype(kept_c)::value;
    constexpr int kSent = decltype(sent_c)::value;
    lds_f32x4* mine = reinterpret_cast<lds_f32x4*>(vt) + lane;
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int rq = 0; rq < 4; rq++) {
        const f32x16& o = acc_o[kSent + u];
        mine[(4 * u + rq) * 64] = f32x4{o[4 * rq], o[4 * rq + 1], o[4 * rq + 2], o[4 * rq + 3]};
      }
    lds_sync_p();
    const lds_f32x4* theirs = reinterpret_cast<const lds_f32x4*>(vt_all + other * kVTileP) + lane;
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int rq = 0; rq < 4; rq++) {
        const f32x4 t = theirs[(4 * u + rq) * 64];
        acc_o[kKept + u][4 * rq] += t.x;
        acc_o[kKept + u][4 * rq + 1] += t.y;
        acc_o[kKept + u][4 * rq + 2] += t.z;
        acc_o[kKept + u][4 * rq + 3] += t.w;
      }
  };
  if (pr == 0) send_recv(IntC<0>{}, IntC<4>{});
  else send_recv(IntC<4>{}, IntC<0>{});

  // ---- normalise and write this wave's quarter of the output dims
  const bool single = a.splits == 1;
  float inv[16];
  {
    // one denominator per head (lane tl holds head tl), then to the O layout
    float denom = Lh;
    if (single && a.sink != nullptr && Lh > 0.f) denom += __builtin_amdgcn_exp2f(a.sink[h0 + tl] * kLog2eP - Mh);
    const float invh = Lh > 0.f ? 1.0f / denom : 0.f;
#pragma unroll
    for (int r = 0; r < 16; r++) inv[r] = __shfl(invh, acc_row(r, kg));
  }
  const size_t orow = (size_t)row * a.h_q + h0;
  const size_t prow = ((size_t)split * a.rows + row) * a.h_q + h0;
  auto write_blocks = [&](auto base_c) {
    constexpr int kB = decltype(base_c)::value;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int dv = 256 * hf + 32 * (kB + u) + tl;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int hr = acc_row(r, kg);
        const float v = acc_o[kB + u][r] * inv[r];
        if (single)
          a.out[(orow + hr) * kVDim + dv] = __builtin_bit_cast(uint16_t, (__bf16)v);
        else
          a.o_part[(prow + hr) * kVDim + dv] = v;
      }
    }
  };
  if (pr == 0) write_blocks(IntC<0>{});
  else write_blocks(IntC<4>{});
  if (wave == 0 && kg == 0) {
    const float lse = Lh > 0.f ? (Mh + __log2f(Lh)) * kLn2P : -INFINITY;
    if (single) a.lse[orow + tl] = lse;
    else a.lse_part[prow + tl] = lse;
  }
}

size_t decode_w32_lds_bytes() { return 4 * kVTileP + 2 * 4 * kXsBytes + 4 * 2 * 32 * sizeof(float); }

hipError_t launch_decode_w32(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.rows * (a.h_q / 32) * a.splits;
  const size_t lds = decode_w32_lds_bytes();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_w32_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(decode_w32_kernel, dim3(grid), dim3(256), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  // split partials are merged by the combine kernel: the launch boundary
  // makes them visible across XCDs without device-scope fences (on a
  // multi-XCD part those write back and invalidate L2)
  return launch_combine(a.o_part, a.lse_part, a.splits, a.rows, a.h_q, a.sink, a.out, a.lse, stream);
}

}  // namespace nvfp4
