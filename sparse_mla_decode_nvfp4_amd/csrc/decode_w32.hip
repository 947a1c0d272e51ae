// Sparse MLA decode for head counts that are multiples of 32, gfx950.
//
// Computes the decode of FlashMLA PR #18 ("W4A16 DSA: NVFP4 KV cache format
// for SM100 sparse decode", PR description): gather the top-k NVFP4 token
// records, dequantize, S = scale * Q K^T over 576 dims, softmax with an
// optional per-head sink, O = P V over 512 dims.  Organisation:
//
//   * a workgroup of eight waves (two per SIMD) owns one (query row, 32-head
//     group, split).  Waves 2p and 2p+1 form pair p (p = 0..3); the pairs
//     share out the split's 16-token chunks.  Launches of many workgroups
//     per CU use workgroups of two pairs instead, two per CU, so that one
//     workgroup's set-up and merge overlap the other's chunks.  Within a pair, wave half hf
//     owns NoPE blocks 16hf..16hf+15 plus RoPE dims 32hf..32hf+31 of the QK
//     contraction (288 dims) and output dims 256hf..256hf+255 of O;
//   * a wave gathers its half of each chunk's records straight into
//     registers, refilling each piece for the next chunk as soon as it has
//     been used, and dequantizes them to fp16 MFMA operands: every E2M1 x
//     E4M3 product has at most 6 significant bits and lies in [2^-10, 2688],
//     so it is exact in fp16: the codes convert exactly and one packed
//     multiply by the scale (converted exactly to fp16) gives the product;
//   * partial S^T = K Q^T (16 tokens x 32 heads: 16x16x32 MFMAs for two
//     16-head blocks sharing each K operand) goes through LDS to the other
//     half of the pair; both halves add the two partials (bit-identical sums)
//     and run the same online softmax; P moves to the 32x32 operand layout
//     with one lane-row swap, and O^T += V^T P^T runs as 32x32x16 MFMAs on
//     the wave's own V half, read transposed from a wave-private XOR-swizzled
//     LDS tile (each lane accumulates one head's output dims);
//   * Q is converted to fp16 once per workgroup with a per-head power-of-two
//     scale folded into the softmax scale (exact for every bf16 element
//     within 2^31 of its head's largest) and read from LDS as MFMA operands;
//   * P enters the PV product as fp16 hi + lo parts (two MFMAs per block,
//     P carried to about 2^-22); the running max is raised lazily, only when
//     a score exceeds it by more than 2^15 (P stays in fp16 range and
//     rescales of O are rare);
//   * the pairs merge their states through LDS at the end (pairwise sums: two
//     rounds for four pairs, one for two), and each wave writes its share of
//     the output dims.
// Split partials (sink-free O normalised within the split, in fp16, and LSE)
// are merged by the combine kernel launched right after; all workgroups of a row share an
// XCD when the row count allows (the row's records stay in that XCD's L2).
#include <math.h>

#include <atomic>

#include "device_common.h"
#include "kv_source.h"
#include "lane_ops.h"
#include "launch.h"

namespace nvfp4 {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

constexpr int kChunkP = 16;                        // tokens per chunk
constexpr int kVRowP = 256 * 2;                    // fp16 V half-row
constexpr int kVTileP = kChunkP * kVRowP;          // 8 KB per wave
constexpr int kXsBytes = 2 * 64 * 16;              // partial S^T of one wave: 2 KB
constexpr int kQBytes = 2 * 2 * 9 * 64 * 16;       // Q operands: [half][block][k-step][lane]
constexpr float kLazyP = 15.0f;                    // P = 2^(s - m_run) <= 2^15
constexpr int kSpinLimit = 1 << 22;                // polls of a partner wait (~0.1 s)
constexpr float kLn2P = 0.6931471805599453f;
constexpr float kLog2eP = 1.4426950408889634f;

// LDS map (bytes) of a workgroup of kPairs pairs: V tiles, partial-S
// exchange, Q operands, per-head statistics, then the pair counters.  Four
// pairs (one workgroup per CU) double-buffer the exchange; two pairs keep one
// exchange buffer per wave so that two workgroups fit in a CU's 160 KB.  The
// merge of the pairs at the end reuses the space below the statistics.
template <int kPairs>
struct LdsW32 {
  static constexpr int kWaves = 2 * kPairs;
  static constexpr int kXsBufs = kPairs == 4 ? 2 : 1;
  static constexpr int kOffXs = kWaves * kVTileP;
  static constexpr int kOffQ = kOffXs + kXsBufs * kWaves * kXsBytes;
  static constexpr int kOffStat = kOffQ + kQBytes;
  static constexpr int kOffFlag = kOffStat + kWaves * 2 * 32 * 4 + 2 * 32 * 4;
  // published and consumed counters per wave, then the lost-wait flag
  static constexpr int kOffFail = kOffFlag + 2 * kWaves * 4;
  // the sink logits of the group's 32 heads
  static constexpr int kOffSink = kOffFail + 16;
  static constexpr int kBytes = kOffSink + 32 * 4;
  // merge: 4 slots of 4 KB per wave in round one
  static_assert(4 * kWaves * 4096 <= kOffStat, "merge slots overlap the statistics");
};
static_assert(LdsW32<2>::kBytes <= 80 * 1024, "two workgroups of two pairs must fit in a CU");

// This lane's share of one record (token n of the chunk, half hf, lane group
// g): NoPE blocks s = 16hf + 4g + u (u = 0..3), 32 contiguous bytes; their
// scales; RoPE dims 32hf + 8g .. +7.  In the 352-byte record block s's scale
// sits at 320 + 8(s&3) + (s>>2), so the four are byte g of the dwords at
// 320 + 8u + 4hf (two wide gathers cover them rather than four narrow ones),
// and RoPE is 8 E4M3 bytes; in the 432-byte record they are the four bytes
// of the dword at 256 + 16hf + 4g, and RoPE is 8 bf16.
template <class F>
struct RawP;
// Scale dword 2u + hf of the 352-byte record's scale area holds blocks
// 16hf + 4g + u (byte g).  A byte permute with selector byte 4hf + g picks
// byte g of the first or second dword of a pair.
template <>
struct RawP<Fmt352> {
  u32x4 nope[2];
  u32x4 sc[2];           // the scale area: dword 2u + hf holds blocks 16hf + 4g + u
  u32x2 rope;
  // this lane's four scale bytes (block 16hf + 4g + u in byte u); sel[u]
  // holds 4hf + g in byte u and 0x0c (a zero byte) elsewhere
  __device__ __forceinline__ uint32_t scales(const uint32_t (&sel)[4]) const {
    return (__builtin_amdgcn_perm(sc[0].y, sc[0].x, sel[0]) | __builtin_amdgcn_perm(sc[0].w, sc[0].z, sel[1])) |
           (__builtin_amdgcn_perm(sc[1].y, sc[1].x, sel[2]) | __builtin_amdgcn_perm(sc[1].w, sc[1].z, sel[3]));
  }
};
template <>
struct RawP<Fmt432> {
  u32x4 nope[2];
  uint32_t sc;           // block 16hf + 4g + u in byte u
  u32x4 rope;
  __device__ __forceinline__ uint32_t scales(const uint32_t (&)[4]) const { return sc; }
};

template <class F>
__device__ __forceinline__ void load_nope(RawP<F>& r, int q, const uint8_t* rec, int hf, int g) {
  r.nope[q] = *reinterpret_cast<const u32x4*>(rec + 128 * hf + 32 * g + 16 * q);
}
__device__ __forceinline__ void load_tail(RawP<Fmt352>& r, const uint8_t* rec, int hf, int g) {
  r.sc[0] = *reinterpret_cast<const u32x4*>(rec + Fmt352::kScaleOff);
  r.sc[1] = *reinterpret_cast<const u32x4*>(rec + Fmt352::kScaleOff + 16);
  r.rope = *reinterpret_cast<const u32x2*>(rec + Fmt352::kRopeOff + 32 * hf + 8 * g);
}
__device__ __forceinline__ void load_tail(RawP<Fmt432>& r, const uint8_t* rec, int hf, int g) {
  r.sc = *reinterpret_cast<const uint32_t*>(rec + Fmt432::kScaleOff + 16 * hf + 4 * g);
  r.rope = *reinterpret_cast<const u32x4*>(rec + Fmt432::kRopeOff + 64 * hf + 16 * g);
}

__device__ __forceinline__ void lds_sync_p() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t pack_f16p(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}


}  // namespace

// Lane l: n = l%16, g = l/16, kg = l/32, tl = l%32.
//   QK (16x16x32), k-step j of half hf (8 dims per lane group g):
//     j < 8: NoPE block 16hf + 4g + (j>>1), elements 8(j&1)..+7,
//     j = 8: RoPE dims 32hf + 8g..+7;
//   A = K[token n][those dims], B = Q^T[same dims][head 16b+n],
//   C = S^T[token 4g+r][head 16b+n] for head blocks b = 0, 1.
//   PV (32x32x16), computed as O^T = V^T P^T: A = V^T[dv 32nb + tl][token
//   8kg+i], B = P^T[token 8kg+i][head tl], C = O^T[dv 256hf + 32nb + 8(r>>2) +
//   4kg + (r&3)][head tl]: a lane's 128 accumulators all belong to head tl.
template <bool kDual, class F, int kPairs>
__global__ void __launch_bounds__(128 * kPairs, kPairs == 4 ? 1 : 2) decode_w32_kernel(DecodeArgs a) {
  using L = LdsW32<kPairs>;
  constexpr int kWavesP = L::kWaves;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_p[];
  lds_u8* const lds = (lds_u8*)smem_p;
  lds_u8* const xs_all = lds + L::kOffXs;
  lds_u8* const qlds = lds + L::kOffQ;
  lds_f32* const stat = (lds_f32*)(lds + L::kOffStat);                        // [wave][m, l][32]
  lds_u32* const qmax = (lds_u32*)(lds + L::kOffStat + kWavesP * 2 * 32 * 4); // [half][32]
  lds_u32* const flag = (lds_u32*)(lds + L::kOffFlag);   // [wave]: chunks whose partial S is published
  lds_u32* const consumed = flag + kWavesP;              // [wave]: partner chunks read (one buffer)
  lds_u32* const failed = (lds_u32*)(lds + L::kOffFail); // a wave gave up waiting for its partner
  lds_f32* const sinkl = (lds_f32*)(lds + L::kOffSink);  // [32] sink logits (without splits)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pr = wave >> 1;     // pair: token stream
  const int hf = wave & 1;      // half: dims / output dims
  const int n = lane & 15;
  const int g = lane >> 4;
  const int kg = lane >> 5;
  const int tl = lane & 31;
  lds_u8* const vt = lds + wave * kVTileP;

  // ---- work unit: (row, 32-head group) x split.  Workgroups are dealt to
  // the 8 XCDs round-robin by blockIdx; when the row count allows, every
  // workgroup of a row (all head groups and splits) goes to XCD row % 8, so
  // the head groups share the row's gathered records in that XCD's L2.
  const int hgroups = a.h_q >> 5;
  int row, hgrp, split;
  {
    const int x = blockIdx.x;
    if (a.s_q > 1 && a.rows % (8 * a.s_q) == 0) {
      // several query rows per sequence: sequence q's rows go to XCD q % 8
      // (they share their most recent tokens)
      int y = x >> 3;
      split = y % a.splits;
      y /= a.splits;
      hgrp = y % hgroups;
      const int r = y / hgroups;
      row = ((r / a.s_q) * 8 + (x & 7)) * a.s_q + r % a.s_q;
    } else if ((a.rows & 7) == 0) {
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
  const RowSource<kDual> src(a, row);

  // Chunks are numbered within the split and dealt in blocks of 14: pairs 0
  // and 1 take 4 of each block (offsets p, p+4, p+8, 12+p), pairs 2 and 3
  // take 3 (p, p+4, p+8).  Pairs 0 and 1 are the first waves of their SIMDs,
  // which issue first and run about 1.35 times as fast, so the pairs finish
  // together; the fixed deal keeps the summation order, and so the result,
  // the same on every run.  With two pairs (both the first, or both the
  // second, waves of their SIMDs) the chunks alternate.  cid0..cid2 are this
  // pair's chunks pos, pos+1 and pos+2.
  const int kp = pr < 2 ? 4 : 3;
  auto cid_of = [&](int i) {
    if constexpr (kPairs == 2) return pr + 2 * i;
    const int blk = i / kp, j = i - blk * kp;
    return 14 * blk + (j < 3 ? pr + 4 * j : 12 + pr);
  };
  int cid0 = cid_of(0), cid1 = cid_of(1), cid2 = cid_of(2);
  // joined-list position of token n of chunk c
  auto tok_pos = [&](int c) { return (c_begin + min(c, span)) * kChunkP + n; };
  // its index: the load is unconditional (clamped in bounds) and chunk_ok
  // marks the entries that exist; the two are combined a chunk after the
  // load, so no wait follows it
  auto load_idx = [&](int c) -> int32_t { return src.load(min(tok_pos(c), a.topk - 1)); };
  auto chunk_ok = [&](int c) -> bool { return c < span && tok_pos(c) < a.topk; };

  // the first chunk's indices and records are requested before the Q
  // set-up below, which hides part of their latency
  RawP<F> buf;
  bool ok_cur = false;
  int32_t idx_nxt = -1;
  if (cid0 < span) {
    const int32_t idx0 = load_idx(cid0);
    idx_nxt = load_idx(cid1);
    const RecRef r = resolve_rec<kDual>(a, idx0, chunk_ok(cid0), tok_pos(cid0), src.topk0);
    ok_cur = r.ok;
    load_nope(buf, 0, r.ptr, hf, g);
    load_nope(buf, 1, r.ptr, hf, g);
    load_tail(buf, r.ptr, hf, g);
  }

  // ---- Q^T operands in fp16 with a per-head power-of-two scale.  The waves
  // of pairs 0 and 1 convert head block b = pr of half hf; the two halves
  // agree on each head's scale through LDS.
  float qscale[2];   // |softmax_scale| * log2(e) * 2^p of heads n and 16+n
  {
    u32x4 raw[9];
    if (pr < 2) {
      const uint16_t* qrow = a.q + ((size_t)row * a.h_q + h0 + 16 * pr + n) * kQkDim;
#pragma unroll
      for (int j = 0; j < 8; j++)
        raw[j] = *reinterpret_cast<const u32x4*>(qrow + 16 * (16 * hf + 4 * g + (j >> 1)) + 8 * (j & 1));
      raw[8] = *reinterpret_cast<const u32x4*>(qrow + kNopeDim + 32 * hf + 8 * g);
      // wave 0 also fetches the group's sink logits for the epilogue; they
      // arrive with its Q elements, which it waits for next
      float sink_v = 0.f;
      if (wave == 0 && a.splits == 1 && a.sink != nullptr) sink_v = a.sink[h0 + (lane & 31)];
      uint32_t amax_bits = 0;
#pragma unroll
      for (int j = 0; j < 9; j++)
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const uint32_t x = raw[j][w];
          amax_bits = max(amax_bits, max((x << 16) & 0x7FFFFFFFu, x & 0x7FFF0000u));
        }
      amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 16));
      amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 32));
      if (g == 0) qmax[hf * 32 + 16 * pr + n] = amax_bits;
      if (wave == 0 && lane < 32) sinkl[lane] = sink_v;
    }
    if (lane == 0) {
      flag[wave] = 0;
      consumed[wave] = 0;
      if (wave == 0) *failed = 0;
    }
    lds_sync_p();
    int pq[2];
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const uint32_t am = max(qmax[16 * b + n], qmax[32 + 16 * b + n]);
      // largest magnitude's exponent e: scale by 2^-(e-14) so it lands in [2^14, 2^15)
      int e = (int)(am >> 23) - 127;
      if (am == 0 || am >= 0x7F800000u) e = 14;
      pq[b] = max(e - 14, -100);
      qscale[b] = fabsf(a.scale_log2) * __builtin_ldexpf(1.0f, pq[b]);
    }
    if (pr < 2) {
      // a negative softmax scale flips Q's sign (exact), so the score scale
      // is positive and the max of the raw scores is the max of the scaled ones
      const int p = pr == 0 ? pq[0] : pq[1];
      const float mul = a.scale_log2 < 0.f ? -__builtin_ldexpf(1.0f, -p) : __builtin_ldexpf(1.0f, -p);
#pragma unroll
      for (int j = 0; j < 9; j++) {
        lds_u8* const dst = qlds + (((hf * 2 + pr) * 9 + j) * 64 + lane) * 16;
        if (F::kBf16Rope && j == 8) {
          // bf16 RoPE keys meet a bf16 Q operand (x * 2^-p is exact in bf16)
          bf16x8 v;
#pragma unroll
          for (int w = 0; w < 4; w++) {
            const uint32_t x = raw[j][w];
            v[2 * w] = (__bf16)(__uint_as_float(x << 16) * mul);
            v[2 * w + 1] = (__bf16)(__uint_as_float(x & 0xFFFF0000u) * mul);
          }
          *reinterpret_cast<lds_bf16x8*>(dst) = v;
        } else {
          f16x8 v;
#pragma unroll
          for (int w = 0; w < 4; w++) {
            const uint32_t x = raw[j][w];
            v[2 * w] = (_Float16)(__uint_as_float(x << 16) * mul);
            v[2 * w + 1] = (_Float16)(__uint_as_float(x & 0xFFFF0000u) * mul);
          }
          *reinterpret_cast<lds_f16x8*>(dst) = v;
        }
      }
    }
    lds_sync_p();
  }

  f32x16 acc_o[8];
  float m_use[2] = {-INFINITY, -INFINITY};    // running max (log2 units) of heads n, 16+n
  // the exponent offset of P: -m_use, or 0 while m_use is -inf (every
  // score so far masked); changes only when the max is raised
  float neg_m[2] = {0.f, 0.f};
  float l_part[2] = {0.f, 0.f};

  // V tile: k-step j of row n is 16-byte chunk 8g + j of the half-row
  const int vsw = vswz_p(n);
  const uint32_t wbase = (uint32_t)(size_t)vt + (uint32_t)(n * kVRowP);
  // transposed reads: lane reads 4 fp16 of row 8kg + 4q + i (i = (l%16)/4)
  // at dv 32nb + 16((l/16)&1) + 4(l%4); block nb at rb[q][nb&3] + 256(nb>>2)
  uint32_t rb[2][4];
  {
    const int j16 = lane & 15, i = j16 >> 2, c = j16 & 3, gp = g & 1;
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int lo = (2 * gp + (c >> 1)) ^ ((2 * kg + q) & 3);
#pragma unroll
      for (int u = 0; u < 4; u++)
        rb[q][u] = (uint32_t)(size_t)vt +
                   (uint32_t)((8 * kg + 4 * q + i) * kVRowP + 64 * (u ^ i) + 16 * lo + 8 * (c & 1));
    }
  }
  const int partner = wave ^ 1;
  // byte selectors of the 352-byte record's scales: byte u takes byte g of
  // scale dword 2u + hf (selector 4hf + g over the dword pair), the others
  // 0x0c (a zero byte)
  uint32_t ssel[4];
#pragma unroll
  for (int u = 0; u < 4; u++)
    ssel[u] = (0x0c0c0c0cu & ~(0xFFu << (8 * u))) | ((uint32_t)(4 * hf + g) << (8 * u));

  // Chunk pos from `cur` (cur_ok: whether this lane's token takes part), up to
  // the partial-S exchange; each raw piece is refilled with the next chunk's
  // bytes (raw index nxt_raw, loaded a chunk earlier) right after its use.
  f32x4 sacc[2];
  uint32_t okbits = 0;   // bit r: token 4g+r of the current chunk takes part
  // A partner wait that runs out of polls (correct execution never gets
  // near the limit) sets `lost`; the workgroup then writes NaN O and LSE
  // instead of results built from a partial S that may be stale.
  bool lost = false;
  auto pre = [&](RawP<F>& cur, bool& cur_ok, int32_t& nxt_raw, int pos) {
    const int32_t nxt2_raw = load_idx(cid2);
    const bool v = cur_ok;
    // validity of tokens 4g..4g+3 (the rows of this lane's partial S^T),
    // taken from the lanes that hold those tokens' bytes
    okbits = ((uint32_t)__ballot(v) >> (4 * g)) & 0xFu;
    const RecRef rn = resolve_rec<kDual>(a, nxt_raw, chunk_ok(cid1), tok_pos(cid1), src.topk0);
    const uint8_t* const rec_next = rn.ptr;
    // block scales of this lane; zero for an invalid token, so its V row is
    // zero (a mask, not a select: the compiler turns the select into a branch
    // around the byte permutes, whose join waits for more of the gathers)
    const uint32_t sw = cur.scales(ssel) & (0u - (uint32_t)v);
    // the four block scales as fp16 (exact), two per convert
    const f16x2 sp[2] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true)};
    const auto rope = cur.rope;
    load_tail(cur, rec_next, hf, g);      // scales and RoPE of the next chunk
#pragma unroll
    for (int b = 0; b < 2; b++) sacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int u = j >> 1;
      // codes convert exactly; times the fp16 scale (a half-select of its
      // pair) the product is exact
      const _Float16 sv = sp[u >> 1][u & 1];
      const f16x2 Fs = {sv, sv};
      const uint32_t w = cur.nope[u >> 1][2 * (u & 1) + (j & 1)];
      const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * Fs;
      const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * Fs;
      const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * Fs;
      const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * Fs;
      const f16x8 k = f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
      *reinterpret_cast<lds_f16x8*>((lds_u8*)(size_t)wbase + (((8 * g + j) ^ vsw) << 4)) = k;
#pragma unroll
      for (int b = 0; b < 2; b++) {
        const f16x8 qv = *reinterpret_cast<const lds_f16x8*>(qlds + (((hf * 2 + b) * 9 + j) * 64 + lane) * 16);
        sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k, qv, sacc[b], 0, 0, 0);
      }
      if (j == 3) load_nope(cur, 0, rec_next, hf, g);
      if (j == 7) load_nope(cur, 1, rec_next, hf, g);
    }
    if constexpr (F::kBf16Rope) {
      // bf16 RoPE straight from the record into a bf16 MFMA
      const bf16x8 k = __builtin_bit_cast(bf16x8, rope);
#pragma unroll
      for (int b = 0; b < 2; b++) {
        const bf16x8 qv = *reinterpret_cast<const lds_bf16x8*>(qlds + (((hf * 2 + b) * 9 + 8) * 64 + lane) * 16);
        sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, qv, sacc[b], 0, 0, 0);
      }
    } else {
      const f16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rope.x, 1.0f, false);
      const f16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rope.x, 1.0f, true);
      const f16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rope.y, 1.0f, false);
      const f16x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rope.y, 1.0f, true);
      const f16x8 k = f16x8{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
#pragma unroll
      for (int b = 0; b < 2; b++) {
        const f16x8 qv = *reinterpret_cast<const lds_f16x8*>(qlds + (((hf * 2 + b) * 9 + 8) * 64 + lane) * 16);
        sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k, qv, sacc[b], 0, 0, 0);
      }
    }
    cur_ok = rn.ok;
    nxt_raw = nxt2_raw;
    lds_u8* const xs = xs_all + (L::kXsBufs == 2 ? (pos & 1) : 0) * kWavesP * kXsBytes;
    if constexpr (L::kXsBufs == 1) {
      // one buffer: the partner must have read this wave's previous chunk
      // (bounded: it reads it right after its own exchange write)
      bool seen = false;
      for (int it = 0; it < kSpinLimit; it++) {
        if ((int)__hip_atomic_load(consumed + partner, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= pos) {
          seen = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      lost |= !seen;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
#pragma unroll
    for (int b = 0; b < 2; b++)
      *reinterpret_cast<lds_f32x4*>(xs + wave * kXsBytes + (b * 64 + lane) * 16) = sacc[b];
    // publish: the partial S (and every earlier LDS access of this wave)
    // completes before the count moves.  One lane stores it: 64 lanes
    // storing to one LDS word conflict with each other, about 64 stall
    // cycles per chunk.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0)
      __hip_atomic_store(flag + wave, (uint32_t)(pos + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  // wait until the partner has published chunk pos (bounded: the partner
  // runs the same number of chunks in the same workgroup)
  auto pair_wait = [&](int pos) {
    bool seen = false;
    for (int it = 0; it < kSpinLimit; it++) {
      if ((int)__hip_atomic_load(flag + partner, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) > pos) {
        seen = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    lost |= !seen;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  // After the exchange: full S^T, online softmax, O += P V.
  auto post = [&](int pos) {
    lds_u8* const xs = xs_all + (L::kXsBufs == 2 ? (pos & 1) : 0) * kWavesP * kXsBytes;
    float s[2][4];
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const f32x4 o4 = *reinterpret_cast<const lds_f32x4*>(xs + partner * kXsBytes + (b * 64 + lane) * 16);
#pragma unroll
      for (int r = 0; r < 4; r++) s[b][r] = sacc[b][r] + o4[r];
    }
    if constexpr (L::kXsBufs == 1) {
      // the partner's partial S is read: it may write its next one
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0)
        __hip_atomic_store(consumed + wave, (uint32_t)(pos + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // lane holds heads n, 16+n and tokens 4g+r; invalid tokens -> -inf
    // (a per-lane select on okbits: no scalar mask building)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const bool ok = (okbits >> r) & 1u;
#pragma unroll
      for (int b = 0; b < 2; b++) s[b][r] = ok ? s[b][r] : -INFINITY;
    }
    // maxima of the raw scores, then scaled (the score scale is positive)
    float bm[2];
#pragma unroll
    for (int b = 0; b < 2; b++) bm[b] = fmaxf(fmaxf(s[b][0], s[b][1]), fmaxf(s[b][2], s[b][3]));
    max_blocks(bm[0], bm[1]);
    bool need = false;
#pragma unroll
    for (int b = 0; b < 2; b++) {
      bm[b] *= qscale[b];
      need |= bm[b] > m_use[b] + kLazyP;
    }
    if (__any(need)) {
      float alpha[2];
#pragma unroll
      for (int b = 0; b < 2; b++) {
        const float m_new = bm[b] > m_use[b] + kLazyP ? bm[b] : m_use[b];
        alpha[b] = (m_new == m_use[b]) ? 1.0f : __builtin_amdgcn_exp2f(m_use[b] - m_new);
        l_part[b] *= alpha[b];
        m_use[b] = m_new;
        neg_m[b] = (m_new == -INFINITY) ? 0.f : -m_new;
      }
      // a lane's rows of O are all its head's (tl: head n for tl < 16,
      // 16 + n otherwise).  Before the pair's first PV, O is all +0 and
      // stays so: the first chunk, which always raises the max, skips the
      // multiplies
      if (pos > 0) {
        const float al = tl < 16 ? alpha[0] : alpha[1];
#pragma unroll
        for (int nb = 0; nb < 8; nb++)
#pragma unroll
          for (int r = 0; r < 16; r++) acc_o[nb][r] *= al;
      }
    }
    // P as fp16 hi + lo parts (the lo part holds P - hi exactly to fp16's
    // precision), so PV carries P to about 2^-22 instead of 2^-11
    uint32_t pd[2][2], pl[2][2];
#pragma unroll
    for (int b = 0; b < 2; b++) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], qscale[b], neg_m[b]));
        l_part[b] += p[r];
      }
#pragma unroll
      for (int w = 0; w < 2; w++) split_p(p[2 * w], p[2 * w + 1], pd[b][w], pl[b][w]);
    }
    // P into the 32x32 operand layout: lane 16G+n takes head 16(G&1)+n,
    // tokens 8(G>>1)+0..7; tokens +0..3 sit in row 2(G>>1), +4..7 in row
    // 2(G>>1)+1.  Swapping the odd rows of block 0 with the even rows of
    // block 1 leaves exactly that: even rows get (own block 0, next row's
    // block 0), odd rows (previous row's block 1, own block 1).
    const auto c0 = __builtin_amdgcn_permlane16_swap(pd[0][0], pd[1][0], false, false);
    const auto c1 = __builtin_amdgcn_permlane16_swap(pd[0][1], pd[1][1], false, false);
    const f16x8 pA = __builtin_bit_cast(f16x8, u32x4{c0[0], c1[0], c0[1], c1[1]});
    const auto e0 = __builtin_amdgcn_permlane16_swap(pl[0][0], pl[1][0], false, false);
    const auto e1 = __builtin_amdgcn_permlane16_swap(pl[0][1], pl[1][1], false, false);
    const f16x8 pL = __builtin_bit_cast(f16x8, u32x4{e0[0], e1[0], e0[1], e1[1]});
    // ---- O += P V on this half's output dims
    // two blocks at a time: both lo products, then both hi products, so
    // the two products into one accumulator are not back to back
#pragma unroll
    for (int nb = 0; nb < 8; nb += 2) {
      f16x8 bv[2];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((lds_u8*)(size_t)rb[0][(nb + u) & 3] + 256 * ((nb + u) >> 2)));
        const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((lds_u8*)(size_t)rb[1][(nb + u) & 3] + 256 * ((nb + u) >> 2)));
        bv[u] = __builtin_bit_cast(f16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int u = 0; u < 2; u++)
        acc_o[nb + u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[u], pL, acc_o[nb + u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 2; u++)
        acc_o[nb + u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[u], pA, acc_o[nb + u], 0, 0, 0);
    }
  };

  // The halves of a pair meet once per chunk (the partial-S exchange) through
  // LDS counters; the pairs run independently until the final merge.  A
  // wave rewrites its exchange buffer (pos & 1) two chunks later, after it
  // has seen its partner publish the chunk in between, which the partner
  // does only once it has read that buffer.
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
  // both halves of a pair hold the same chunk ids, so they run the same
  // iterations
  for (int pos = 0; cid0 < span; pos++) {
    pre(buf, ok_cur, idx_nxt, pos);
    pair_wait(pos);
    post(pos);
    cid0 = cid1;
    cid1 = cid2;
    cid2 = cid_of(pos + 3);
  }

  // ---- merge the four pairs (same heads and output dims, disjoint tokens)
  // Lane l keeps the merged statistics of head hh = l % 32 of the group: the
  // maximum M over the pairs' running maxima, the denominator L, and this
  // pair's weight exp2(m_pair - M); accumulator rows fetch them by lane.
  const bool single = a.splits == 1;
  const int hh = lane & 31;
  if (lost && lane == 0) __hip_atomic_store(failed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  sum_blocks(l_part[0], l_part[1]);
  if (g == 0) {
#pragma unroll
    for (int b = 0; b < 2; b++) {
      stat[(wave * 2 + 0) * 32 + 16 * b + n] = m_use[b];
      stat[(wave * 2 + 1) * 32 + 16 * b + n] = l_part[b];
    }
  }
  lds_sync_p();
  const bool wg_failed = *failed != 0u;
  float Mh, Lh, fown;
  {
    // every pair's statistics are read up front (reads under a branch would
    // wait for each one in turn); an empty pair (m = -inf) adds exactly zero
    float mp[kPairs], lp[kPairs];
#pragma unroll
    for (int p = 0; p < kPairs; p++) {
      mp[p] = stat[((2 * p + hf) * 2) * 32 + hh];
      lp[p] = stat[((2 * p + hf) * 2 + 1) * 32 + hh];
    }
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < kPairs; p++) M = fmaxf(M, mp[p]);
    float L = 0.f;
#pragma unroll
    for (int p = 0; p < kPairs; p++)
      L += mp[p] != -INFINITY ? lp[p] * __builtin_amdgcn_exp2f(mp[p] - M) : 0.f;
    Mh = M;
    Lh = L;
    // this wave's own running max of head hh is the value it posted
    const float mown = mp[pr];
    fown = (mown == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mown - M);
  }
  // this pair's weight: a lane's accumulators are all head hh's
  const float fr = fown;
  // Two rounds of pairwise sums through LDS (slots of 16 floats x 64 lanes,
  // lane-contiguous, over the first 128 KB): round 1 pairs p and p^1 (even p
  // keeps blocks 0..3, odd p 4..7), round 2 pairs p and p^2 (each keeps two
  // of its four blocks).
  auto put = [&](int slot, const f32x16& o) {
    lds_f32x4* d = reinterpret_cast<lds_f32x4*>(lds + slot * 4096) + lane;
#pragma unroll
    for (int rq = 0; rq < 4; rq++) d[rq * 64] = f32x4{o[4 * rq], o[4 * rq + 1], o[4 * rq + 2], o[4 * rq + 3]};
  };
  auto put_scaled = [&](int slot, const f32x16& o) {
    lds_f32x4* d = reinterpret_cast<lds_f32x4*>(lds + slot * 4096) + lane;
#pragma unroll
    for (int rq = 0; rq < 4; rq++)
      d[rq * 64] = f32x4{o[4 * rq] * fr, o[4 * rq + 1] * fr, o[4 * rq + 2] * fr, o[4 * rq + 3] * fr};
  };
  auto fma_add = [&](int slot, f32x16& o) {
    const lds_f32x4* d = reinterpret_cast<const lds_f32x4*>(lds + slot * 4096) + lane;
#pragma unroll
    for (int rq = 0; rq < 4; rq++) {
      const f32x4 t = d[rq * 64];
#pragma unroll
      for (int e = 0; e < 4; e++) o[4 * rq + e] = __builtin_fmaf(o[4 * rq + e], fr, t[e]);
    }
  };
  auto add = [&](int slot, f32x16& o) {
    const lds_f32x4* d = reinterpret_cast<const lds_f32x4*>(lds + slot * 4096) + lane;
#pragma unroll
    for (int rq = 0; rq < 4; rq++) {
      const f32x4 t = d[rq * 64];
      o[4 * rq] += t.x;
      o[4 * rq + 1] += t.y;
      o[4 * rq + 2] += t.z;
      o[4 * rq + 3] += t.w;
    }
  };
  // round 1 (which also applies each pair's weight): wave (p, hf) writes
  // the four blocks it gives away, weighted, into slots 4*wave .. 4*wave+3;
  // its partner (p^1, hf) is wave ^ 2
  auto round1 = [&](auto keep_c) {
    constexpr int kKeep = decltype(keep_c)::value;     // first kept block: 0 or 4
    constexpr int kGive = 4 - kKeep;
#pragma unroll
    for (int u = 0; u < 4; u++) put_scaled(4 * wave + u, acc_o[kGive + u]);
    lds_sync_p();
#pragma unroll
    for (int u = 0; u < 4; u++) fma_add(4 * (wave ^ 2) + u, acc_o[kKeep + u]);
    lds_sync_p();
  };
  if ((pr & 1) == 0) round1(IntC<0>{});
  else round1(IntC<4>{});
  // round 2: of its four blocks, wave (p, hf) keeps two and gives two; its
  // partner (p^2, hf) is wave ^ 4
  auto round2 = [&](auto keep_c, auto give_c) {
    constexpr int kKeep = decltype(keep_c)::value;
    constexpr int kGive = decltype(give_c)::value;
#pragma unroll
    for (int u = 0; u < 2; u++) put(2 * wave + u, acc_o[kGive + u]);
    lds_sync_p();
#pragma unroll
    for (int u = 0; u < 2; u++) add(2 * (wave ^ 4) + u, acc_o[kKeep + u]);
  };
  // blocks owned at the end: pair 0: 0,1; pair 1: 4,5; pair 2: 2,3; pair 3: 6,7
  // (two pairs: pair 0 keeps 0..3 and pair 1 4..7 after round 1)
  if constexpr (kPairs == 4) {
    switch (pr) {
      case 0: round2(IntC<0>{}, IntC<2>{}); break;
      case 1: round2(IntC<4>{}, IntC<6>{}); break;
      case 2: round2(IntC<2>{}, IntC<0>{}); break;
      default: round2(IntC<6>{}, IntC<4>{}); break;
    }
  }

  // ---- normalise and write this wave's output blocks.  Lane l holds head
  // tl's values at dv 256hf + 32nb + 8q + 4kg + 0..3 (q = 0..3) of each
  // block nb.  Packed to 16 bits and swapped between lane halves (the upper
  // 32 lanes' q = 2p values with the lower 32's q = 2p+1 ones), a lane holds 8
  // consecutive dv, 8q' + 0..7 with q' = 2p + kg, and stores them as 16 bytes.
  float inv;
  {
    float denom = Lh;
    if (single && a.sink != nullptr && Lh > 0.f) denom += __builtin_amdgcn_exp2f(sinkl[hh] * kLog2eP - Mh);
    inv = Lh > 0.f ? 1.0f / denom : 0.f;
    if (wg_failed) inv = __builtin_nanf("");
  }
  const size_t orow = (size_t)row * a.h_q + h0;
  const size_t prow = ((size_t)split * a.rows + row) * a.h_q + h0;
  auto store_block = [&](auto nb_c) {
    constexpr int kB = decltype(nb_c)::value;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    // two 16-bit values of run q, elements e, e+1
    auto pack = [&](int q, int e) -> uint32_t {
      const f32x2 v = {acc_o[kB][4 * q + e] * inv, acc_o[kB][4 * q + e + 1] * inv};
      return single ? __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2))
                    : __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    };
#pragma unroll
    for (int p2 = 0; p2 < 2; p2++) {
      // x: run 2p2 (lanes of kg 0: dv +0..3, kg 1: +4..7), y: run 2p2 + 1
      const auto s0 = __builtin_amdgcn_permlane32_swap(pack(2 * p2, 0), pack(2 * p2 + 1, 0), false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(pack(2 * p2, 2), pack(2 * p2 + 1, 2), false, false);
      // lanes of kg 0 now hold run 2p2's dv +0..7, lanes of kg 1 run 2p2+1's
      const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
      const int dv = 256 * hf + 32 * kB + 8 * (2 * p2 + kg);
      if (single)
        *reinterpret_cast<u32x4*>(a.out + (orow + tl) * kVDim + dv) = v;
      else
        // split partial in fp16: normalised within the split, so a convex
        // combination of V rows (|value| <= 6 * 448), rounded to nearest
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.o_part) + (prow + tl) * kVDim + dv) = v;
    }
  };
  auto store_pair = [&](auto nb_c) {
    constexpr int kB = decltype(nb_c)::value;
    store_block(IntC<kB>{});
    store_block(IntC<kB + 1>{});
  };
  if constexpr (kPairs == 4) {
    switch (pr) {
      case 0: store_pair(IntC<0>{}); break;
      case 1: store_pair(IntC<4>{}); break;
      case 2: store_pair(IntC<2>{}); break;
      default: store_pair(IntC<6>{}); break;
    }
  } else if (pr == 0) {
    store_pair(IntC<0>{});
    store_pair(IntC<2>{});
  } else {
    store_pair(IntC<4>{});
    store_pair(IntC<6>{});
  }
  if (wave == 0 && lane < 32) {
    float lse = Lh > 0.f ? (Mh + __log2f(Lh)) * kLn2P : -INFINITY;
    if (wg_failed) lse = __builtin_nanf("");
    if (single) a.lse[orow + hh] = lse;
    else a.lse_part[prow + hh] = lse;
  }
}

template <bool kDual, class F, int kPairs>
static hipError_t launch_w32_kernel(const DecodeArgs& a, int grid, hipStream_t stream) {
  constexpr size_t lds = LdsW32<kPairs>::kBytes;
  // the dynamic-LDS limit is raised once per device (setting it again, as two
  // threads may, is harmless)
  constexpr int kDevices = 64;
  static std::atomic<bool> attr_set[kDevices];
  int dev = 0;
  hipError_t ed = hipGetDevice(&dev);
  if (ed != hipSuccess) return ed;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_w32_kernel<kDual, F, kPairs>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL((decode_w32_kernel<kDual, F, kPairs>), dim3(grid), dim3(128 * kPairs), lds, stream, a);
  return hipSuccess;
}

template <bool kDual, class F>
static hipError_t launch_w32_pairs(const DecodeArgs& a, int grid, hipStream_t stream) {
  // Four pairs per workgroup (one per CU) when the launch is at most a few
  // workgroups per CU.  With many (a prefill), two pairs per workgroup and
  // two workgroups per CU: one workgroup's set-up and final merge then run
  // beside the other's chunk loop.
  if ((int64_t)grid >= 4 * (int64_t)a.num_cus) return launch_w32_kernel<kDual, F, 2>(a, grid, stream);
  return launch_w32_kernel<kDual, F, 4>(a, grid, stream);
}

hipError_t launch_decode_w32(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.rows * (a.h_q / 32) * a.splits;
  const bool f432 = a.pa.record_bytes == Fmt432::kBytes;
  hipError_t e0 = a.cache1 ? (f432 ? launch_w32_pairs<true, Fmt432>(a, grid, stream)
                                   : launch_w32_pairs<true, Fmt352>(a, grid, stream))
                           : (f432 ? launch_w32_pairs<false, Fmt432>(a, grid, stream)
                                   : launch_w32_pairs<false, Fmt352>(a, grid, stream));
  if (e0 != hipSuccess) return e0;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  // split partials are merged by the combine kernel: the launch boundary
  // makes them visible across XCDs without device-scope fences (on a
  // multi-XCD part those write back and invalidate L2)
  return launch_combine_f16(reinterpret_cast<const uint16_t*>(a.o_part), a.lse_part, a.splits, a.rows,
                            a.h_q, a.sink, a.out, a.lse, stream);
}

}  // namespace nvfp4
