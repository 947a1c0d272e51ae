// Sparse MLA decode over 352-byte NVFP4 records, gfx950: the 16-head kernel
// (head counts that are not a multiple of 32).
//
// What it computes (FlashMLA PR #18 "W4A16 DSA: NVFP4 KV cache format for
// SM100 sparse decode", PR description): for each query row and head, gather
// the top-k token records by slot id (negative = invalid), dequantize them
// (NoPE = e2m1 * block scale, RoPE = e4m3), S = scale * Q K^T over the 576
// dims, softmax with an optional per-head sink, O = P V over the 512 NoPE
// dims, with fp32 accumulation.
//
// Kernel organisation (16 heads per workgroup, 4 waves, two workgroups per
// CU):
//   * a workgroup owns one query row, one group of 16 heads and one split of
//     the top-k list, and walks it in 64-token tiles; wave w loads and
//     dequantizes tokens [16w, 16w+16) of each tile;
//   * a lane loads the bytes of one token it needs straight from HBM (64
//     NoPE bytes, half the scale area, 16 RoPE values) and dequantizes them to
//     fp16 QK operands: every E2M1 x E4M3 product has at most 6 significant
//     bits and lies in [2^-10, 2688], so it is exact in fp16 (the codes
//     convert exactly, the scales convert exactly to fp16, one packed
//     multiply gives the product); K never visits LDS, the NoPE half goes to the
//     shared V tile (chunk-major: conflict-free row writes and transposed
//     reads at immediate offsets);
//   * Q is converted to fp16 once per wave with a per-head power-of-two scale
//     folded into the softmax scale (exact for every bf16 element within 2^31
//     of its head's largest);
//   * S^T = K Q^T per wave; the per-head tile maximum is exchanged through
//     LDS so every wave applies the same running max; P goes to two shared
//     tiles as fp16 hi + lo parts (PV runs on both, P carried to ~2^-22);
//   * wave w accumulates O[16 heads, dv 128w .. 128w+127] over all 64 tokens
//     of the tile (V read back with ds_read_b64_tr_b16), as O^T so that a
//     lane's 32 accumulators are one head's, and two workgroups fit per CU;
//   * indices are prefetched two tiles ahead and token bytes one tile ahead;
//   * the running max is only raised (and O rescaled) when a tile exceeds it
//     by more than 2^8, so rescales are rare.
// With several splits, each split writes its partial result (fp32 O
// normalised within the split, and its LSE) and the combine kernel, launched
// right after, merges them: the launch boundary makes the partials visible
// across XCDs, where an in-kernel merge needs device-scope fences that write
// back and invalidate L2.
#include <math.h>

#include "device_common.h"
#include "kv_source.h"
#include "launch.h"
#include "record_lanes.h"

namespace nvfp4 {

namespace {

typedef __attribute__((address_space(3))) uint8_t lds_b;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kTile = 16 * kWaves;          // tokens per tile
// V tile, chunk-major: chunk j (dims 8j .. 8j+7) holds the 64 tokens' 16-byte
// pieces contiguously, chunks kVChunk bytes apart.  kVChunk = 1088 (64 mod
// 256): a row write (16 lanes, consecutive tokens, one chunk) covers 256
// contiguous bytes, and each 32-lane half of a transposed read (tokens
// {0..3, 8..11} + 4i, two chunks, two 8-byte halves) hits 32 distinct 8-byte
// bank slots.  Every address is a base register plus an immediate.
constexpr int kVChunk = kTile * 16 + 64;
constexpr int kPRow = kTile + 8;            // padded LDS row of the P tile (fp16)
constexpr float kLazyThreshold = 8.0f;      // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m); }

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

}  // namespace

// Lane l of wave w: g = l/16 (lane group), n = l%16.
//   QK (16x16x32): A = K[token 16w+n][k-chunk g], B = Q^T[k-chunk g][head n],
//   C = S^T[token 16w+4g+r][head n].  K-step ks < 16 covers NoPE dims
//   16*(4c+g) + 8*(ks&1) + [0,8) with c = ks/2 for lane group g (so a lane's
//   blocks are {4c+g}, whose scales are the contiguous bytes 8g..8g+7);
//   ks 16, 17 cover RoPE dims 16g + 8*(ks-16) + [0,8).  Q is laid out to match.
//   PV (16x16x32), computed as O^T = V^T P^T: A = V^T[dv 128w + 16nb + n][token
//   32ks+8g+i], B = P^T[token 32ks+8g+i][head n], C = O^T[dv 128w + 16nb + 4g +
//   r][head n]: a lane's 32 accumulators all belong to head n.
template <bool kDual, class F>
__global__ void __launch_bounds__(64 * kWaves, 2)
decode_tile16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t vtile[64 * kVChunk];
  __shared__ __attribute__((aligned(16))) uint16_t ptile[16][kPRow];
  __shared__ __attribute__((aligned(16))) uint16_t ptile_lo[16][kPRow];   // P - fp16(P)
  __shared__ float tmax[kWaves][16];
  __shared__ float lsum[kWaves][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;

  // work unit (row, 16-head group, split).  Workgroups are dealt to the 8
  // XCDs round-robin by blockIdx; when the row count allows, every workgroup
  // of row r goes to XCD r % 8, so its head groups share the row's records
  // and the combine kernel finds its partials in that XCD's L2.  With several
  // query rows per sequence (and at least 8 sequences) the rows of sequence
  // q go to XCD q % 8 instead: they share their most recent tokens.
  const int hgroups = a.h_q >> 4;
  int split, hg, row;
  {
    const int x = blockIdx.x;
    if (a.s_q > 1 && a.rows % (8 * a.s_q) == 0) {
      int y = x >> 3;
      split = y % a.splits;
      y /= a.splits;
      hg = y % hgroups;
      const int r = y / hgroups;            // this XCD's r-th row
      row = ((r / a.s_q) * 8 + (x & 7)) * a.s_q + r % a.s_q;
    } else if ((a.rows & 7) == 0) {
      int y = x >> 3;
      split = y % a.splits;
      y /= a.splits;
      hg = y % hgroups;
      row = (y / hgroups) * 8 + (x & 7);
    } else {
      split = x % a.splits;
      const int unit = x / a.splits;
      hg = unit % hgroups;
      row = unit / hgroups;
    }
  }
  const int h0 = hg * 16;

  // token range of this split, in whole tiles
  const int ntiles_total = (a.topk + kTile - 1) / kTile;
  const int tiles_per_split = (ntiles_total + a.splits - 1) / a.splits;
  const int tile0 = split * tiles_per_split;
  const int tile1 = min(ntiles_total, tile0 + tiles_per_split);
  const int t_end = min(a.topk, tile1 * kTile);       // first token past the split
  const RowSource<kDual> src(a, row);
  const int my_tok = 16 * wave + n;                    // this lane's token within a tile
  // raw index of this lane's token of tile t (clamped in bounds: topk >= 1)
  auto load_idx = [&](int t) { return src.load(min(t * kTile + my_tok, a.topk - 1)); };
  auto resolve = [&](int32_t v, int t) {
    const int p = t * kTile + my_tok;
    return resolve_rec<kDual>(a, v, p < t_end, p, src.topk0);
  };

  // ---- prologue: indices of tiles 0 and 1, then this wave's Q elements
  // (their latency overlaps the indices'), then the token bytes of tile 0
  // once its indices are back; the Q set-up below overlaps their flight
  int tile = tile0;
  const int32_t idx0 = load_idx(tile);
  int32_t idx_nxt = load_idx(tile + 1);
  constexpr int kQPer = (18 + kWaves - 1) / kWaves;   // k-steps per wave, at most
  const uint16_t* qrow = a.q + ((size_t)row * a.h_q + h0 + n) * kQkDim;
  u32x4 raw[kQPer];
  // one unconditional load per k-step slot, its address picked without a
  // branch (a load under a branch makes the compiler wait for all earlier
  // loads, the record gathers included, before the next one); a wave with
  // fewer than kQPer k-steps loads an in-row element it does not use
#pragma unroll
  for (int i = 0; i < kQPer; i++) {
    const int ks = wave + kWaves * i;                 // uniform over the wave
    const int off = ks < 16 ? 16 * blk(g, ks >> 1) + 8 * (ks & 1)
                            : kNopeDim + 16 * g + 8 * min(ks - 16, 1);
    raw[i] = *reinterpret_cast<const u32x4*>(qrow + off);
  }
  const RecRef r0 = resolve(idx0, tile);
  bool ok_cur = r0.ok;             // this lane's token of the current tile takes part
  RawTok<F> cur;
  load_tok(cur, r0.ptr, g);

  // ---- Q^T operand registers (head n, k-chunk g) in fp16 with a per-head
  // power-of-two scale; a negative softmax scale flips Q's sign (exact), so
  // the score scale is positive.  The workgroup converts Q once: wave w
  // takes k-steps w, w+4, ..., the per-head maxima meet in LDS, the
  // operands are staged in the V tile (untouched until the first tile's
  // barrier) and every wave reads all 18 back.
  h16x8 qB[18];
  float qscale;          // |softmax_scale| * log2(e) * 2^p of head n
  {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < kQPer; i++)
      if (wave + kWaves * i < 18)
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const uint32_t x = raw[i][w];
          am = max(am, max((x << 16) & 0x7FFFFFFFu, x & 0x7FFF0000u));
        }
    am = max(am, (uint32_t)__shfl_xor((int)am, 16));
    am = max(am, (uint32_t)__shfl_xor((int)am, 32));
    // the loop's tile maxima reuse tmax only after the first tile's barrier
    if (g == 0) tmax[wave][n] = __uint_as_float(am);
    lds_barrier();
#pragma unroll
    for (int w = 0; w < kWaves; w++) am = max(am, __float_as_uint(tmax[w][n]));
    // largest magnitude's exponent e: scale by 2^-(e-14) so it lands in [2^14, 2^15)
    int e = (int)(am >> 23) - 127;
    if (am == 0 || am >= 0x7F800000u) e = 14;
    const int p = max(e - 14, -100);
    const float mul = a.scale_log2 < 0.f ? -__builtin_ldexpf(1.0f, -p) : __builtin_ldexpf(1.0f, -p);
    qscale = fabsf(a.scale_log2) * __builtin_ldexpf(1.0f, p);
    lds_b* const qst = (lds_b*)vtile;                   // [k-step][lane] x 16 bytes
#pragma unroll
    for (int i = 0; i < kQPer; i++) {
      const int ks = wave + kWaves * i;
      if (ks >= 18) continue;
      h16x8 v;
      if (F::kBf16Rope && ks >= 16) {
        // bf16 RoPE keys meet a bf16 Q operand (x * 2^-p is exact in bf16),
        // held in the same registers
        bf16x8 b;
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const uint32_t x = raw[i][w];
          b[2 * w] = (__bf16)(__uint_as_float(x << 16) * mul);
          b[2 * w + 1] = (__bf16)(__uint_as_float(x & 0xFFFF0000u) * mul);
        }
        v = __builtin_bit_cast(h16x8, b);
      } else {
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const uint32_t x = raw[i][w];
          v[2 * w] = (_Float16)(__uint_as_float(x << 16) * mul);
          v[2 * w + 1] = (_Float16)(__uint_as_float(x & 0xFFFF0000u) * mul);
        }
      }
      *reinterpret_cast<__attribute__((address_space(3))) h16x8*>(qst + (ks * 64 + lane) * 16) = v;
    }
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < 18; ks++)
      qB[ks] = *reinterpret_cast<const __attribute__((address_space(3))) h16x8*>(qst + (ks * 64 + lane) * 16);
  }

  f32x4 acc_o[8];
#pragma unroll
  for (int nb = 0; nb < 8; nb++) acc_o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running max (log2 units) of head n; every wave derives it from the same
  // LDS values, so they agree, and lane 4g+r holds that of O row 4g+r
  float m_n = -INFINITY;
  float l_part = 0.f;          // this lane's share of head n's denominator

  // V tile addresses.  Write (k-step 2c+h): chunk 2 blk(g, c) + h = 16g + 2c
  // + h, token my_tok.  Read (PV k-step ks, half hb, block nb): token 32ks +
  // 8g + 4hb + (l%16)/4, chunk 16w + 2nb + ((l%4)>>1), byte 8(l&1).
  const uint32_t vw_base = (uint32_t)(size_t)(vtile + 2 * blk(g, 0) * kVChunk + my_tok * 16);
  const uint32_t vr_base = (uint32_t)(size_t)(vtile + (16 * wave + ((lane & 3) >> 1)) * kVChunk +
                                             (8 * g + ((lane >> 2) & 3)) * 16 + 8 * (lane & 1));

  // One tile step.  `cur` holds this lane's bytes of tile t, `nxt` receives
  // tile t+1's; the loop below alternates the two buffers so the prefetched
  // bytes are never copied.
  auto step = [&](RawTok<F>& cur, RawTok<F>& nxt, int t) {
    // ---- prefetch: indices two tiles ahead, token bytes one tile ahead.
    // The scale and RoPE bytes are requested here and each NoPE piece inside
    // the dequant loop below: the eight waves of a CU reach this point
    // together after a barrier, and issuing all their gathers at once backs
    // up the address unit for thousands of cycles.
    const int32_t idx_nn = load_idx(t + 2);
    const RecRef rn = resolve(idx_nxt, t + 1);
    load_tok_tail(nxt, rn.ptr, g);
    const bool cur_valid = ok_cur;
    const uint64_t vmask = __ballot(cur_valid);

    // all waves are done reading the previous tile's V and P
    lds_barrier();
    // ---- dequantize this wave's 16 tokens k-step by k-step: each K operand
    // goes to the V tile (NoPE) and straight into S^T = K Q^T (two
    // accumulation chains)
    const u32x2 bsc = block_scales(cur, g);
    const uint32_t scx = cur_valid ? bsc.x : 0u;
    const uint32_t scy = cur_valid ? bsc.y : 0u;
    // the eight block scales as fp16 (exact), two per convert
    const h16x2 sp[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scx, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scx, 1.0f, true),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scy, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scy, 1.0f, true)};
    f32x4 s_acc = {0.f, 0.f, 0.f, 0.f}, s_acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const _Float16 sv = sp[c >> 1][c & 1];
      const h16x2 Fs = {sv, sv};
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const h16x8 k = dequant8_f16(nope_word(cur, c, h), Fs);
        *reinterpret_cast<__attribute__((address_space(3))) h16x8*>(
            (lds_b*)(size_t)vw_base + (2 * c + h) * kVChunk) = k;
        if (h == 0) s_acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k, qB[2 * c], s_acc, 0, 0, 0);
        else s_acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k, qB[2 * c + 1], s_acc1, 0, 0, 0);
      }
      if (c & 1) {
        load_tok_nope(nxt, rn.ptr, g, c >> 1);
        __builtin_amdgcn_sched_barrier(0);  // keep the gathers spread out
      }
    }
    if constexpr (F::kBf16Rope) {
      s_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.rope[0]),
                                                     __builtin_bit_cast(bf16x8, qB[16]), s_acc, 0, 0, 0);
      s_acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.rope[1]),
                                                      __builtin_bit_cast(bf16x8, qB[17]), s_acc1, 0, 0, 0);
    } else {
      s_acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(rope8_f16(cur.rope.x, cur.rope.y), qB[16], s_acc, 0, 0, 0);
      s_acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(rope8_f16(cur.rope.z, cur.rope.w), qB[17], s_acc1, 0, 0, 0);
    }
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; r++)
      s[r] = ((vmask >> (4 * g + r)) & 1ull) ? (s_acc[r] + s_acc1[r]) * qscale : -INFINITY;
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    bm = fmaxf(bm, shfl_xor(bm, 16));
    bm = fmaxf(bm, shfl_xor(bm, 32));
    if (g == 0) tmax[wave][n] = bm;

    // ---- P for this wave's tokens -> P tiles (fp16 hi + lo parts, so PV
    // carries P to about 2^-22), computed with the running max as it stands.
    // It stays valid unless the tile raises the max; the barrier below posts
    // every wave's tile maxima with the P and V tiles, and only a raise (the
    // same decision in every wave, a rare event after the first tile) pays
    // for recomputing P and a second barrier.
    float p[4];
    auto write_p = [&]() {
      const float m_safe = (m_n == -INFINITY) ? 0.f : m_n;   // s = -inf -> p = 0
#pragma unroll
      for (int r = 0; r < 4; r++) p[r] = fast_exp2(s[r] - m_safe);
      uint32_t hi[2], lo[2];
      split_p(p[0], p[1], hi[0], lo[0]);
      split_p(p[2], p[3], hi[1], lo[1]);
      *reinterpret_cast<u32x2*>(&ptile[n][16 * wave + 4 * g]) = u32x2{hi[0], hi[1]};
      *reinterpret_cast<u32x2*>(&ptile_lo[n][16 * wave + 4 * g]) = u32x2{lo[0], lo[1]};
    };
    write_p();
    lds_barrier();                        // maxima, P and V tiles complete

    // ---- running max update (same rule in every wave), lazy O rescale:
    // every accumulator of a lane is head n's
    float tm_n = tmax[0][n];
#pragma unroll
    for (int w = 1; w < kWaves; w++) tm_n = fmaxf(tm_n, tmax[w][n]);
    const bool raise = tm_n > m_n + kLazyThreshold;
    if (__any(raise)) {
      // every wave holds the same m_n and reads the same maxima, so every
      // wave takes this branch or none does
      float alpha_n = 1.0f;
      if (raise) {
        alpha_n = fast_exp2(m_n - tm_n);  // m_n = -inf gives 0 (l_part and O are 0 then)
        l_part *= alpha_n;
        m_n = tm_n;
      }
#pragma unroll
      for (int nb = 0; nb < 8; nb++)
#pragma unroll
        for (int r = 0; r < 4; r++) acc_o[nb][r] *= alpha_n;
      write_p();
      lds_barrier();                      // P tiles rewritten
    }
    l_part += (p[0] + p[1]) + (p[2] + p[3]);

    // ---- O[:, 128w .. 128w+127] += P V over the tile's 64 tokens
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const h16x8 pa = *reinterpret_cast<const h16x8*>(&ptile[n][32 * ks + 8 * g]);
      const h16x8 pl = *reinterpret_cast<const h16x8*>(&ptile_lo[n][32 * ks + 8 * g]);
      // two blocks at a time: both lo products, then both hi products
#pragma unroll
      for (int nb = 0; nb < 8; nb += 2) {
        h16x8 bv[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
          lds_b* const rb = (lds_b*)(size_t)vr_base + 2 * (nb + u) * kVChunk + 32 * ks * 16;
          const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)rb);
          const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(rb + 4 * 16));
          bv[u] = __builtin_bit_cast(h16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int u = 0; u < 2; u++)
          acc_o[nb + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv[u], pl, acc_o[nb + u], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 2; u++)
          acc_o[nb + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv[u], pa, acc_o[nb + u], 0, 0, 0);
      }
    }
    ok_cur = rn.ok;
    idx_nxt = idx_nn;
    // keep the next step's index checks out of this step's PV: there they
    // wait for the index load issued at the top of this step
    __builtin_amdgcn_sched_barrier(0);
  };

  RawTok<F> other;
  for (; tile + 1 < tile1; tile += 2) {
    step(cur, other, tile);
    step(other, cur, tile + 1);
  }
  if (tile < tile1) step(cur, other, tile);

  // ---- epilogue: denominators over lanes and waves, normalise, write.
  // The sink logit of this lane's head is requested first, and the barriers
  // order LDS only (the last tile's unused prefetch need not land first).
  const float skv = (a.splits == 1 && a.sink != nullptr) ? a.sink[h0 + n] : 0.f;
  float lt = l_part;
  lt += shfl_xor(lt, 16);
  lt += shfl_xor(lt, 32);
  lds_barrier();                                  // every wave is done with the tiles
  if (g == 0) lsum[wave][n] = lt;
  lds_barrier();
  const size_t orow = (size_t)row * a.h_q + h0;
  const size_t prow = ((size_t)split * a.rows + row) * a.h_q + h0;
  const float lh = lsum[0][n] + lsum[1][n] + lsum[2][n] + lsum[3][n];
  float inv;
  {
    float denom = lh;
    if (a.splits == 1 && a.sink != nullptr && lh > 0.f) denom += exp2f(skv * kLog2e - m_n);
    inv = lh > 0.f ? 1.0f / denom : 0.f;
  }
  // Lane (n, g) holds head n's values at dv 128w + 16nb + 4g + 0..3 of each
  // block nb.  As fp32 partials they are stored as 16 bytes per block; as
  // bf16, blocks nb and nb+1 are packed and swapped between neighbouring
  // lane groups (odd groups' block nb with even groups' block nb+1), so that
  // a lane holds 8 consecutive dv, 16 bytes: block nb + (g & 1), dv
  // 16nb' + 8(g >> 1) + 0..7.
  if (a.splits == 1) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    auto pack = [&](int nb, int e) -> uint32_t {
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(
          f32x2{acc_o[nb][e] * inv, acc_o[nb][e + 1] * inv}, bf16x2));
    };
#pragma unroll
    for (int nb = 0; nb < 8; nb += 2) {
      const auto s0 = __builtin_amdgcn_permlane16_swap(pack(nb, 0), pack(nb + 1, 0), false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(pack(nb, 2), pack(nb + 1, 2), false, false);
      const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
      const int dv = 128 * wave + 16 * (nb + (g & 1)) + 8 * (g >> 1);
      *reinterpret_cast<u32x4*>(a.out + (orow + n) * kVDim + dv) = v;
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < 8; nb++) {
      const f32x4 v = {acc_o[nb][0] * inv, acc_o[nb][1] * inv, acc_o[nb][2] * inv, acc_o[nb][3] * inv};
      *reinterpret_cast<f32x4*>(a.o_part + (prow + n) * kVDim + 128 * wave + 16 * nb + 4 * g) = v;
    }
  }
  if (wave == 0 && g == 0) {
    const float lse = lh > 0.f ? (m_n + log2f(lh)) * kLn2 : -INFINITY;
    if (a.splits == 1) a.lse[orow + n] = lse;
    else a.lse_part[prow + n] = lse;
  }
}

bool decode_uses_w32(int32_t h_q) { return h_q % 32 == 0; }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  if (decode_uses_w32(a.h_q)) return launch_decode_w32(a, stream);
  const int grid = a.rows * (a.h_q / 16) * a.splits;
  const bool f432 = a.pa.record_bytes == Fmt432::kBytes;
  if (a.cache1 && f432)
    hipLaunchKernelGGL((decode_tile16_kernel<true, Fmt432>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  else if (a.cache1)
    hipLaunchKernelGGL((decode_tile16_kernel<true, Fmt352>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  else if (f432)
    hipLaunchKernelGGL((decode_tile16_kernel<false, Fmt432>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_tile16_kernel<false, Fmt352>), dim3(grid), dim3(64 * kWaves), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_combine(a.o_part, a.lse_part, a.splits, a.rows, a.h_q, a.sink, a.out, a.lse, stream);
}

}  // namespace nvfp4
