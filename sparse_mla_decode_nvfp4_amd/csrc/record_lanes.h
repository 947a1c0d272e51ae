// Per-lane gather and dequantization of token records for the decode
// kernels whose lane (n, g) of a wave takes token n's NoPE blocks 8g..8g+7,
// their block scales and RoPE elements 16g..16g+15 (both record widths), and
// turns them into fp16 MFMA operands.  gfx950.
#pragma once

#include "device_common.h"

namespace nvfp4 {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

// The bytes one lane needs of one token record.  Lane group g takes NoPE
// blocks 8g .. 8g+7: 64 contiguous bytes, four 16-byte loads (few, wide
// gathers: the address unit, not HBM, limits this kernel's loads).  In the
// 432-byte record their scales are the eight bytes 256 + 8g .. (block
// order).  In the 352-byte record block s's scale sits at 320 + 8(s&3) +
// (s>>2), so the lane's scales are the 16-bit words at 320 + 8k + 2g (k =
// 0..3): word k holds blocks 8g+k (low byte) and 8g+4+k (high byte), in
// scale dword 2k + (g>>1).  Lanes 0..31 (g = 0, 1) load scale dwords 0..3 and
// lanes 32..63 dwords 4..7, one 16-byte gather each; a swap between the lane
// halves then leaves every lane the four dwords of its parity.
template <class F>
struct RawTok;
template <>
struct RawTok<Fmt352> {
  u32x4 nope[4];         // NoPE bytes 64g + 16i .. +15
  u32x4 sc;              // scale area bytes 16(g>>1) .. +15
  u32x4 rope;            // RoPE elements 16g .. 16g+15 (E4M3)
};
template <>
struct RawTok<Fmt432> {
  u32x4 nope[4];
  u32x2 scale;           // scale bytes 8g .. 8g+7 (= blocks 8g .. 8g+7)
  u32x4 rope[2];         // RoPE elements 16g .. 16g+15 (bf16)
};

// NoPE block of lane group g's c-th k-step pair.
__device__ __forceinline__ int blk(int g, int c) { return 8 * g + c; }

// Scale bytes of blocks 8g .. 8g+3 (x) and 8g+4 .. 8g+7 (y), one byte each.
__device__ __forceinline__ u32x2 block_scales(const RawTok<Fmt432>& t, int) { return t.scale; }
__device__ __forceinline__ u32x2 block_scales(const RawTok<Fmt352>& t, int g) {
  // Lane halves swap dwords 1 and 3 of the lower half's load with dwords 0
  // and 2 of the upper half's: afterwards scale dword 2k + (g>>1) is word k of
  // every lane (the lower half keeps the even dwords, the upper the odd).
  const auto s01 = __builtin_amdgcn_permlane32_swap(t.sc.x, t.sc.y, false, false);
  const auto s23 = __builtin_amdgcn_permlane32_swap(t.sc.z, t.sc.w, false, false);
  const uint32_t sh = 16u * (uint32_t)(g & 1);
  const uint32_t w0 = s01[0] >> sh;
  const uint32_t w1 = s23[0] >> sh;
  const uint32_t w2 = s01[1] >> sh;
  const uint32_t w3 = s23[1] >> sh;
  // byte i of perm(a, b, sel) is byte sel_i of the 8-byte value {a : b}
  const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x0c0c0400u) |
                      (__builtin_amdgcn_perm(w3, w2, 0x0c0c0400u) << 16);
  const uint32_t hi = __builtin_amdgcn_perm(w1, w0, 0x0c0c0501u) |
                      (__builtin_amdgcn_perm(w3, w2, 0x0c0c0501u) << 16);
  return u32x2{lo, hi};
}

// The dword holding codes 8h .. 8h+7 of block 8g + c.
template <class F>
__device__ __forceinline__ uint32_t nope_word(const RawTok<F>& t, int c, int h) {
  const u32x4& q = t.nope[c >> 1];
  return (c & 1) ? (h ? q.w : q.z) : (h ? q.y : q.x);
}

// Unconditional loads (uniform control flow keeps the prefetch in flight:
// after a divergent load the compiler can only wait for every outstanding
// load).  Invalid tokens read record 0, which always exists; their scale
// bytes are zeroed when consumed, so their NoPE values are exact zeros and
// cannot carry NaN into P V, and their scores are masked.
template <class F>
__device__ __forceinline__ void load_tok_nope(RawTok<F>& t, const uint8_t* rec, int g, int i) {
  t.nope[i] = *reinterpret_cast<const u32x4*>(rec + 64 * g + 16 * i);
}
template <class F>
__device__ __forceinline__ void load_tok_tail(RawTok<F>& t, const uint8_t* rec, int g) {
  if constexpr (F::kBf16Rope) {
    t.scale = *reinterpret_cast<const u32x2*>(rec + F::kScaleOff + 8 * g);
    t.rope[0] = *reinterpret_cast<const u32x4*>(rec + F::kRopeOff + 32 * g);
    t.rope[1] = *reinterpret_cast<const u32x4*>(rec + F::kRopeOff + 32 * g + 16);
  } else {
    t.sc = *reinterpret_cast<const u32x4*>(rec + F::kScaleOff + 16 * (g >> 1));
    t.rope = *reinterpret_cast<const u32x4*>(rec + F::kRopeOff + 16 * g);
  }
}
template <class F>
__device__ __forceinline__ void load_tok(RawTok<F>& t, const uint8_t* rec, int g) {
#pragma unroll
  for (int i = 0; i < 4; i++) load_tok_nope(t, rec, g, i);
  load_tok_tail(t, rec, g);
}

// Eight E2M1 codes times a block scale -> eight fp16, exact: the codes
// convert exactly, the scale is an E4M3 value held exactly in fp16, and their
// product has at most 6 significant bits in [2^-10, 2688].  F holds the
// scale in both halves (a half-select of a packed pair of scales).
__device__ __forceinline__ h16x8 dequant8_f16(uint32_t w, h16x2 F) {
  const h16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * F;
  const h16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * F;
  const h16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * F;
  const h16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * F;
  return h16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Eight E4M3 RoPE bytes -> eight fp16 (exact).
__device__ __forceinline__ h16x8 rope8_f16(uint32_t x, uint32_t y) {
  const h16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
  const h16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
  const h16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y, 1.0f, false);
  const h16x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y, 1.0f, true);
  return h16x8{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
}

}  // namespace nvfp4
