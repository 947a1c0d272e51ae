// Device-side helpers shared by the codec, dequantize-gather and decode
// kernels: the two record layouts, exact E2M1/E4M3 -> bf16 dequantization
// and slot -> record addressing.  gfx950 only.
//
// 352-byte record (FlashMLA PR #18 "W4A16 DSA: NVFP4 KV cache format for
// SM100 sparse decode", PR description): bytes [0,256) hold 512 E2M1 NoPE
// codes two per byte (element 2j in the low nibble of byte j), [256,320) 64
// unscaled E4M3 RoPE values, [320,352) 32 E4M3 block scales with the scale of
// 16-element block s at byte 320 + 8*(s&3) + (s>>2).
//
// 432-byte record (vLLM PR #82 "kv: nvfp4_ds_mla -- 4-bit NVFP4 KV cache for
// B12X sparse MLA (SM120)", summary and Fix): the same NoPE codes in [0,256),
// 32 E4M3 block scales in block order in [256,288), a zeroed 16-byte pad in
// [288,304), and 64 bf16 RoPE values copied verbatim in [304,432).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kNopeDim = 512;
constexpr int kRopeDim = 64;
constexpr int kQkDim = 576;
constexpr int kVDim = 512;
constexpr int kNopeBytes = 256;

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Byte of the scale area holding NoPE block s (the 8x4 -> 4x8 transpose).
__host__ __device__ constexpr int scale_byte(int s) { return 8 * (s & 3) + (s >> 2); }

// Record formats as compile-time traits.
struct Fmt352 {                      // E4M3 RoPE, permuted scales
  static constexpr int kBytes = 352;
  static constexpr int kScaleOff = 320;
  static constexpr int kRopeOff = 256;
  static constexpr bool kBf16Rope = false;
  __host__ __device__ static constexpr int scale_at(int s) { return kScaleOff + scale_byte(s); }
};
struct Fmt432 {                      // bf16 RoPE, scales in block order, 16-byte pad
  static constexpr int kBytes = 432;
  static constexpr int kScaleOff = 256;
  static constexpr int kPadOff = 288;
  static constexpr int kRopeOff = 304;
  static constexpr bool kBf16Rope = true;
  __host__ __device__ static constexpr int scale_at(int s) { return kScaleOff + s; }
};

// Two packed bf16 from the upper halves of two fp32 values.  Exact whenever
// both values are bf16-representable (true for every dequantized value).
__device__ __forceinline__ uint32_t pack_bf16_trunc(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Two E4M3 bytes (selected 16-bit word of `w`) -> two fp32, exact.  The
// scaled-convert's scale is 1.0, so its exponent-only scaling is the identity.
template <int kWord>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, kWord != 0);
}

// Two E4M3 bytes -> two packed bf16 (one dword), exact.
template <int kWord>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kWord != 0);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times
// one block scale -> eight bf16 (four dwords, element order).  Every product
// e2m1 * e4m3 has at most 6 significant bits and lies in [2^-10, 2688], so the
// fp32 products are exact and truncation to bf16 is exact.  The fp4 convert
// runs with scale 1.0 (its scale operand applies only an exponent).
__device__ __forceinline__ void dequant8(uint32_t nib, float scale, uint32_t out[4]) {
  f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 0);
  f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 1);
  f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 2);
  f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 3);
  out[0] = pack_bf16_trunc(a.x * scale, a.y * scale);
  out[1] = pack_bf16_trunc(b.x * scale, b.y * scale);
  out[2] = pack_bf16_trunc(c.x * scale, c.y * scale);
  out[3] = pack_bf16_trunc(d.x * scale, d.y * scale);
}

// Slot -> byte offset of its record in the paged cache.  Pages of
// `block_size` records of `record_bytes` each start every `block_stride`
// bytes.  Unpadded pages (stride = block_size * record_bytes) make the
// offset slot * record_bytes, one multiply; padded power-of-two page sizes
// use shift/mask; others use a 64-bit reciprocal (exact for every 32-bit
// slot: floor(n * ceil(2^64/d) / 2^64) == n / d).  The case flags are
// kernel arguments, so the choice is one uniform branch.
struct PageAddr {
  uint64_t block_stride;
  uint64_t recip;        // ceil(2^64 / block_size), unused for powers of two
  uint32_t block_size;
  uint32_t shift;        // log2(block_size) when pow2
  uint32_t pow2;
  uint32_t record_bytes; // 352 or 432
  uint32_t contig;       // block_stride == block_size * record_bytes
  uint32_t pad_;
  __device__ __forceinline__ uint64_t offset(uint32_t slot) const {
    if (contig) return (uint64_t)slot * record_bytes;
    uint32_t page, off;
    if (pow2) {
      page = slot >> shift;
      off = slot & (block_size - 1);
    } else if (block_size == 1) {
      page = slot;
      off = 0;
    } else {
      page = (uint32_t)__umul64hi((uint64_t)slot, recip);
      off = slot - page * block_size;
    }
    return (uint64_t)page * block_stride + (uint64_t)off * record_bytes;
  }
};

typedef _Float16 h16x2_t __attribute__((ext_vector_type(2)));

// P = hi + lo for a pair of fp32 values: hi = fp16(p) packed, lo = fp16(p -
// hi) packed.  p - hi is exact in fp32 (hi is p rounded to 11 significant
// bits), so each mixed-precision FMA (-1 * hi + p, hi read as fp16, rounded
// once to fp16) gives the same bits as subtracting in fp32 and converting:
// three instructions per pair instead of six.
__device__ __forceinline__ void split_p(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, h16x2_t));
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hi), "v"(p0));
  asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(r) : "v"(hi), "v"(p1));
  lo = r;
}

}  // namespace nvfp4
