// Quantize-append (write path) and dequantize-gather kernels for the 352- and
// 432-byte NVFP4 records.  gfx950.
//
// Write rule (vLLM PR #82 "kv: nvfp4_ds_mla -- 4-bit NVFP4 KV cache for B12X
// sparse MLA (SM120)", Fix and Tests; 352-byte layout from FlashMLA PR #18,
// PR description): per 16-element NoPE block, scale S = E4M3(amax/6) rounded
// to nearest-even and saturated at 448; each element's magnitude is rounded
// to the nearest E2M1 grid point of |x|/value(S) (ties to the even code, 0
// when the scale is 0), its sign copied.  The 352-byte record stores RoPE as
// unscaled E4M3 (RNE, saturating, sign kept); the 432-byte record copies the
// bf16 RoPE bits verbatim and zeroes its 16-byte pad.  Tokens whose slot is
// negative are skipped.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

// E4M3 code of a non-negative finite fp32 value, round-to-nearest-even on the
// finite grid, saturating to 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_rne_sat_mag(float q) {
  q = fminf(q, 448.0f);
  if (q < 0.015625f) {                       // below 2^-6: subnormal grid m * 2^-9
    return (uint32_t)__builtin_rintf(q * 512.0f);   // 8 -> 0x08 (= 2^-6) is right too
  }
  uint32_t b = __float_as_uint(q);
  b += 0x7FFFFu + ((b >> 20) & 1u);          // RNE of the mantissa to 3 bits
  return (b >> 20) - (120u << 3);            // rebias exponent 127 -> 7
}

// The block scale byte E4M3(amax / 6), rounded once from the exact quotient
// (ties to even, saturating at 448) without a division:
//   * q = amax * fl(1/6) is within 2^-23 of amax / 6, relative;
//   * a midpoint m of the E4M3 grid has at most 5 significant bits, so amax /
//     6 is a tie only when amax = 6 m exactly (6 m has at most 7 significant
//     bits); every other bf16 or fp16 amax (at most 11 significant bits)
//     differs from 6 m by at least 2^-11 relative;
//   * so rounding q to 16 significant bits returns every tie exactly and
//     leaves every other quotient on its side of every midpoint.
// The minimum comes first, so a NaN (or infinite) amax saturates to 448.
__device__ __forceinline__ uint32_t e4m3_scale_of_amax(float amax) {
  float q = fminf(amax * (1.0f / 6.0f), 448.0f);
  q = __uint_as_float((__float_as_uint(q) + 0x80u) & 0xFFFFFF00u);
  return e4m3_rne_sat_mag(q);
}

// The E2M1 code of x / s, rounded to nearest with ties to the even code,
// comes from the hardware fp32 -> E2M1 convert (round to nearest even,
// saturating at 6, sign kept, including for zero) applied to a quotient that
// rounds the same way as the exact x / s:
//   * q = |x| * r with r within one unit in the last place of 1/s is within
//     2^-21 of |x| / s for every quotient below 8;
//   * a tie t (a midpoint of the grid, .25 .. 5) has |x| = t s exactly, and
//     otherwise |x| and t s are different bf16 values (t s has at most 7
//     significant bits), at least 2^-8 t >= 2^-10 apart relative to s;
//   * so rounding q to a multiple of 2^-12 returns an exact tie exactly and
//     leaves every other quotient on its side of every tie.
// Quotients above 5 all give code 7 (the convert saturates) and stay finite
// for finite inputs (q <= amax / s, and s is amax / 6 rounded unless it
// saturates at 448), so they need no clamp: adding and removing 3072 leaves
// them above 5.  A zero scale gives q = 0 (code 0, sign kept).
__device__ __forceinline__ float e2m1_quotient(float x, float r) {
#pragma clang fp contract(off)
  float q = fabsf(x) * r;
  q = (q + 3072.0f) - 3072.0f;          // 3072 = 1.5 * 2^11: its ulp is 2^-12
  return __builtin_copysignf(q, x);
}

// A 16-bit input element (bf16, or fp16 when kF16) widened to fp32, exactly.
template <bool kF16>
__device__ __forceinline__ float widen16(uint32_t bits16) {
  if constexpr (kF16) return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  else return __uint_as_float(bits16 << 16);
}

// ---- the fused prologue: RMSNorm and rotary turn in binary32, each step
// rounded to nearest even (no fused multiply-add), then bf16 rounding.  The
// sum of squares has a fixed order: lane l adds the squares of its elements
// 8l..8l+7 in element order, then the 64 partial sums meet in a butterfly
// (neighbours first), which leaves every lane the same total.

// bf16 value nearest to a finite fp32 value (ties to even), as fp32.
__device__ __forceinline__ float round_bf16(float y) {
  uint32_t u = __float_as_uint(y);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xFFFF0000u);
}

// x[8] (elements 8l..8l+7 of one token's latent) <- x * w / sqrt(mean(x^2) + eps),
// before rounding.  Every lane of the wave takes part (the butterfly).
__device__ __forceinline__ void rms_norm8(float (&x)[8], const float (&w)[8], float eps) {
#pragma clang fp contract(off)
  float p = x[0] * x[0];
#pragma unroll
  for (int i = 1; i < 8; i++) p = p + x[i] * x[i];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) p = p + __shfl_xor(p, d);
  const float v = p * (1.0f / 512.0f) + eps;          // the scaling is exact
  const float r = 1.0f / __builtin_sqrtf(v);          // IEEE sqrt, IEEE divide
#pragma unroll
  for (int i = 0; i < 8; i++) x[i] = (x[i] * r) * w[i];
}

// One element of a rotated pair: a*c - b*s for the first element (xl = a,
// xp = b), b*c + a*s for the second (xl = b, xp = a).
__device__ __forceinline__ float rotate1(float xl, float xp, float c, float s, bool first) {
#pragma clang fp contract(off)
  const float u = xl * c;
  const float t = xp * s;
  return first ? u - t : u + t;
}

// Lane l's RoPE element after the turn for a token at `pos` (the table row is
// read only for a position inside the table; others give NaN).  The pair
// partner is lane l^1 (interleaved) or l^32 (neox); its frequency l>>1 or
// l&31.  Every lane of the wave takes part (the partner exchange).
__device__ __forceinline__ float rope_turn(float xl, int64_t pos, const NormRope& nr, int lane) {
  const int partner = nr.neox ? (lane ^ 32) : (lane ^ 1);
  const int freq = nr.neox ? (lane & 31) : (lane >> 1);
  const bool first = nr.neox ? lane < 32 : (lane & 1) == 0;
  const float xp = __shfl(xl, partner);
  const bool in_table = pos >= 0 && pos < nr.max_position;
  const float* row = nr.cos_sin + (in_table ? pos : 0) * 64;
  const float r = rotate1(xl, xp, row[freq], row[32 + freq], first);
  return in_table ? r : __builtin_nanf("");
}

// One wavefront per kTokW consecutive tokens; 4 waves per 256-thread block.
// Lane l quantizes NoPE elements [8l, 8l+8) (block l/2) and RoPE element l;
// each record is assembled in LDS and written with 16-byte stores (22 or 27).
// The input is bf16, or fp16 when kF16 (352-byte record only): every fp16 or
// bf16 value is exact in fp32, so the rounding below is the same for both.
constexpr int kTokW = 2;

// With kFused the tokens first go through the norm + rotary prologue and
// are rounded to bf16 (bf16 inputs only); a token whose position lies outside
// the table is skipped like an unmapped one.
template <bool kF16, class F, bool kFused = false>
__global__ void __launch_bounds__(256)
quantize_append_kernel(const uint16_t* __restrict__ latent, int64_t lstride,
                       const uint16_t* __restrict__ rope, int64_t rstride,
                       const int64_t* __restrict__ slot_mapping, int64_t num_tokens,
                       uint8_t* __restrict__ cache, int64_t num_slots, PageAddr pa,
                       NormRope nr) {
  static_assert(!(kF16 && F::kBf16Rope), "the 432-byte record holds bf16 RoPE");
  static_assert(!(kF16 && kFused), "the fused path takes bf16 inputs");
  __shared__ __attribute__((aligned(16))) uint8_t rec[4][F::kBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: token math in scalar registers
  const int lane = threadIdx.x & 63;
  const int64_t tok0 = ((int64_t)blockIdx.x * 4 + wave) * kTokW;
  if (tok0 >= num_tokens) return;
  // every token's slot, latent and RoPE are requested up front (one memory
  // round trip for the wave's tokens); a skipped token's record is built too
  // and only its store is dropped
  int64_t slot[kTokW];
  u32x4 raw[kTokW];
  uint32_t rbits[kTokW];
  int64_t pos[kTokW];
#pragma unroll
  for (int t = 0; t < kTokW; t++) {
    const int64_t tok = min(tok0 + t, num_tokens - 1);
    slot[t] = tok0 + t < num_tokens ? slot_mapping[tok] : -1;
    raw[t] = *reinterpret_cast<const u32x4*>(latent + tok * lstride + 8 * lane);
    rbits[t] = (uint32_t)rope[tok * rstride + lane];
    if constexpr (kFused) pos[t] = nr.positions[tok];
  }
  float wgt[8];
  if constexpr (kFused) {
    const u32x4 wr = *reinterpret_cast<const u32x4*>(nr.weight + 8 * lane);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      wgt[2 * i] = __uint_as_float(wr[i] << 16);
      wgt[2 * i + 1] = __uint_as_float(wr[i] & 0xFFFF0000u);
    }
  }
  uint8_t* r = rec[wave];
#pragma unroll
  for (int t = 0; t < kTokW; t++) {
    bool mapped = slot[t] >= 0 && slot[t] < num_slots;   // uniform over the wave
    // ---- NoPE: 8 elements per lane, two lanes per 16-element block
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      x[2 * i] = widen16<kF16>(raw[t][i] & 0xFFFFu);
      x[2 * i + 1] = widen16<kF16>(raw[t][i] >> 16);
    }
    float rv = widen16<kF16>(rbits[t]);
    if constexpr (kFused) {
      rms_norm8(x, wgt, nr.eps);
#pragma unroll
      for (int i = 0; i < 8; i++) x[i] = round_bf16(x[i]);
      rv = round_bf16(rope_turn(rv, pos[t], nr, lane));
      mapped = mapped && pos[t] >= 0 && pos[t] < nr.max_position;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const uint32_t scode = e4m3_scale_of_amax(amax);
    const float sv = e4m3x2_to_f32<0>(scode).x;
    const float rs = sv == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(sv);
    // codes 2i (low nibble) and 2i+1 of byte i
    uint32_t packed = 0;
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, e2m1_quotient(x[0], rs),
                                                      e2m1_quotient(x[1], rs), 1.0f, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, e2m1_quotient(x[2], rs),
                                                      e2m1_quotient(x[3], rs), 1.0f, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, e2m1_quotient(x[4], rs),
                                                      e2m1_quotient(x[5], rs), 1.0f, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, e2m1_quotient(x[6], rs),
                                                      e2m1_quotient(x[7], rs), 1.0f, 3);
    // the previous token's record has been read out of the staging area
    __builtin_amdgcn_wave_barrier();
    reinterpret_cast<uint32_t*>(r)[lane] = packed;
    if ((lane & 1) == 0) r[F::scale_at(lane >> 1)] = (uint8_t)scode;
    // ---- RoPE: lane l handles element l
    if constexpr (F::kBf16Rope) {
      // verbatim bf16 (the rounded turn in the fused path)
      reinterpret_cast<uint16_t*>(r + F::kRopeOff)[lane] =
          kFused ? (uint16_t)(__float_as_uint(rv) >> 16) : (uint16_t)rbits[t];
      if (lane < 4) reinterpret_cast<uint32_t*>(r + F::kPadOff)[lane] = 0u;
    } else {
      const uint32_t rcode = e4m3_rne_sat_mag(fabsf(rv)) | ((__float_as_uint(rv) >> 24) & 0x80u);
      r[F::kRopeOff + lane] = (uint8_t)rcode;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if (mapped && lane < F::kBytes / 16) {
      uint8_t* dst = cache + pa.offset((uint32_t)slot[t]);
      reinterpret_cast<u32x4*>(dst)[lane] = reinterpret_cast<const u32x4*>(r)[lane];
    }
  }
}

// One wavefront per output row: lane l dequantizes NoPE elements [8l, 8l+8)
// through the decode's own routine; lanes 0..7 produce the 64 RoPE values
// (E4M3 -> bf16, exact, or the stored bf16 bits).
template <class F>
__global__ void __launch_bounds__(256)
dequantize_gather_kernel(const uint8_t* __restrict__ cache, int64_t num_slots, PageAddr pa,
                         const int32_t* __restrict__ slots, int64_t n,
                         uint16_t* __restrict__ out) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: token math in scalar registers
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= n) return;
  const int32_t slot = slots[row];
  u32x4* dst = reinterpret_cast<u32x4*>(out + row * kQkDim);
  if (slot < 0 || (int64_t)slot >= num_slots) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    dst[lane] = z;
    if (lane < 8) dst[64 + lane] = z;
    return;
  }
  const uint8_t* src = cache + pa.offset((uint32_t)slot);
  const uint32_t nib = reinterpret_cast<const uint32_t*>(src)[lane];
  const int s = lane >> 1;
  const float sv = e4m3x2_to_f32<0>((uint32_t)src[F::scale_at(s)]).x;
  uint32_t o[4];
  dequant8(nib, sv, o);
  const u32x4 ov = {o[0], o[1], o[2], o[3]};
  dst[lane] = ov;
  if (lane < 8) {
    if constexpr (F::kBf16Rope) {
      dst[64 + lane] = reinterpret_cast<const u32x4*>(src + F::kRopeOff)[lane];
    } else {
      const u32x2 rb = reinterpret_cast<const u32x2*>(src + F::kRopeOff)[lane];
      const u32x4 rv = {e4m3x2_to_bf16x2<0>(rb.x), e4m3x2_to_bf16x2<1>(rb.x),
                        e4m3x2_to_bf16x2<0>(rb.y), e4m3x2_to_bf16x2<1>(rb.y)};
      dst[64 + lane] = rv;
    }
  }
}

hipError_t launch_quantize_append(const uint16_t* latent, int64_t lstride,
                                  const uint16_t* rope, int64_t rstride,
                                  const int64_t* slot_mapping, int64_t num_tokens,
                                  uint8_t* cache, int64_t num_slots, const PageAddr& pa,
                                  bool f16_input, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const dim3 grid((uint32_t)((num_tokens + 4 * kTokW - 1) / (4 * kTokW)));
  if (pa.record_bytes == Fmt432::kBytes) {
    if (f16_input) return hipErrorInvalidValue;    // rejected by the caller already
    hipLaunchKernelGGL((quantize_append_kernel<false, Fmt432>), grid, dim3(256), 0, stream,
                       latent, lstride, rope, rstride, slot_mapping, num_tokens, cache,
                       num_slots, pa, NormRope{});
  } else if (f16_input) {
    hipLaunchKernelGGL((quantize_append_kernel<true, Fmt352>), grid, dim3(256), 0, stream,
                       latent, lstride, rope, rstride, slot_mapping, num_tokens, cache,
                       num_slots, pa, NormRope{});
  } else {
    hipLaunchKernelGGL((quantize_append_kernel<false, Fmt352>), grid, dim3(256), 0, stream,
                       latent, lstride, rope, rstride, slot_mapping, num_tokens, cache,
                       num_slots, pa, NormRope{});
  }
  return hipGetLastError();
}

hipError_t launch_norm_rope_quantize_append(const uint16_t* latent, int64_t lstride,
                                            const uint16_t* rope, int64_t rstride,
                                            const NormRope& nr, const int64_t* slot_mapping,
                                            int64_t num_tokens, uint8_t* cache,
                                            int64_t num_slots, const PageAddr& pa,
                                            hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const dim3 grid((uint32_t)((num_tokens + 4 * kTokW - 1) / (4 * kTokW)));
  if (pa.record_bytes == Fmt432::kBytes)
    hipLaunchKernelGGL((quantize_append_kernel<false, Fmt432, true>), grid, dim3(256), 0, stream,
                       latent, lstride, rope, rstride, slot_mapping, num_tokens, cache,
                       num_slots, pa, nr);
  else
    hipLaunchKernelGGL((quantize_append_kernel<false, Fmt352, true>), grid, dim3(256), 0, stream,
                       latent, lstride, rope, rstride, slot_mapping, num_tokens, cache,
                       num_slots, pa, nr);
  return hipGetLastError();
}

// One wavefront per token: the fused prologue's fp32 results before their
// bf16 rounding (lane l: latent elements 8l..8l+7, RoPE element l).
__global__ void __launch_bounds__(256)
norm_rope_f32_kernel(const uint16_t* __restrict__ latent, int64_t lstride,
                     const uint16_t* __restrict__ rope, int64_t rstride, NormRope nr,
                     int64_t num_tokens, float* __restrict__ out) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: token math in scalar registers
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + wave;
  if (tok >= num_tokens) return;
  const u32x4 raw = *reinterpret_cast<const u32x4*>(latent + tok * lstride + 8 * lane);
  const u32x4 wr = *reinterpret_cast<const u32x4*>(nr.weight + 8 * lane);
  float x[8], w[8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = __uint_as_float(raw[i] << 16);
    x[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
    w[2 * i] = __uint_as_float(wr[i] << 16);
    w[2 * i + 1] = __uint_as_float(wr[i] & 0xFFFF0000u);
  }
  rms_norm8(x, w, nr.eps);
  const float rv = __uint_as_float((uint32_t)rope[tok * rstride + lane] << 16);
  const float turned = rope_turn(rv, nr.positions[tok], nr, lane);
  float* o = out + tok * kQkDim;
  reinterpret_cast<f32x4*>(o + 8 * lane)[0] = f32x4{x[0], x[1], x[2], x[3]};
  reinterpret_cast<f32x4*>(o + 8 * lane)[1] = f32x4{x[4], x[5], x[6], x[7]};
  o[kNopeDim + lane] = turned;
}

hipError_t launch_norm_rope_f32(const uint16_t* latent, int64_t lstride, const uint16_t* rope,
                                int64_t rstride, const NormRope& nr, int64_t num_tokens,
                                float* out, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const dim3 grid((uint32_t)((num_tokens + 3) / 4));
  hipLaunchKernelGGL(norm_rope_f32_kernel, grid, dim3(256), 0, stream, latent, lstride, rope,
                     rstride, nr, num_tokens, out);
  return hipGetLastError();
}

hipError_t launch_dequantize_gather(const uint8_t* cache, int64_t num_slots, const PageAddr& pa,
                                    const int32_t* slots, int64_t n, uint16_t* out,
                                    hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const dim3 grid((uint32_t)((n + 3) / 4));
  if (pa.record_bytes == Fmt432::kBytes)
    hipLaunchKernelGGL(dequantize_gather_kernel<Fmt432>, grid, dim3(256), 0, stream,
                       cache, num_slots, pa, slots, n, out);
  else
    hipLaunchKernelGGL(dequantize_gather_kernel<Fmt352>, grid, dim3(256), 0, stream,
                       cache, num_slots, pa, slots, n, out);
  return hipGetLastError();
}

}  // namespace nvfp4
