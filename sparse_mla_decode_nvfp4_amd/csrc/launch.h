// Internal launchers behind the C ABI (include/nvfp4_mla.h).  Arguments are
// validated by the caller (api.cpp) before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace nvfp4 {

hipError_t launch_quantize_append(const uint16_t* latent, int64_t lstride,
                                  const uint16_t* rope, int64_t rstride,
                                  const int64_t* slot_mapping, int64_t num_tokens,
                                  uint8_t* cache, int64_t num_slots, const PageAddr& pa,
                                  bool f16_input, hipStream_t stream);

// The fused write path's prologue: RMSNorm of the latent and the rotary
// turn of the RoPE part, both rounded to bf16 before the write rule.
struct NormRope {
  const uint16_t* weight;   // [512] bf16 RMSNorm weight
  float eps;
  const float* cos_sin;     // [max_position, 64] fp32: cos of the 32 frequencies, then sin
  int64_t max_position;
  const int64_t* positions; // [num_tokens]
  int32_t neox;             // 1: pairs (i, i+32); 0: pairs (2i, 2i+1)
};

// Quantize-append of normalised and rotated bf16 inputs (one pass).
hipError_t launch_norm_rope_quantize_append(const uint16_t* latent, int64_t lstride,
                                            const uint16_t* rope, int64_t rstride,
                                            const NormRope& nr, const int64_t* slot_mapping,
                                            int64_t num_tokens, uint8_t* cache,
                                            int64_t num_slots, const PageAddr& pa,
                                            hipStream_t stream);

// The fused path's fp32 values before their bf16 rounding: out [n, 576] =
// [normalised latent (512) | rotated RoPE (64)] (test export).
hipError_t launch_norm_rope_f32(const uint16_t* latent, int64_t lstride, const uint16_t* rope,
                                int64_t rstride, const NormRope& nr, int64_t num_tokens,
                                float* out, hipStream_t stream);

hipError_t launch_dequantize_gather(const uint8_t* cache, int64_t num_slots, const PageAddr& pa,
                                    const int32_t* slots, int64_t n, uint16_t* out,
                                    hipStream_t stream);

// One decode call.  The joined top-k list of a row has `topk` positions:
// [0, topk0) are slot ids of `cache` (list `indices`, [rows, topk0]); in the
// dual-cache decode [topk0, topk) are slot ids of the extra cache `cache1`
// (list `indices1`, [rows, topk - topk0]), which has its own page geometry.
// Without an extra cache topk0 == topk and the *1 fields are unused.
struct DecodeArgs {
  const uint16_t* q;        // [rows, h_q, 576] bf16
  const uint8_t* cache;
  PageAddr pa;
  int64_t num_slots;
  const int32_t* indices;   // [rows, topk0]
  const uint8_t* cache1;    // extra cache, or null
  PageAddr pa1;
  int64_t num_slots1;
  const int32_t* indices1;  // [rows, topk - topk0]
  int32_t topk0;
  int32_t rows;             // batch * s_q
  int32_t s_q;              // query rows per sequence (consecutive rows)
  int32_t h_q;
  int32_t topk;             // length of the joined list
  const float* sink;        // [h_q] or null
  float scale_log2;         // softmax_scale * log2(e)
  uint16_t* out;            // [rows, h_q, 512] bf16
  float* lse;               // [rows, h_q]
  float* o_part;            // [splits, rows, h_q, 512] (splits > 1): fp32, or fp16
                            // in its first half from the 32-head kernel
  float* lse_part;          // [splits, rows, h_q]
  int32_t splits;
  int32_t num_cus;          // compute units of the device (picks the 32-head kernel's shape)
};

// Decode launch: head counts that are multiples of 32 run the 32-head-group
// kernel (decode_w32.hip), other head counts the 16-head tile kernel
// (decode.hip); with several splits the combine kernel merges their partials
// right after.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_w32(const DecodeArgs& a, hipStream_t stream);
bool decode_uses_w32(int32_t h_q);

hipError_t launch_combine(const float* o_part, const float* lse_part, int32_t splits,
                          int64_t rows, int32_t h_q, const float* sink, uint16_t* out,
                          float* lse, hipStream_t stream);
// The same merge over fp16 partials (the 32-head kernel's own workspace use).
hipError_t launch_combine_f16(const uint16_t* o_part, const float* lse_part, int32_t splits,
                              int64_t rows, int32_t h_q, const float* sink, uint16_t* out,
                              float* lse, hipStream_t stream);

}  // namespace nvfp4
