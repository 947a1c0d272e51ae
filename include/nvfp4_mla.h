/*
 * nvfp4_mla.h -- C ABI of the MI355X (gfx950) NVFP4 sparse-MLA decode library.
 *
 * Operations (sources named by page title and section):
 *   - quantize-append: writes 352-byte NVFP4 token records into a paged KV
 *     cache by slot id.  Record layout from FlashMLA PR #18 "W4A16 DSA: NVFP4
 *     KV cache format for SM100 sparse decode", PR description; scale rule
 *     E4M3(group_amax/6) and the slot-mapping convention from vLLM PR #82
 *     "kv: nvfp4_ds_mla -- 4-bit NVFP4 KV cache for B12X sparse MLA (SM120)",
 *     Fix and Tests sections.
 *   - sparse decode: gathers top-k records by slot id (-1 = invalid),
 *     dequantizes them to bf16, and computes softmax(scale * Q K^T) V over all
 *     heads sharing the latent, with an optional per-head attention sink;
 *     d_qk = 576, d_v = 512 (FlashMLA PR #18, PR description).  Returns O and
 *     the log-sum-exp LSE.  The dual-cache form attends over two lists in two
 *     caches with one softmax.
 *   - combine: LSE-weighted merge of split-KV partial results.
 *   - dequantize-gather: the decode's own dequantization, exported so its
 *     bf16 output can be checked bit for bit.
 *
 * The 352-byte record ("nvfp4.fp8rope"):
 *   [0,256)   512 E2M1 NoPE codes, element 2j in the low nibble of byte j
 *   [256,320) 64 E4M3 RoPE values, no scale
 *   [320,352) 32 E4M3 block scales (16 NoPE elements each); the scale of
 *             block s is at byte 320 + 8*(s&3) + (s>>2)
 *
 * The 432-byte record ("nvfp4_ds_mla", vLLM PR #82, summary and Fix; the
 * *_ds_mla entry points):
 *   [0,256)   512 E2M1 NoPE codes, packed as above
 *   [256,288) 32 E4M3 block scales in block order (block s at byte 256 + s)
 *   [288,304) zero pad
 *   [304,432) 64 bf16 RoPE values, copied verbatim from the input
 * Both records use the same NoPE codes and scales for the same latent.
 *
 * Conventions for every entry point:
 *   - All pointers are device pointers owned by the caller unless stated
 *     otherwise; the library never allocates, frees or retains them.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     on it and the call returns without synchronising; no host<->device
 *     copies and no allocations happen inside, so calls may be captured
 *     into a HIP graph.
 *   - Paged cache: `num_blocks` pages of `block_size` tokens; page p starts
 *     `block_stride_bytes` after page p-1; a token record is 352 bytes and
 *     records within a page are contiguous.  slot = page*block_size + offset.
 *     The cache base and block_stride_bytes must be multiples of 16 and
 *     block_stride_bytes >= block_size * 352.
 *   - bf16 tensors are IEEE bfloat16 bit patterns (uint16) in row-major
 *     order with the layouts stated per call.
 *   - Return value: NVFP4_MLA_OK (0) or a negative error code; arguments are
 *     validated before any HIP call, and a human-readable message for the
 *     last error of the calling thread is available from
 *     nvfp4_mla_last_error().  NVFP4_MLA_ERR_HIP reports a failed launch.
 */
#ifndef NVFP4_MLA_H
#define NVFP4_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle, declared as hip_runtime_api.h declares it (so either
 * header may be included first); NULL is the null stream. */
typedef struct ihipStream_t* hipStream_t;

#define NVFP4_MLA_ABI_VERSION 1

#define NVFP4_MLA_RECORD_BYTES 352
/* The 432-byte "nvfp4_ds_mla" record (the *_ds_mla entry points). */
#define NVFP4_MLA_DS_MLA_RECORD_BYTES 432
#define NVFP4_MLA_NOPE_DIM 512
#define NVFP4_MLA_ROPE_DIM 64
#define NVFP4_MLA_QK_DIM 576
#define NVFP4_MLA_V_DIM 512
/* Largest number of split-KV partitions a decode accepts. */
#define NVFP4_MLA_MAX_SPLITS 64

enum nvfp4_mla_status {
  NVFP4_MLA_OK = 0,
  NVFP4_MLA_ERR_INVALID_ARGUMENT = -1,   /* null/misaligned pointer, bad size */
  NVFP4_MLA_ERR_UNSUPPORTED_FORMAT = -2, /* record size or head dims differ */
  NVFP4_MLA_ERR_UNSUPPORTED_DEVICE = -3, /* no device, or not gfx950 */
  NVFP4_MLA_ERR_WORKSPACE_TOO_SMALL = -4,
  NVFP4_MLA_ERR_HIP = -5                 /* a HIP call or launch failed */
};

/* ABI version of the loaded library (NVFP4_MLA_ABI_VERSION). */
int nvfp4_mla_abi_version(void);

/* Message describing the calling thread's most recent error ("" if none).
 * The string is owned by the library and valid until the thread's next call. */
const char* nvfp4_mla_last_error(void);

/* Checks that record_bytes / nope / rope / v dimensions are ones this
 * library implements (352 or 432 / 512 / 64 / 512) -- the shape-based format
 * dispatch of FlashMLA PR #18 reduced to these two records.  Returns
 * NVFP4_MLA_OK or NVFP4_MLA_ERR_UNSUPPORTED_FORMAT.  Host-only; never
 * touches the device. */
int nvfp4_mla_check_format(int32_t record_bytes, int32_t nope_dim,
                           int32_t rope_dim, int32_t v_dim);

/*
 * Quantize-append (write path).  For each token n with slot_mapping[n] >= 0,
 * writes its 352-byte record at that slot: per 16-element NoPE block,
 * scale = E4M3(amax/6) (round-to-nearest-even, saturating at 448), codes =
 * round-to-nearest-even E2M1 of x/scale (ties to the even code, sign kept,
 * 0 when the scale is 0), RoPE = unscaled round-to-nearest-even E4M3 with
 * the sign kept (vLLM PR #82, Fix and Tests; FlashMLA PR #18, record layout).
 *
 *   latent_bf16       [num_tokens, >= 512] bf16; row n starts at
 *                     n * latent_row_stride elements; 16-byte aligned rows
 *   rope_bf16         [num_tokens, >= 64] bf16, row stride rope_row_stride
 *                     elements; 16-byte aligned rows
 *   slot_mapping      [num_tokens] int64; < 0 skips the token; mapped slots
 *                     must be distinct (duplicates race); >= num_blocks *
 *                     block_size is skipped as well
 *   kv_cache          paged cache (see conventions); bytes of unmapped slots
 *                     are never written
 * num_tokens == 0 is a no-op.  Inputs must be finite.
 */
int nvfp4_mla_quantize_append(const void* latent_bf16, int64_t latent_row_stride,
                              const void* rope_bf16, int64_t rope_row_stride,
                              const int64_t* slot_mapping, int64_t num_tokens,
                              uint8_t* kv_cache, int64_t num_blocks,
                              int32_t block_size, int64_t block_stride_bytes,
                              hipStream_t stream);

/*
 * Quantize-append from fp16 inputs: the same write rule and 352-byte record
 * as nvfp4_mla_quantize_append, with latent and RoPE given as IEEE fp16
 * instead of bf16 (the write kernel of vLLM PR #82 is dispatched over both
 * 16-bit float types: the review thread on its host launch).  Every fp16
 * value is exact in fp32, so the scale, code and RoPE rounding is the one
 * stated above, applied to the fp16 values.  Arguments, layouts, alignment,
 * ownership, skipping and errors are those of nvfp4_mla_quantize_append.
 */
int nvfp4_mla_quantize_append_fp16(const void* latent_fp16, int64_t latent_row_stride,
                                   const void* rope_fp16, int64_t rope_row_stride,
                                   const int64_t* slot_mapping, int64_t num_tokens,
                                   uint8_t* kv_cache, int64_t num_blocks,
                                   int32_t block_size, int64_t block_stride_bytes,
                                   hipStream_t stream);

/*
 * Fused norm + rotary + quantize-append: one pass that normalises the latent,
 * turns the RoPE part, rounds both to bf16 and writes the records by the rule
 * of nvfp4_mla_quantize_append -- the store sglang PR #38646 "[SM120] opt-in
 * NVFP4 sparse-MLA KV cache format for DeepSeek-V4" lists as missing under
 * Limitations (without it the path pays a bf16 intermediate plus a separate
 * quantize kernel).  Per token n with slot_mapping[n] >= 0 and
 * 0 <= positions[n] < max_position:
 *     y   = RMSNorm(latent[n]) = latent[n] * w / sqrt(mean(latent[n]^2) + eps)
 *     k   = RoPE part turned by the angles of row positions[n] of cos_sin:
 *           (a, b) -> (a cos_i - b sin_i, b cos_i + a sin_i) over the pairs
 *           (2i, 2i+1) (rope_neox = 0, the DeepSeek layout) or (i, i+32)
 *           (rope_neox = 1)
 *     the 352-byte record of (bf16(y), bf16(k))
 * The arithmetic is binary32, each step rounded to nearest even with no fused
 * multiply-add, in a fixed order: squares; a sum of elements 8l..8l+7 in
 * element order for l = 0..63; those 64 sums added pairwise, neighbours
 * first; times 1/512; plus eps; sqrt; 1 / that; (x * r) * w; then products,
 * then the difference or sum for the turn; bf16 = round to nearest even.
 * The records are therefore exactly those nvfp4_mla_quantize_append writes
 * from the bf16 intermediate an unfused norm and rotary step would store.
 *
 *   latent_bf16, rope_bf16  un-normalised latent [num_tokens, >= 512] and
 *                    un-rotated RoPE [num_tokens, >= 64], bf16, with row
 *                    strides in elements as for nvfp4_mla_quantize_append
 *   norm_weight_bf16 [512] bf16 RMSNorm weight, 16-byte aligned
 *   eps              finite, >= 0 (a zero latent row needs eps > 0)
 *   cos_sin          [max_position, 64] float32 contiguous: cos of the 32
 *                    frequencies, then their sin, per position
 *   positions        [num_tokens] int64; a token whose position is outside
 *                    [0, max_position) is not written, like slot -1
 *   rope_neox        0 or 1 (pair layout above)
 * slot_mapping, kv_cache and the page geometry are as for
 * nvfp4_mla_quantize_append, whose skip rules and errors apply as well.
 */
int nvfp4_mla_norm_rope_quantize_append(const void* latent_bf16, int64_t latent_row_stride,
                                        const void* rope_bf16, int64_t rope_row_stride,
                                        const void* norm_weight_bf16, float eps,
                                        const float* cos_sin, int64_t max_position,
                                        const int64_t* positions, int32_t rope_neox,
                                        const int64_t* slot_mapping, int64_t num_tokens,
                                        uint8_t* kv_cache, int64_t num_blocks,
                                        int32_t block_size, int64_t block_stride_bytes,
                                        hipStream_t stream);

/* The fused write path into 432-byte "nvfp4_ds_mla" records: the arguments
 * and arithmetic of nvfp4_mla_norm_rope_quantize_append, the records those of
 * nvfp4_mla_quantize_append_ds_mla (the turned RoPE stored as its bf16
 * bits); block_stride_bytes >= block_size * 432. */
int nvfp4_mla_norm_rope_quantize_append_ds_mla(const void* latent_bf16, int64_t latent_row_stride,
                                               const void* rope_bf16, int64_t rope_row_stride,
                                               const void* norm_weight_bf16, float eps,
                                               const float* cos_sin, int64_t max_position,
                                               const int64_t* positions, int32_t rope_neox,
                                               const int64_t* slot_mapping, int64_t num_tokens,
                                               uint8_t* kv_cache, int64_t num_blocks,
                                               int32_t block_size, int64_t block_stride_bytes,
                                               hipStream_t stream);

/* Test export of the fused write path: out_f32 [num_tokens, 576] float32
 * contiguous (16-byte aligned) receives, for every token, the binary32 values
 * the fused path rounds to bf16: [normalised latent (512) | turned RoPE (64)],
 * computed by the same device code; a position outside [0, max_position)
 * gives NaN in that row's 64 RoPE values.  Arguments as for
 * nvfp4_mla_norm_rope_quantize_append. */
int nvfp4_mla_norm_rope_f32(const void* latent_bf16, int64_t latent_row_stride,
                            const void* rope_bf16, int64_t rope_row_stride,
                            const void* norm_weight_bf16, float eps, const float* cos_sin,
                            int64_t max_position, const int64_t* positions, int32_t rope_neox,
                            int64_t num_tokens, float* out_f32, hipStream_t stream);

/*
 * Quantize-append into 432-byte "nvfp4_ds_mla" records (layout above): the
 * NoPE codes and block scales of nvfp4_mla_quantize_append, the scales in
 * block order, the 16-byte pad zeroed and the bf16 RoPE bits copied verbatim
 * (vLLM PR #82, Fix and Tests).  Inputs are bf16 only: the record's RoPE lane
 * is bf16.  block_stride_bytes must be >= block_size * 432.  Every other
 * argument, layout, alignment rule, skip rule and error is that of
 * nvfp4_mla_quantize_append.
 */
int nvfp4_mla_quantize_append_ds_mla(const void* latent_bf16, int64_t latent_row_stride,
                                     const void* rope_bf16, int64_t rope_row_stride,
                                     const int64_t* slot_mapping, int64_t num_tokens,
                                     uint8_t* kv_cache, int64_t num_blocks,
                                     int32_t block_size, int64_t block_stride_bytes,
                                     hipStream_t stream);

/*
 * Dequantize-gather: out[i, :] = the 576 bf16 values of the record at
 * slots[i] ([512 NoPE = e2m1 * scale | 64 RoPE]): the values the decode
 * uses as its K and V operands, which are exact there (in fp16) and here (in
 * bf16), so both hold the same numbers.  slots[i] < 0 or beyond the cache
 * gives a row of zeros.
 *   slots   [n] int32;  out_bf16 [n, 576] bf16 contiguous.
 */
int nvfp4_mla_dequantize_gather(const uint8_t* kv_cache, int64_t num_blocks,
                                int32_t block_size, int64_t block_stride_bytes,
                                const int32_t* slots, int64_t n,
                                void* out_bf16, hipStream_t stream);

/* Dequantize-gather over a cache of 432-byte records: NoPE as above, RoPE
 * the stored bf16 bits.  Arguments and errors as nvfp4_mla_dequantize_gather
 * (block_stride_bytes >= block_size * 432). */
int nvfp4_mla_dequantize_gather_ds_mla(const uint8_t* kv_cache, int64_t num_blocks,
                                       int32_t block_size, int64_t block_stride_bytes,
                                       const int32_t* slots, int64_t n,
                                       void* out_bf16, hipStream_t stream);

/*
 * Split planner.  Chooses the number of split-KV partitions for a decode of
 * this shape on the current device (deterministic, no calibration; the same
 * inputs always give the same answer on the same device model).  The pages'
 * decode paths pick their launch shape per problem shape in the same way:
 * a planner memoised per shape that skips calibration while a stream is
 * capturing (sglang PR #38646, Modifications, the attention branch) and a
 * decode plan built ahead of the call (vLLM PR #82, Fix: the read path's
 * plan construction).
 * Writes 1 <= *num_splits_out <= NVFP4_MLA_MAX_SPLITS.
 */
int nvfp4_mla_sparse_decode_plan(int32_t batch, int32_t s_q, int32_t h_q,
                                 int32_t topk, int32_t* num_splits_out);

/*
 * Workspace bytes a decode with num_splits partitions needs (0 when
 * num_splits == 1).  num_splits == 0 means "what the planner picks".  The
 * caller allocates it once and keeps it for every later call, so that a
 * call never allocates and can be captured into a graph (sglang PR #38646,
 * Modifications: the graph-safe planner).
 * Returns 0 and sets the error on invalid arguments.
 *
 * The workspace holds the splits' partial O and LSE, which a combine kernel
 * launched right after the decode merges.  It needs no initialisation and
 * keeps nothing between calls, so one workspace serves every later decode
 * whose size it covers.  Decodes that may run concurrently need separate
 * workspaces.
 */
size_t nvfp4_mla_sparse_decode_workspace_size(int32_t batch, int32_t s_q,
                                              int32_t h_q, int32_t topk,
                                              int32_t num_splits);

/*
 * Sparse MLA decode.  For every query row (b, s) and head h, over the valid
 * indices t (0 <= indices[b,s,t] < num_blocks*block_size; duplicates count
 * each time they appear):
 *     z_t  = softmax_scale * <q[b,s,h,:], K_t>,     K_t = dequantized record
 *     LSE  = ln sum_t exp(z_t)
 *     O    = sum_t exp(z_t) V_t / (exp(LSE) + exp(attn_sink[h]))
 * with V_t the first 512 dims of K_t and the sink term present only when
 * attn_sink is non-NULL.  Rows with no valid index give O = 0, LSE = -inf.
 * LSE excludes the sink.
 *
 *   q_bf16     [batch, s_q, h_q, 576] bf16 contiguous; dims [0,512) pair with
 *              the NoPE part of the record, [512,576) with RoPE
 *   indices    [batch, s_q, topk] int32 contiguous slot ids, < 0 = invalid
 *   attn_sink  [h_q] float32 or NULL
 *   out_bf16   [batch, s_q, h_q, 512] bf16 contiguous
 *   lse        [batch, s_q, h_q] float32 (natural log)
 *   workspace  device scratch of nvfp4_mla_sparse_decode_workspace_size()
 *              bytes (may be NULL when that size is 0); 256-byte aligned
 *   num_splits 0 = planner's choice, else 1..NVFP4_MLA_MAX_SPLITS
 * h_q must be a multiple of 16 (1..16 * 16), topk in [1, 65536].
 * The decode is one kernel launch, plus one combine launch when more than
 * one split runs.  A call whose launches would exceed 2^32 - 1 work-items
 * (rows * h_q * splits * 16 for the decode, rows * h_q * 64 for the combine)
 * returns NVFP4_MLA_ERR_INVALID_ARGUMENT before any launch: split the batch.
 * Accuracy: K and V are exact; Q is exact for every element within 2^31 of
 * its head's largest magnitude; scores and sums are fp32; P enters PV as
 * fp16 hi + lo parts (about 2^-22 relative); O is rounded once to bf16 (with
 * splits, partial O is held in fp16 or fp32 first).  The results are the
 * same bits on every run and in graph replays.  The waves of a workgroup
 * wait for each other through bounded polls; a wait that ran out (correct
 * execution never comes near the bound) makes that workgroup's rows and
 * heads NaN in O and LSE rather than silently wrong.
 */
int nvfp4_mla_sparse_decode(const void* q_bf16, const uint8_t* kv_cache,
                            int64_t num_blocks, int32_t block_size,
                            int64_t block_stride_bytes, const int32_t* indices,
                            int32_t batch, int32_t s_q, int32_t h_q,
                            int32_t topk, const float* attn_sink,
                            float softmax_scale, void* out_bf16, float* lse,
                            void* workspace, size_t workspace_bytes,
                            int32_t num_splits, hipStream_t stream);

/*
 * Allocation-free sparse decode, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): nvfp4_mla_sparse_decode without the workspace
 * arguments.  Split partials go to a static device array of
 * NVFP4_MLA_NOALLOC_SCRATCH_BYTES held by the library, one per GPU, looked
 * up on the first call on each device and kept until the process ends; the
 * call allocates and frees nothing.  Arguments, results and errors are those
 * of nvfp4_mla_sparse_decode; a decode whose split partials
 * (nvfp4_mla_sparse_decode_workspace_size for the chosen split count) exceed
 * the array returns NVFP4_MLA_ERR_WORKSPACE_TOO_SMALL before any launch.
 * Every call on one GPU shares that GPU's array (it needs no clearing: each
 * call writes the partials it reads), so calls that may overlap on one GPU,
 * on different streams or threads, race and must be serialised by the
 * caller.
 */
#define NVFP4_MLA_NOALLOC_SCRATCH_BYTES (32u << 20)
int nvfp4_mla_sparse_decode_noalloc(const void* q_bf16, const uint8_t* kv_cache,
                                    int64_t num_blocks, int32_t block_size,
                                    int64_t block_stride_bytes, const int32_t* indices,
                                    int32_t batch, int32_t s_q, int32_t h_q, int32_t topk,
                                    const float* attn_sink, float softmax_scale,
                                    void* out_bf16, float* lse, int32_t num_splits,
                                    hipStream_t stream);

/*
 * Sparse decode over a cache of 432-byte records: the attention of
 * nvfp4_mla_sparse_decode, with K the record's dequantized NoPE followed by
 * its bf16 RoPE.  Arguments, workspace (nvfp4_mla_sparse_decode_plan and
 * _workspace_size apply unchanged) and errors as nvfp4_mla_sparse_decode;
 * block_stride_bytes >= block_size * 432.
 */
int nvfp4_mla_sparse_decode_ds_mla(const void* q_bf16, const uint8_t* kv_cache,
                                   int64_t num_blocks, int32_t block_size,
                                   int64_t block_stride_bytes, const int32_t* indices,
                                   int32_t batch, int32_t s_q, int32_t h_q,
                                   int32_t topk, const float* attn_sink,
                                   float softmax_scale, void* out_bf16, float* lse,
                                   void* workspace, size_t workspace_bytes,
                                   int32_t num_splits, hipStream_t stream);

/*
 * Dual-cache sparse decode: the same attention as nvfp4_mla_sparse_decode,
 * with one softmax (and the sink applied once) over the union of two top-k
 * lists that index two different paged caches: the primary cache (the
 * sliding window, 64-token pages in the pages' setup) and an extra cache (the
 * indexer's top-k, 2- or 64-token pages).  Each list holds slot ids of its
 * own cache; the caches may differ in block_size and block_stride_bytes
 * (sglang PR #38646 "[SM120] opt-in NVFP4 sparse-MLA KV cache format for
 * DeepSeek-V4": Modifications, the pool's page sizes; Performance, primary
 * top-k 128 plus extra top-k 512).  The result equals
 * nvfp4_mla_sparse_decode over one cache holding both pools' records, with
 * the two lists concatenated (primary first).
 *
 *   indices        [batch, s_q, topk] int32 slot ids of kv_cache, < 0 or
 *                  >= num_blocks*block_size = invalid
 *   extra_indices  [batch, s_q, extra_topk] int32 slot ids of extra_kv_cache,
 *                  the same invalid rule against its own slot count
 *   topk, extra_topk >= 0 with topk + extra_topk in [1, 65536]; a list whose
 *                  top-k is 0 may be NULL.  Both caches must be valid
 *                  (checked as for nvfp4_mla_sparse_decode) even when a list
 *                  is empty.
 * Every other argument is as for nvfp4_mla_sparse_decode.  The split planner
 * and the workspace size are those of a single-cache decode with
 * topk + extra_topk: call nvfp4_mla_sparse_decode_plan and
 * nvfp4_mla_sparse_decode_workspace_size with that sum.
 */
int nvfp4_mla_sparse_decode_dual(const void* q_bf16, const uint8_t* kv_cache,
                                 int64_t num_blocks, int32_t block_size,
                                 int64_t block_stride_bytes, const int32_t* indices,
                                 int32_t topk, const uint8_t* extra_kv_cache,
                                 int64_t extra_num_blocks, int32_t extra_block_size,
                                 int64_t extra_block_stride_bytes,
                                 const int32_t* extra_indices, int32_t extra_topk,
                                 int32_t batch, int32_t s_q, int32_t h_q,
                                 const float* attn_sink, float softmax_scale,
                                 void* out_bf16, float* lse, void* workspace,
                                 size_t workspace_bytes, int32_t num_splits,
                                 hipStream_t stream);

/* Dual-cache sparse decode over two caches of 432-byte records: arguments
 * and errors as nvfp4_mla_sparse_decode_dual, both caches holding 432-byte
 * records. */
int nvfp4_mla_sparse_decode_dual_ds_mla(const void* q_bf16, const uint8_t* kv_cache,
                                        int64_t num_blocks, int32_t block_size,
                                        int64_t block_stride_bytes, const int32_t* indices,
                                        int32_t topk, const uint8_t* extra_kv_cache,
                                        int64_t extra_num_blocks, int32_t extra_block_size,
                                        int64_t extra_block_stride_bytes,
                                        const int32_t* extra_indices, int32_t extra_topk,
                                        int32_t batch, int32_t s_q, int32_t h_q,
                                        const float* attn_sink, float softmax_scale,
                                        void* out_bf16, float* lse, void* workspace,
                                        size_t workspace_bytes, int32_t num_splits,
                                        hipStream_t stream);

/*
 * Split-KV combine.  Given num_splits sink-free partial results over
 * disjoint index subsets (O_i normalised within its subset, LSE_i natural
 * log; an empty subset has LSE_i = -inf) -- the merge a decode split over
 * its top-k list, or over context-parallel ranks each holding part of the
 * cache (vLLM PR #82 validates at TP4/DCP4, summary), needs to give the
 * softmax of the whole list; the sink belongs to that whole softmax, so it is
 * applied once here (FlashMLA PR #18, PR description: the attention sink):
 *     LSE = ln sum_i exp(LSE_i)
 *     O   = sum_i exp(LSE_i - LSE) O_i / (1 + exp(attn_sink[h] - LSE))
 * (sink factor only when attn_sink is non-NULL); all LSE_i = -inf gives
 * O = 0, LSE = -inf, and a NaN LSE_i gives a NaN row.
 *   o_partial   [num_splits, rows, h_q, 512] float32 contiguous
 *   lse_partial [num_splits, rows, h_q] float32 contiguous
 *   out_bf16    [rows, h_q, 512] bf16;  lse [rows, h_q] float32
 * num_splits in [1, 4096]; rows * h_q below 2^26 (one launch of 64
 * work-items per row and head), else NVFP4_MLA_ERR_INVALID_ARGUMENT.
 */
int nvfp4_mla_combine(const float* o_partial, const float* lse_partial,
                      int32_t num_splits, int64_t rows, int32_t h_q,
                      const float* attn_sink, void* out_bf16, float* lse,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MLA_H */
