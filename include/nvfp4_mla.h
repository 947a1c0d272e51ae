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
                              void* stream);

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
                                   void* stream);

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
                                     void* stream);

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
                                void* out_bf16, void* stream);

/* Dequantize-gather over a cache of 432-byte records: NoPE as above, RoPE
 * the stored bf16 bits.  Arguments and errors as nvfp4_mla_dequantize_gather
 * (block_stride_bytes >= block_size * 432). */
int nvfp4_mla_dequantize_gather_ds_mla(const uint8_t* kv_cache, int64_t num_blocks,
                                       int32_t block_size, int64_t block_stride_bytes,
                                       const int32_t* slots, int64_t n,
                                       void* out_bf16, void* stream);

/*
 * Split planner.  Chooses the number of split-KV partitions for a decode of
 * this shape on the current device (deterministic, no calibration; the same
 * inputs always give the same answer on the same device model).
 * Writes 1 <= *num_splits_out <= NVFP4_MLA_MAX_SPLITS.
 */
int nvfp4_mla_sparse_decode_plan(int32_t batch, int32_t s_q, int32_t h_q,
                                 int32_t topk, int32_t* num_splits_out);

/*
 * Workspace bytes a decode with num_splits partitions needs (0 when
 * num_splits == 1).  num_splits == 0 means "what the planner picks".
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
 * one split runs.
 * Accuracy: K and V are exact; Q is exact for every element within 2^31 of
 * its head's largest magnitude; scores and sums are fp32; P enters PV as
 * fp16 hi + lo parts (about 2^-22 relative); O is rounded once to bf16 (with
 * splits, partial O is held in fp16 or fp32 first).  The results are the
 * same bits on every run and in graph replays.
 */
int nvfp4_mla_sparse_decode(const void* q_bf16, const uint8_t* kv_cache,
                            int64_t num_blocks, int32_t block_size,
                            int64_t block_stride_bytes, const int32_t* indices,
                            int32_t batch, int32_t s_q, int32_t h_q,
                            int32_t topk, const float* attn_sink,
                            float softmax_scale, void* out_bf16, float* lse,
                            void* workspace, size_t workspace_bytes,
                            int32_t num_splits, void* stream);

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
                                    void* stream);

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
                                   int32_t num_splits, void* stream);

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
                                 void* stream);

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
                                        void* stream);

/*
 * Split-KV combine.  Given num_splits sink-free partial results over
 * disjoint index subsets (O_i normalised within its subset, LSE_i natural
 * log; an empty subset has LSE_i = -inf):
 *     LSE = ln sum_i exp(LSE_i)
 *     O   = sum_i exp(LSE_i - LSE) O_i / (1 + exp(attn_sink[h] - LSE))
 * (sink factor only when attn_sink is non-NULL); all LSE_i = -inf gives
 * O = 0, LSE = -inf.
 *   o_partial   [num_splits, rows, h_q, 512] float32 contiguous
 *   lse_partial [num_splits, rows, h_q] float32 contiguous
 *   out_bf16    [rows, h_q, 512] bf16;  lse [rows, h_q] float32
 */
int nvfp4_mla_combine(const float* o_partial, const float* lse_partial,
                      int32_t num_splits, int64_t rows, int32_t h_q,
                      const float* attn_sink, void* out_bf16, float* lse,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MLA_H */
