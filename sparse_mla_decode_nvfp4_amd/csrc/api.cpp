// C ABI of the NVFP4 sparse-MLA library (declared in include/nvfp4_mla.h):
// argument validation, the gfx950 device gate, the split planner, workspace
// sizing, the thread-local error message, and the kernel launches.
//
// Every argument is validated before the first HIP call, so argument errors
// are reported identically with or without a GPU.  Failures are loud: each has
// its own status code and message (the convention of the pages' write path,
// which rejects unsupported dims and devices with explicit errors).
#include "../../include/nvfp4_mla.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <algorithm>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return NVFP4_MLA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-device cache: 0 = not yet checked, 1 = gfx950, 2 = other.  Zero-
// initialised statics; racing first calls both store the same values.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

// Returns OK when the current device is gfx950; fills cus when non-null.
int check_device(int* cus) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(NVFP4_MLA_ERR_UNSUPPORTED_DEVICE, "no HIP device available (%s)",
                hipGetErrorString(e));
  if (dev >= kMaxDevices)
    return fail(NVFP4_MLA_ERR_UNSUPPORTED_DEVICE, "device index %d out of range", dev);
  int known = g_dev_state[dev].load(std::memory_order_acquire);
  if (known == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(NVFP4_MLA_ERR_UNSUPPORTED_DEVICE, "hipGetDeviceProperties failed: %s",
                  hipGetErrorString(e));
    const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    known = is950 ? 1 : 2;
    g_dev_state[dev].store(known, std::memory_order_release);
    if (!is950)
      return fail(NVFP4_MLA_ERR_UNSUPPORTED_DEVICE,
                  "device %d is %s; this library is built for gfx950 (MI355X) only", dev,
                  prop.gcnArchName);
  }
  if (known != 1)
    return fail(NVFP4_MLA_ERR_UNSUPPORTED_DEVICE,
                "device %d is not gfx950; this library is built for gfx950 (MI355X) only", dev);
  if (cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return NVFP4_MLA_OK;
}

int check_cache(const void* kv_cache, int64_t num_blocks, int32_t block_size,
                int64_t block_stride_bytes, int64_t* num_slots,
                int32_t record_bytes = NVFP4_MLA_RECORD_BYTES) {
  if (kv_cache == nullptr) return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "kv_cache is NULL");
  if (!aligned(kv_cache, 16))
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "kv_cache must be 16-byte aligned");
  if (num_blocks < 1) return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "num_blocks must be >= 1");
  if (block_size < 1) return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "block_size must be >= 1");
  if (block_stride_bytes % 16 != 0)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "block_stride_bytes must be a multiple of 16");
  if (block_stride_bytes < (int64_t)block_size * record_bytes)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                "block_stride_bytes %lld < block_size * %d = %lld",
                (long long)block_stride_bytes, record_bytes,
                (long long)block_size * record_bytes);
  const int64_t slots = num_blocks * (int64_t)block_size;
  if (num_blocks > INT64_C(0x7FFFFFFF) || slots > INT64_C(0x7FFFFFFF))
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                "num_blocks * block_size = %lld exceeds the 2^31-1 slot ids int32 indices address",
                (long long)slots);
  *num_slots = slots;
  return NVFP4_MLA_OK;
}

nvfp4::PageAddr make_page_addr(int32_t block_size, int64_t block_stride_bytes,
                               int32_t record_bytes = NVFP4_MLA_RECORD_BYTES) {
  nvfp4::PageAddr pa{};
  pa.record_bytes = (uint32_t)record_bytes;
  pa.block_stride = (uint64_t)block_stride_bytes;
  pa.block_size = (uint32_t)block_size;
  pa.pow2 = (block_size & (block_size - 1)) == 0;
  pa.contig = (uint64_t)block_stride_bytes == (uint64_t)block_size * (uint64_t)record_bytes;
  pa.shift = 0;
  while ((1u << pa.shift) < (uint32_t)block_size) pa.shift++;
  // ceil(2^64 / d) for d >= 2 that is not a power of two
  if (!pa.pow2) {
    const unsigned __int128 one = (unsigned __int128)1 << 64;
    pa.recip = (uint64_t)((one + block_size - 1) / (unsigned __int128)block_size);
  }
  return pa;
}

int check_decode_shape(int32_t batch, int32_t s_q, int32_t h_q, int32_t topk) {
  if (batch < 0 || s_q < 0)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "batch and s_q must be >= 0");
  if ((int64_t)batch * s_q > INT64_C(0x7FFFFFFF))
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "batch * s_q too large");
  if (h_q < 16 || h_q > 256 || h_q % 16 != 0)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "h_q = %d must be a multiple of 16 in [16, 256]",
                h_q);
  if (topk < 1 || topk > 65536)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "topk = %d must be in [1, 65536]", topk);
  return NVFP4_MLA_OK;
}

// Deterministic split choice: enough splits to give every CU work, no more
// than the top-k list can feed.  The 32-head-group kernel runs one workgroup
// per (row, 32 heads, split), aiming at one per CU; its wave pairs each take a
// token stream of 16-token chunks (four pairs, or two pairs at two
// workgroups per CU once the grid is that large).  The 16-head tile kernel runs
// one workgroup per (row, 16 heads, split), two per CU, at least one 64-token
// tile each.
int plan_splits(int32_t rows, int32_t h_q, int32_t topk, int cus) {
  const bool w32 = nvfp4::decode_uses_w32(h_q);
  const int64_t wgs = (int64_t)rows * (w32 ? h_q / 32 : h_q / 16);
  if (wgs == 0) return 1;
  const int64_t per_cu = w32 ? 1 : 2;
  int64_t want = (per_cu * (int64_t)cus + wgs - 1) / wgs;
  // w32: 16-token chunks over four token streams; keep at least two steps per split
  const int64_t max_by_work = w32 ? std::max<int64_t>(1, ((topk + 15) / 16) / 8) : (topk + 63) / 64;
  if (want > max_by_work) want = max_by_work;
  if (want > NVFP4_MLA_MAX_SPLITS) want = NVFP4_MLA_MAX_SPLITS;
  if (want < 1) want = 1;
  return (int)want;
}

// A decode launch's work-items must fit HIP's 32-bit grid size: the decode
// kernel runs rows * (h_q / 32 or / 16) * splits workgroups of at most 512
// work-items (256 for the 16-head kernel), and with splits the combine runs
// 64 work-items per (row, head).  Larger calls are rejected, never truncated.
int check_launch_size(int64_t rows, int32_t h_q, int32_t splits) {
  const bool w32 = nvfp4::decode_uses_w32(h_q);
  const int64_t wgs = rows * (w32 ? h_q / 32 : h_q / 16) * (int64_t)splits;
  const int64_t items = wgs * (w32 ? 512 : 256);
  const int64_t combine_items = splits > 1 ? rows * h_q * 64 : 0;
  if (items > INT64_C(0xFFFFFFFF) || combine_items > INT64_C(0xFFFFFFFF))
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                "a decode of %lld rows x %d heads with %d splits needs %lld decode work-items "
                "(and %lld for the combine); one launch holds at most 2^32 - 1: split the batch",
                (long long)rows, h_q, splits, (long long)items, (long long)combine_items);
  return NVFP4_MLA_OK;
}

// Workspace layout for splits > 1 (each region 256-byte aligned):
//   o_part   [splits, rows, h_q, 512] fp32 (the 32-head kernel fills the first half
//            of it with fp16 partials)
//   lse_part [splits, rows, h_q] fp32
struct WsLayout {
  size_t o_off, lse_off, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(int64_t rows, int32_t h_q, int32_t splits) {
  WsLayout w{0, 0, 0};
  if (splits <= 1) return w;
  const size_t o = (size_t)splits * rows * h_q * NVFP4_MLA_V_DIM * sizeof(float);
  const size_t l = (size_t)splits * rows * h_q * sizeof(float);
  w.o_off = 0;
  w.lse_off = align256(o);
  w.total = w.lse_off + align256(l);
  return w;
}

size_t workspace_bytes(int64_t rows, int32_t h_q, int32_t splits) {
  return ws_layout(rows, h_q, splits).total;
}

}  // namespace

// Split-partial scratch of nvfp4_mla_sparse_decode_noalloc: one array per GPU
// the library runs on, held until the process ends.  Its name is a host-side
// stand-in in host code; only the address hipGetSymbolAddress returns for the
// current device is ever passed to a kernel.
namespace {
constexpr size_t kScratchBytes = NVFP4_MLA_NOALLOC_SCRATCH_BYTES;
}
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];     // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device (with
// that device current) on its first use.
int device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(NVFP4_MLA_ERR_UNSUPPORTED_DEVICE, "no usable HIP device (%s)", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(NVFP4_MLA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_MLA_OK;
}

}  // namespace

namespace {

// Shared by the bf16 and fp16 exports: the same checks, one kernel template.
int quantize_append_impl(const char* fn, const void* latent_bf16, int64_t latent_row_stride,
                         const void* rope_bf16, int64_t rope_row_stride,
                         const int64_t* slot_mapping, int64_t num_tokens, uint8_t* kv_cache,
                         int64_t num_blocks, int32_t block_size, int64_t block_stride_bytes,
                         bool f16_input, int32_t record_bytes, hipStream_t stream,
                         const nvfp4::NormRope* fused = nullptr) {
  if (num_tokens < 0) return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0");
  int64_t num_slots = 0;
  int rc = check_cache(kv_cache, num_blocks, block_size, block_stride_bytes, &num_slots,
                       record_bytes);
  if (rc) return rc;
  if (num_tokens > 0) {
    if (!latent_bf16 || !rope_bf16 || !slot_mapping)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "latent, rope and slot_mapping must be non-NULL");
    if (latent_row_stride < NVFP4_MLA_NOPE_DIM || rope_row_stride < NVFP4_MLA_ROPE_DIM)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                  "row strides (%lld, %lld) must be >= (512, 64) elements",
                  (long long)latent_row_stride, (long long)rope_row_stride);
    if (!aligned(latent_bf16, 16) || latent_row_stride % 8 != 0)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                  "latent rows must be 16-byte aligned (aligned base, stride multiple of 8)");
    if (!aligned(rope_bf16, 2) || !aligned(slot_mapping, 8))
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "rope / slot_mapping misaligned");
    if (num_tokens > (int64_t)0x7FFFFFFF * 4)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "num_tokens too large");
  }
  rc = check_device(nullptr);
  if (rc) return rc;
  const nvfp4::PageAddr pa = make_page_addr(block_size, block_stride_bytes, record_bytes);
  hipError_t e =
      fused ? nvfp4::launch_norm_rope_quantize_append(
                  static_cast<const uint16_t*>(latent_bf16), latent_row_stride,
                  static_cast<const uint16_t*>(rope_bf16), rope_row_stride, *fused, slot_mapping,
                  num_tokens, kv_cache, num_slots, pa, stream)
            : nvfp4::launch_quantize_append(
                  static_cast<const uint16_t*>(latent_bf16), latent_row_stride,
                  static_cast<const uint16_t*>(rope_bf16), rope_row_stride, slot_mapping,
                  num_tokens, kv_cache, num_slots, pa, f16_input, stream);
  if (e != hipSuccess)
    return fail(NVFP4_MLA_ERR_HIP, "%s launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

// Checks the fused prologue's arguments (needed only when tokens are
// written) and fills `nr`.
int check_norm_rope(const void* norm_weight_bf16, float eps, const float* cos_sin,
                    int64_t max_position, const int64_t* positions, int32_t rope_neox,
                    int64_t num_tokens, nvfp4::NormRope* nr) {
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (rope_neox != 0 && rope_neox != 1)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "rope_neox must be 0 (pairs 2i, 2i+1) or 1 "
                "(pairs i, i+32)");
  if (max_position < 1)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "max_position must be >= 1");
  if (max_position > (INT64_MAX / 256))
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "max_position too large");
  if (num_tokens > 0) {
    if (!norm_weight_bf16 || !cos_sin || !positions)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                  "norm_weight, cos_sin and positions must be non-NULL");
    if (!aligned(norm_weight_bf16, 16) || !aligned(cos_sin, 4) || !aligned(positions, 8))
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                  "norm_weight must be 16-byte aligned, cos_sin 4-byte and positions 8-byte");
  }
  nr->weight = static_cast<const uint16_t*>(norm_weight_bf16);
  nr->eps = eps;
  nr->cos_sin = cos_sin;
  nr->max_position = max_position;
  nr->positions = positions;
  nr->neox = rope_neox;
  return NVFP4_MLA_OK;
}

// Shared by the single- and dual-cache exports.  `extra` is null for the
// single-cache decode; topk0 is the primary list's length, topk the joined
// list's.
struct ExtraCache {
  const uint8_t* kv_cache;
  int64_t num_blocks;
  int32_t block_size;
  int64_t block_stride_bytes;
  const int32_t* indices;
  int32_t topk;
};

int sparse_decode_impl(const char* fn, const void* q_bf16, const uint8_t* kv_cache,
                       int64_t num_blocks, int32_t block_size, int64_t block_stride_bytes,
                       const int32_t* indices, int32_t topk0, const ExtraCache* extra,
                       int32_t batch, int32_t s_q, int32_t h_q, const float* attn_sink,
                       float softmax_scale, void* out_bf16, float* lse, void* workspace,
                       size_t workspace_bytes_in, int32_t num_splits, int32_t record_bytes,
                       hipStream_t stream, bool static_scratch = false) {
  if (extra && (topk0 < 0 || extra->topk < 0 || topk0 > 65536 || extra->topk > 65536))
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "topk = %d and extra_topk = %d must be in [0, 65536]",
                topk0, extra ? extra->topk : 0);
  const int32_t topk = topk0 + (extra ? extra->topk : 0);
  int rc = check_decode_shape(batch, s_q, h_q, topk);
  if (rc) return rc;
  int64_t num_slots = 0, num_slots1 = 0;
  rc = check_cache(kv_cache, num_blocks, block_size, block_stride_bytes, &num_slots, record_bytes);
  if (rc) return rc;
  if (extra) {
    rc = check_cache(extra->kv_cache, extra->num_blocks, extra->block_size,
                     extra->block_stride_bytes, &num_slots1, record_bytes);
    if (rc) return fail(rc, "extra cache: %s", g_last_error.c_str());
  }
  if (num_splits < 0 || num_splits > NVFP4_MLA_MAX_SPLITS)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "num_splits = %d out of [0, %d]", num_splits,
                NVFP4_MLA_MAX_SPLITS);
  if (!std::isfinite(softmax_scale))
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  const int64_t rows = (int64_t)batch * s_q;
  // the planner never picks fewer than one split
  rc = check_launch_size(rows, h_q, num_splits > 0 ? num_splits : 1);
  if (rc) return rc;
  if (rows > 0) {
    if (!q_bf16 || !out_bf16 || !lse)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "q, indices, out and lse must be non-NULL");
    if ((topk0 > 0 && !indices) || (extra && extra->topk > 0 && !extra->indices))
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                  "q, indices, out and lse must be non-NULL (an index list may be NULL only "
                  "when its top-k is 0)");
    if (!aligned(q_bf16, 16) || !aligned(out_bf16, 16) || !aligned(lse, 4) ||
        !aligned(indices, 4) || (extra && !aligned(extra->indices, 4)) ||
        (attn_sink && !aligned(attn_sink, 4)))
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                  "q and out must be 16-byte aligned; indices, lse, sink 4-byte aligned");
  }
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;
  int splits = num_splits == 0 ? plan_splits((int32_t)rows, h_q, topk, cus) : num_splits;
  rc = check_launch_size(rows, h_q, splits);
  if (rc) return rc;
  const size_t need = workspace_bytes(rows, h_q, splits);
  if (static_scratch && need > 0) {
    if (need > kScratchBytes)
      return fail(NVFP4_MLA_ERR_WORKSPACE_TOO_SMALL,
                  "%s: a decode of %lld rows x %d heads with %d splits needs %zu bytes of split "
                  "partials; the allocation-free entry point holds at most %zu (use fewer splits "
                  "or nvfp4_mla_sparse_decode with a workspace)",
                  fn, (long long)rows, h_q, splits, need, kScratchBytes);
    rc = device_scratch(&workspace);
    if (rc) return rc;
    workspace_bytes_in = kScratchBytes;
  }
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes_in < need)
      return fail(NVFP4_MLA_ERR_WORKSPACE_TOO_SMALL,
                  "decode with %d splits needs %zu workspace bytes, got %zu", splits, need,
                  workspace == nullptr ? (size_t)0 : workspace_bytes_in);
    if (!aligned(workspace, 256))
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  }
  if (rows == 0) return ok();
  nvfp4::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.cache = kv_cache;
  a.pa = make_page_addr(block_size, block_stride_bytes, record_bytes);
  a.num_slots = num_slots;
  a.indices = indices;
  a.topk0 = topk0;
  if (extra) {
    a.cache1 = extra->kv_cache;
    a.pa1 = make_page_addr(extra->block_size, extra->block_stride_bytes, record_bytes);
    a.num_slots1 = num_slots1;
    a.indices1 = extra->indices;
  }
  a.rows = (int32_t)rows;
  a.s_q = s_q;
  a.h_q = h_q;
  a.topk = topk;
  a.sink = attn_sink;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  a.out = static_cast<uint16_t*>(out_bf16);
  a.lse = lse;
  a.splits = splits;
  a.num_cus = cus;
  if (splits > 1) {
    const WsLayout w = ws_layout(rows, h_q, splits);
    char* base = static_cast<char*>(workspace);
    a.o_part = reinterpret_cast<float*>(base + w.o_off);
    a.lse_part = reinterpret_cast<float*>(base + w.lse_off);
  }
  hipError_t e = nvfp4::launch_decode(a, stream);
  if (e != hipSuccess)
    return fail(NVFP4_MLA_ERR_HIP, "%s launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int dequantize_gather_impl(const char* fn, const uint8_t* kv_cache, int64_t num_blocks,
                           int32_t block_size, int64_t block_stride_bytes, const int32_t* slots,
                           int64_t n, void* out_bf16, int32_t record_bytes, hipStream_t stream) {
  if (n < 0) return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "n must be >= 0");
  int64_t num_slots = 0;
  int rc = check_cache(kv_cache, num_blocks, block_size, block_stride_bytes, &num_slots,
                       record_bytes);
  if (rc) return rc;
  if (n > 0) {
    if (!slots || !out_bf16)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "slots and out must be non-NULL");
    if (!aligned(out_bf16, 16) || !aligned(slots, 4))
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                  "out must be 16-byte aligned and slots 4-byte aligned");
    if (n > (int64_t)0x7FFFFFFF * 4)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "n too large");
  }
  rc = check_device(nullptr);
  if (rc) return rc;
  hipError_t e = nvfp4::launch_dequantize_gather(kv_cache, num_slots,
                                                 make_page_addr(block_size, block_stride_bytes,
                                                                record_bytes),
                                                 slots, n, static_cast<uint16_t*>(out_bf16),
                                                 stream);
  if (e != hipSuccess)
    return fail(NVFP4_MLA_ERR_HIP, "%s launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int nvfp4_mla_abi_version(void) { return NVFP4_MLA_ABI_VERSION; }

const char* nvfp4_mla_last_error(void) { return g_last_error.c_str(); }

int nvfp4_mla_check_format(int32_t record_bytes, int32_t nope_dim, int32_t rope_dim,
                           int32_t v_dim) {
  if ((record_bytes != NVFP4_MLA_RECORD_BYTES && record_bytes != NVFP4_MLA_DS_MLA_RECORD_BYTES) ||
      nope_dim != NVFP4_MLA_NOPE_DIM || rope_dim != NVFP4_MLA_ROPE_DIM || v_dim != NVFP4_MLA_V_DIM)
    return fail(NVFP4_MLA_ERR_UNSUPPORTED_FORMAT,
                "unsupported format: record %d B, NoPE %d, RoPE %d, d_v %d (this library "
                "implements the 352 B and 432 B NVFP4 records with 512/64/512)",
                record_bytes, nope_dim, rope_dim, v_dim);
  return ok();
}


int nvfp4_mla_quantize_append(const void* latent_bf16, int64_t latent_row_stride,
                              const void* rope_bf16, int64_t rope_row_stride,
                              const int64_t* slot_mapping, int64_t num_tokens,
                              uint8_t* kv_cache, int64_t num_blocks, int32_t block_size,
                              int64_t block_stride_bytes, hipStream_t stream) {
  return quantize_append_impl("quantize_append", latent_bf16, latent_row_stride, rope_bf16,
                              rope_row_stride, slot_mapping, num_tokens, kv_cache, num_blocks,
                              block_size, block_stride_bytes, false, NVFP4_MLA_RECORD_BYTES,
                              stream);
}

int nvfp4_mla_quantize_append_ds_mla(const void* latent_bf16, int64_t latent_row_stride,
                                     const void* rope_bf16, int64_t rope_row_stride,
                                     const int64_t* slot_mapping, int64_t num_tokens,
                                     uint8_t* kv_cache, int64_t num_blocks, int32_t block_size,
                                     int64_t block_stride_bytes, hipStream_t stream) {
  return quantize_append_impl("quantize_append_ds_mla", latent_bf16, latent_row_stride,
                              rope_bf16, rope_row_stride, slot_mapping, num_tokens, kv_cache,
                              num_blocks, block_size, block_stride_bytes, false,
                              NVFP4_MLA_DS_MLA_RECORD_BYTES, stream);
}

int nvfp4_mla_quantize_append_fp16(const void* latent_fp16, int64_t latent_row_stride,
                                   const void* rope_fp16, int64_t rope_row_stride,
                                   const int64_t* slot_mapping, int64_t num_tokens,
                                   uint8_t* kv_cache, int64_t num_blocks, int32_t block_size,
                                   int64_t block_stride_bytes, hipStream_t stream) {
  return quantize_append_impl("quantize_append_fp16", latent_fp16, latent_row_stride, rope_fp16,
                              rope_row_stride, slot_mapping, num_tokens, kv_cache, num_blocks,
                              block_size, block_stride_bytes, true, NVFP4_MLA_RECORD_BYTES,
                              stream);
}

int nvfp4_mla_norm_rope_quantize_append(
    const void* latent_bf16, int64_t latent_row_stride, const void* rope_bf16,
    int64_t rope_row_stride, const void* norm_weight_bf16, float eps, const float* cos_sin,
    int64_t max_position, const int64_t* positions, int32_t rope_neox,
    const int64_t* slot_mapping, int64_t num_tokens, uint8_t* kv_cache, int64_t num_blocks,
    int32_t block_size, int64_t block_stride_bytes, hipStream_t stream) {
  nvfp4::NormRope nr{};
  int rc = check_norm_rope(norm_weight_bf16, eps, cos_sin, max_position, positions, rope_neox,
                           num_tokens, &nr);
  if (rc) return rc;
  return quantize_append_impl("norm_rope_quantize_append", latent_bf16, latent_row_stride,
                              rope_bf16, rope_row_stride, slot_mapping, num_tokens, kv_cache,
                              num_blocks, block_size, block_stride_bytes, false,
                              NVFP4_MLA_RECORD_BYTES, stream, &nr);
}

int nvfp4_mla_norm_rope_quantize_append_ds_mla(
    const void* latent_bf16, int64_t latent_row_stride, const void* rope_bf16,
    int64_t rope_row_stride, const void* norm_weight_bf16, float eps, const float* cos_sin,
    int64_t max_position, const int64_t* positions, int32_t rope_neox,
    const int64_t* slot_mapping, int64_t num_tokens, uint8_t* kv_cache, int64_t num_blocks,
    int32_t block_size, int64_t block_stride_bytes, hipStream_t stream) {
  nvfp4::NormRope nr{};
  int rc = check_norm_rope(norm_weight_bf16, eps, cos_sin, max_position, positions, rope_neox,
                           num_tokens, &nr);
  if (rc) return rc;
  return quantize_append_impl("norm_rope_quantize_append_ds_mla", latent_bf16, latent_row_stride,
                              rope_bf16, rope_row_stride, slot_mapping, num_tokens, kv_cache,
                              num_blocks, block_size, block_stride_bytes, false,
                              NVFP4_MLA_DS_MLA_RECORD_BYTES, stream, &nr);
}

int nvfp4_mla_norm_rope_f32(const void* latent_bf16, int64_t latent_row_stride,
                            const void* rope_bf16, int64_t rope_row_stride,
                            const void* norm_weight_bf16, float eps, const float* cos_sin,
                            int64_t max_position, const int64_t* positions, int32_t rope_neox,
                            int64_t num_tokens, float* out_f32, hipStream_t stream) {
  if (num_tokens < 0) return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0");
  nvfp4::NormRope nr{};
  int rc = check_norm_rope(norm_weight_bf16, eps, cos_sin, max_position, positions, rope_neox,
                           num_tokens, &nr);
  if (rc) return rc;
  if (num_tokens > 0) {
    if (!latent_bf16 || !rope_bf16 || !out_f32)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "latent, rope and out must be non-NULL");
    if (latent_row_stride < NVFP4_MLA_NOPE_DIM || rope_row_stride < NVFP4_MLA_ROPE_DIM)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                  "row strides (%lld, %lld) must be >= (512, 64) elements",
                  (long long)latent_row_stride, (long long)rope_row_stride);
    if (!aligned(latent_bf16, 16) || latent_row_stride % 8 != 0 || !aligned(rope_bf16, 2) ||
        !aligned(out_f32, 16))
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                  "latent rows and out must be 16-byte aligned, rope 2-byte aligned");
    if (num_tokens > (int64_t)0x7FFFFFFF * 4)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "num_tokens too large");
  }
  rc = check_device(nullptr);
  if (rc) return rc;
  hipError_t e = nvfp4::launch_norm_rope_f32(static_cast<const uint16_t*>(latent_bf16),
                                             latent_row_stride,
                                             static_cast<const uint16_t*>(rope_bf16),
                                             rope_row_stride, nr, num_tokens, out_f32, stream);
  if (e != hipSuccess)
    return fail(NVFP4_MLA_ERR_HIP, "norm_rope_f32 launch failed: %s", hipGetErrorString(e));
  return ok();
}

int nvfp4_mla_dequantize_gather(const uint8_t* kv_cache, int64_t num_blocks, int32_t block_size,
                                int64_t block_stride_bytes, const int32_t* slots, int64_t n,
                                void* out_bf16, hipStream_t stream) {
  return dequantize_gather_impl("dequantize_gather", kv_cache, num_blocks, block_size,
                                block_stride_bytes, slots, n, out_bf16, NVFP4_MLA_RECORD_BYTES,
                                stream);
}

int nvfp4_mla_dequantize_gather_ds_mla(const uint8_t* kv_cache, int64_t num_blocks,
                                       int32_t block_size, int64_t block_stride_bytes,
                                       const int32_t* slots, int64_t n, void* out_bf16,
                                       hipStream_t stream) {
  return dequantize_gather_impl("dequantize_gather_ds_mla", kv_cache, num_blocks, block_size,
                                block_stride_bytes, slots, n, out_bf16,
                                NVFP4_MLA_DS_MLA_RECORD_BYTES, stream);
}

int nvfp4_mla_sparse_decode_plan(int32_t batch, int32_t s_q, int32_t h_q, int32_t topk,
                                 int32_t* num_splits_out) {
  if (!num_splits_out) return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "num_splits_out is NULL");
  int rc = check_decode_shape(batch, s_q, h_q, topk);
  if (rc) return rc;
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;
  *num_splits_out = plan_splits(batch * s_q, h_q, topk, cus);
  return ok();
}

size_t nvfp4_mla_sparse_decode_workspace_size(int32_t batch, int32_t s_q, int32_t h_q,
                                              int32_t topk, int32_t num_splits) {
  if (check_decode_shape(batch, s_q, h_q, topk)) return 0;
  if (num_splits < 0 || num_splits > NVFP4_MLA_MAX_SPLITS) {
    fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "num_splits = %d out of [0, %d]", num_splits,
         NVFP4_MLA_MAX_SPLITS);
    return 0;
  }
  int splits = num_splits;
  if (splits == 0) {
    int cus = 0;
    if (check_device(&cus)) return 0;
    splits = plan_splits(batch * s_q, h_q, topk, cus);
  }
  ok();
  return workspace_bytes((int64_t)batch * s_q, h_q, splits);
}

int nvfp4_mla_sparse_decode(const void* q_bf16, const uint8_t* kv_cache, int64_t num_blocks,
                            int32_t block_size, int64_t block_stride_bytes,
                            const int32_t* indices, int32_t batch, int32_t s_q, int32_t h_q,
                            int32_t topk, const float* attn_sink, float softmax_scale,
                            void* out_bf16, float* lse, void* workspace, size_t workspace_bytes_in,
                            int32_t num_splits, hipStream_t stream) {
  return sparse_decode_impl("sparse_decode", q_bf16, kv_cache, num_blocks, block_size,
                            block_stride_bytes, indices, topk, nullptr, batch, s_q, h_q,
                            attn_sink, softmax_scale, out_bf16, lse, workspace,
                            workspace_bytes_in, num_splits, NVFP4_MLA_RECORD_BYTES, stream);
}

int nvfp4_mla_sparse_decode_noalloc(const void* q_bf16, const uint8_t* kv_cache,
                                    int64_t num_blocks, int32_t block_size,
                                    int64_t block_stride_bytes, const int32_t* indices,
                                    int32_t batch, int32_t s_q, int32_t h_q, int32_t topk,
                                    const float* attn_sink, float softmax_scale, void* out_bf16,
                                    float* lse, int32_t num_splits, hipStream_t stream) {
  return sparse_decode_impl("sparse_decode_noalloc", q_bf16, kv_cache, num_blocks, block_size,
                            block_stride_bytes, indices, topk, nullptr, batch, s_q, h_q,
                            attn_sink, softmax_scale, out_bf16, lse, nullptr, 0, num_splits,
                            NVFP4_MLA_RECORD_BYTES, stream, /*static_scratch=*/true);
}

int nvfp4_mla_sparse_decode_ds_mla(const void* q_bf16, const uint8_t* kv_cache,
                                   int64_t num_blocks, int32_t block_size,
                                   int64_t block_stride_bytes, const int32_t* indices,
                                   int32_t batch, int32_t s_q, int32_t h_q, int32_t topk,
                                   const float* attn_sink, float softmax_scale, void* out_bf16,
                                   float* lse, void* workspace, size_t workspace_bytes_in,
                                   int32_t num_splits, hipStream_t stream) {
  return sparse_decode_impl("sparse_decode_ds_mla", q_bf16, kv_cache, num_blocks, block_size,
                            block_stride_bytes, indices, topk, nullptr, batch, s_q, h_q,
                            attn_sink, softmax_scale, out_bf16, lse, workspace,
                            workspace_bytes_in, num_splits, NVFP4_MLA_DS_MLA_RECORD_BYTES,
                            stream);
}

int nvfp4_mla_sparse_decode_dual(const void* q_bf16, const uint8_t* kv_cache, int64_t num_blocks,
                                 int32_t block_size, int64_t block_stride_bytes,
                                 const int32_t* indices, int32_t topk,
                                 const uint8_t* extra_kv_cache, int64_t extra_num_blocks,
                                 int32_t extra_block_size, int64_t extra_block_stride_bytes,
                                 const int32_t* extra_indices, int32_t extra_topk, int32_t batch,
                                 int32_t s_q, int32_t h_q, const float* attn_sink,
                                 float softmax_scale, void* out_bf16, float* lse,
                                 void* workspace, size_t workspace_bytes_in, int32_t num_splits,
                                 hipStream_t stream) {
  const ExtraCache extra{extra_kv_cache, extra_num_blocks, extra_block_size,
                         extra_block_stride_bytes, extra_indices, extra_topk};
  return sparse_decode_impl("sparse_decode_dual", q_bf16, kv_cache, num_blocks, block_size,
                            block_stride_bytes, indices, topk, &extra, batch, s_q, h_q,
                            attn_sink, softmax_scale, out_bf16, lse, workspace,
                            workspace_bytes_in, num_splits, NVFP4_MLA_RECORD_BYTES, stream);
}

int nvfp4_mla_sparse_decode_dual_ds_mla(
    const void* q_bf16, const uint8_t* kv_cache, int64_t num_blocks, int32_t block_size,
    int64_t block_stride_bytes, const int32_t* indices, int32_t topk,
    const uint8_t* extra_kv_cache, int64_t extra_num_blocks, int32_t extra_block_size,
    int64_t extra_block_stride_bytes, const int32_t* extra_indices, int32_t extra_topk,
    int32_t batch, int32_t s_q, int32_t h_q, const float* attn_sink, float softmax_scale,
    void* out_bf16, float* lse, void* workspace, size_t workspace_bytes_in, int32_t num_splits,
    hipStream_t stream) {
  const ExtraCache extra{extra_kv_cache, extra_num_blocks, extra_block_size,
                         extra_block_stride_bytes, extra_indices, extra_topk};
  return sparse_decode_impl("sparse_decode_dual_ds_mla", q_bf16, kv_cache, num_blocks,
                            block_size, block_stride_bytes, indices, topk, &extra, batch, s_q,
                            h_q, attn_sink, softmax_scale, out_bf16, lse, workspace,
                            workspace_bytes_in, num_splits, NVFP4_MLA_DS_MLA_RECORD_BYTES,
                            stream);
}

int nvfp4_mla_combine(const float* o_partial, const float* lse_partial, int32_t num_splits,
                      int64_t rows, int32_t h_q, const float* attn_sink, void* out_bf16,
                      float* lse, hipStream_t stream) {
  if (num_splits < 1 || num_splits > 4096)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "num_splits = %d must be in [1, 4096]", num_splits);
  if (rows < 0 || h_q < 1)
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "rows must be >= 0 and h_q >= 1");
  // 64 work-items per (row, head) in one launch of at most 2^32 - 1
  if (rows * (int64_t)h_q * 64 > INT64_C(0xFFFFFFFF))
    return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT,
                "rows * h_q = %lld too large: one launch holds at most 2^26 - 1 (row, head) "
                "pairs (64 work-items each)", (long long)(rows * (int64_t)h_q));
  if (rows > 0) {
    if (!o_partial || !lse_partial || !out_bf16 || !lse)
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "o_partial, lse_partial, out, lse must be non-NULL");
    if (!aligned(o_partial, 16) || !aligned(out_bf16, 8) || !aligned(lse_partial, 4) ||
        !aligned(lse, 4) || (attn_sink && !aligned(attn_sink, 4)))
      return fail(NVFP4_MLA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  }
  int rc = check_device(nullptr);
  if (rc) return rc;
  hipError_t e = nvfp4::launch_combine(o_partial, lse_partial, num_splits, rows, h_q, attn_sink,
                                       static_cast<uint16_t*>(out_bf16), lse,
                                       stream);
  if (e != hipSuccess)
    return fail(NVFP4_MLA_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
