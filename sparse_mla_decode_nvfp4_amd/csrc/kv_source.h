// Where the tokens of one query row's top-k list live, for both decode
// kernels.  The plain decode reads one index list into one paged cache.  The
// dual-cache decode attends, with one softmax, over two lists: a primary
// cache (the sliding window, 64-token pages) and an extra cache (the indexer's
// top-k, 2- or 64-token pages), each list holding slot ids of its own cache
// (sglang PR #38646 "[SM120] opt-in NVFP4 sparse-MLA KV cache format for
// DeepSeek-V4": Modifications, the pool's page sizes; Performance, primary
// top-k 128 plus extra top-k 512).  Positions [0, topk0) of the joined list
// are primary slots, [topk0, topk) extra ones.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

template <bool kDual>
struct RowSource {
  const int32_t* idx0;   // this row's primary list
  const int32_t* idx1;   // this row's extra list (dual only)
  int32_t topk0;         // primary list length (= topk without an extra cache)

  __device__ __forceinline__ RowSource(const DecodeArgs& a, int row) {
    topk0 = kDual ? a.topk0 : a.topk;
    idx0 = a.indices + (size_t)row * topk0;
    idx1 = kDual ? a.indices1 + (size_t)row * (a.topk - topk0) : nullptr;
  }

  // Raw index at joined position p, 0 <= p < topk.
  __device__ __forceinline__ int32_t load(int p) const {
    if constexpr (!kDual) {
      return idx0[p];
    } else {
      const int32_t* ptr = p < topk0 ? idx0 + p : idx1 + (p - topk0);
      return *ptr;
    }
  }
};

struct RecRef {
  const uint8_t* ptr;   // record bytes (record 0 of the primary cache when !ok)
  bool ok;              // the token takes part in the softmax
};

// Record of raw index v found at joined position p.  A token takes part when
// its position is in the list (`in_list`) and v is a slot of its own cache
// (0 <= v < that cache's slot count).  Others read record 0 of the primary
// cache, which always exists, and are masked by the caller.
template <bool kDual>
__device__ __forceinline__ RecRef resolve_rec(const DecodeArgs& a, int32_t v, bool in_list, int p,
                                              int topk0) {
  if constexpr (!kDual) {
    const bool ok = in_list && v >= 0 && (int64_t)v < a.num_slots;
    return {a.cache + (ok ? a.pa.offset((uint32_t)v) : 0), ok};
  } else {
    const bool extra = p >= topk0;
    // both bounds compared, then the results selected: a per-lane select of
    // the two bounds lets the compiler turn them into a per-lane vector load
    // of the kernel argument, and that load waits for every gather in flight
    const bool below0 = (int64_t)v < a.num_slots;
    const bool below1 = (int64_t)v < a.num_slots1;
    const bool ok = in_list && v >= 0 && (extra ? below1 : below0);
    const uint32_t slot = ok ? (uint32_t)v : 0u;
    const uint8_t* r0 = a.cache + a.pa.offset(slot);
    const uint8_t* r1 = a.cache1 + a.pa1.offset(slot);
    return {(ok && extra) ? r1 : (ok ? r0 : a.cache), ok};
  }
}

}  // namespace nvfp4
