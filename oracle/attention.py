"""Sparse MLA decode attention and the split-KV combine, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ([FlashMLA-18] PR description: d_qk = 576, d_v = 512, top-k
token records gathered by index with invalid indices and an optional per-head
attention sink; every query head attends to the same latent):

  for each query row (b, s) and head h, over the valid indices t (index >= 0,
  duplicates counted as often as they appear):
      z_t  = softmax_scale * <q_h, K_t>            (K_t: 576-dim dequantized key)
      m    = max_t z_t,   l = sum_t exp(z_t - m),   LSE = m + ln l
      O    = sum_t exp(z_t - m) V_t / (l + exp(sink_h - m))   (sink term only
                                                               when a sink is given)
  V_t is the first 512 dimensions of K_t.  A row with no valid index has
  O = 0 and LSE = -inf.  LSE is the natural-log sum over tokens and excludes
  the sink, so partial results over disjoint index sets can be merged first and
  the sink applied once afterwards.

Dual-cache decode ([sglang-38646] Modifications: the pool keeps a primary
cache and an extra cache with their own page sizes, and slot ids are those of
each cache; Performance: one attention over primary top-k 128 plus extra top-k
512): the same definition over the joined list of a primary list (rows of the
primary records) followed by an extra list (rows of the extra records).

Split-KV combine (LSE-weighted merge of partial results over disjoint index
subsets): LSE = ln sum_i exp(LSE_i),  O = sum_i exp(LSE_i - LSE) O_i divided
by (1 + exp(sink - LSE)) when a sink is given; all LSE_i = -inf gives O = 0,
LSE = -inf.  The partial O_i are the sink-free normalised outputs of each
subset.
"""

import numpy as np

from .codec import dequantize_records
from .formats import V_DIM


def sparse_decode(q, records, idx, softmax_scale, sink=None):
    """Reference decode.

    q:       float64 [B, S, H, 576]
    records: uint8 [R, 352 or 432]  -- the token records the indices refer to
    idx:     int [B, S, topk] -- row numbers into `records`, < 0 = invalid
    softmax_scale: the float32 scale, used at its exact value
    sink:    float64 [H] or None
    returns  O float64 [B, S, H, 512], LSE float64 [B, S, H]
    """
    q = np.asarray(q, dtype=np.float64)
    idx = np.asarray(idx).astype(np.int64)
    b_, s_, h_, d_ = q.shape
    kv = dequantize_records(records)
    scale = float(np.float32(softmax_scale))
    out = np.zeros((b_, s_, h_, V_DIM))
    lse = np.full((b_, s_, h_), -np.inf)
    for b in range(b_):
        for s in range(s_):
            valid = idx[b, s][idx[b, s] >= 0]
            if valid.size == 0:
                continue
            k = kv[valid]                       # [n, 576]
            v = k[:, :V_DIM]                    # [n, 512]
            z = scale * (q[b, s] @ k.T)         # [H, n]
            m = z.max(axis=1)
            e = np.exp(z - m[:, None])
            l = e.sum(axis=1)
            lse[b, s] = m + np.log(l)
            denom = l.copy()
            if sink is not None:
                denom = denom + np.exp(np.asarray(sink, dtype=np.float64) - m)
            out[b, s] = (e @ v) / denom[:, None]
    return out, lse


def sparse_decode_dual(q, records, idx, extra_records, extra_idx, softmax_scale, sink=None):
    """Reference dual-cache decode.

    records, idx:             primary records [R0, W] and row numbers [B, S, topk0]
    extra_records, extra_idx: extra records [R1, W] and row numbers [B, S, topk1]
    (W = 352 or 432, the same for both).  Every valid entry of either list is
    one token of a single softmax (sink once): sparse_decode over the records
    of both caches stacked, with the extra list's row numbers moved past the
    primary records.
    """
    records = np.asarray(records, dtype=np.uint8)
    extra_records = np.asarray(extra_records, dtype=np.uint8)
    assert records.ndim == 2 and extra_records.ndim == 2
    assert records.shape[1] == extra_records.shape[1], "one record format for both caches"
    idx = np.asarray(idx).astype(np.int64)
    extra_idx = np.asarray(extra_idx).astype(np.int64)
    joined_idx = np.concatenate(
        [idx, np.where(extra_idx >= 0, extra_idx + records.shape[0], -1)], axis=-1)
    joined = np.concatenate([records, extra_records], axis=0)
    return sparse_decode(q, joined, joined_idx, softmax_scale, sink=sink)


def partial_decode(q, records, idx, softmax_scale):
    """Sink-free decode over one index subset: the (O_i, LSE_i) of a split."""
    return sparse_decode(q, records, idx, softmax_scale, sink=None)


def combine(o_parts, lse_parts, sink=None):
    """Merge split results.

    o_parts:   float64 [P, ..., H, 512]  (sink-free, normalised per split)
    lse_parts: float64 [P, ..., H]
    sink:      float64 [H] or None
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    mx = lse_parts.max(axis=0)
    empty = np.isneginf(mx)
    safe_mx = np.where(empty, 0.0, mx)
    w = np.exp(lse_parts - safe_mx)                   # exp(-inf) = 0
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, safe_mx + np.log(np.where(empty, 1.0, tot)))
    norm_w = np.where(empty, 0.0, w / np.where(empty, 1.0, tot))
    out = (norm_w[..., None] * o_parts).sum(axis=0)
    if sink is not None:
        sink = np.asarray(sink, dtype=np.float64)
        factor = np.where(empty, 1.0, 1.0 / (1.0 + np.exp(sink - np.where(empty, 0.0, lse))))
        out = out * factor[..., None]
    out = np.where(empty[..., None], 0.0, out)
    return out, lse
