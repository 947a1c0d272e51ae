"""Seeded synthetic inputs for the NVFP4 sparse-MLA decode path.

This module only draws inputs: latents, queries, top-k slot ids, sinks, page
tables and slot mappings.  It holds none of the method's arithmetic (no
quantization, no attention), so the test suite can feed the same inputs to the
HIP library and to the CPU oracle.

Every draw comes from numpy's PCG64 seeded as default_rng([config, stream,
rep]) with one stream per kind of input:
  0 channel scales, 1 NoPE latents, 2 RoPE latents, 3 queries,
  4 indices + invalid mask, 5 sinks, 6 page tables / lengths,
  7 sentinel cache bytes, 8 slot mapping, 9 norm weights and positions.

Value distributions (the same for every workload):
  NoPE  = N(0,1) * channel_scale[d], channel_scale ~ exp(U(ln 0.1, ln 4)) fixed
          per workload, and each element independently multiplied by 20 with
          probability 1 %;
  RoPE  = N(0,1);  Q = N(0,1);  sink = N(0,1) float32 per head.
All latents and queries are rounded to bfloat16 (round-to-nearest-even).
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

NOPE_DIM = 512
ROPE_DIM = 64
QK_DIM = 576
V_DIM = 512
RECORD_BYTES = 352


def _rng(config_id, stream, rep=0, pool=0):
    # pool > 0 gives the second cache of a dual-cache workload its own draws
    return np.random.default_rng([config_id, stream, rep] + ([pool] if pool else []))


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def channel_scales(config_id):
    r = _rng(config_id, 0)
    return np.exp(r.uniform(np.log(0.1), np.log(4.0), size=NOPE_DIM))


def latents(config_id, n, rep=0, pool=0):
    """bf16 NoPE [n,512] and RoPE [n,64] latents drawn for n tokens."""
    cs = channel_scales(config_id)
    r1 = _rng(config_id, 1, rep, pool)
    nope = r1.standard_normal((n, NOPE_DIM)) * cs[None, :]
    outlier = r1.random((n, NOPE_DIM)) < 0.01
    nope = np.where(outlier, nope * 20.0, nope)
    rope = _rng(config_id, 2, rep, pool).standard_normal((n, ROPE_DIM))
    return _bf16(nope), _bf16(rope)


def latents_torch(config_id, n, generator, device):
    """Same distributions as latents(), drawn with a seeded torch generator
    on `device` (used to fill whole multi-GB pools quickly)."""
    cs = torch.from_numpy(channel_scales(config_id)).to(device=device, dtype=torch.float32)
    nope = torch.randn((n, NOPE_DIM), generator=generator, device=device) * cs
    outlier = torch.rand((n, NOPE_DIM), generator=generator, device=device) < 0.01
    nope = torch.where(outlier, nope * 20.0, nope)
    rope = torch.randn((n, ROPE_DIM), generator=generator, device=device)
    return nope.to(torch.bfloat16), rope.to(torch.bfloat16)


@dataclass
class DecodeWorkload:
    """One decode step's inputs.

    indices are slot ids into a paged cache of num_blocks pages of block_size
    tokens (slot = page * block_size + offset); -1 marks an invalid entry.
    `slots` lists every distinct valid slot the indices (and the step's new
    tokens) reference, sorted, and latent/rope hold those tokens' latents in
    that order.  new_slots are the slots of the B*S_q tokens the step appends
    (the query tokens themselves), a subset of `slots`.
    """
    name: str
    config_id: int
    batch: int
    s_q: int
    h_q: int
    topk: int
    block_size: int
    num_blocks: int
    softmax_scale: float
    q: torch.Tensor                      # bf16 [B, S_q, H, 576]
    indices: np.ndarray                  # int32 [B, S_q, topk]
    sink: Optional[np.ndarray]           # float32 [H] or None
    slots: np.ndarray                    # int64 [n] sorted distinct
    latent: Optional[torch.Tensor]       # bf16 [n, 512] (None: not drawn)
    rope: Optional[torch.Tensor]         # bf16 [n, 64]
    new_slots: np.ndarray                # int64 [B * S_q]
    description: str = ""
    extra: dict = field(default_factory=dict)
    record_bytes: int = RECORD_BYTES     # 352, or 432 for the nvfp4_ds_mla record

    @property
    def num_slots(self):
        return self.num_blocks * self.block_size

    def slot_rows(self, slots):
        """Row of each slot in `self.slots` (-1 for negative slots)."""
        slots = np.asarray(slots, dtype=np.int64)
        rows = np.searchsorted(self.slots, np.maximum(slots, 0))
        return np.where(slots < 0, -1, rows)

    def new_token_rows(self):
        return self.slot_rows(self.new_slots)


def _page_table(r, pages_per_seq):
    """Random global page permutation split into per-sequence tables."""
    total = int(np.sum(pages_per_seq))
    perm = r.permutation(total)
    tables, off = [], 0
    for n in pages_per_seq:
        tables.append(perm[off:off + n])
        off += n
    return tables, total


def _finish(name, cid, batch, s_q, h_q, topk, bs, num_blocks, scale, idx,
            new_slots, with_sink, description, rep=0, extra=None, with_latents=True):
    q = _bf16(_rng(cid, 3, rep).standard_normal((batch, s_q, h_q, QK_DIM)))
    sink = (_rng(cid, 5, 0).standard_normal(h_q).astype(np.float32)
            if with_sink else None)
    used = np.concatenate([idx[idx >= 0].astype(np.int64), new_slots])
    slots = np.unique(used)
    if with_latents:
        latent, rope = latents(cid, len(slots), rep)
    else:
        latent = rope = None
    return DecodeWorkload(name, cid, batch, s_q, h_q, topk, bs, num_blocks,
                          float(np.float32(scale)), q, idx.astype(np.int32),
                          sink, slots, latent, rope, new_slots.astype(np.int64),
                          description, extra or {})


def tiny(rep=0):
    """Batch 1, s_q 1, 16 heads; a 256-token pool (4 pages of 64) that is
    filled entirely, 64 distinct random indices, no invalid entries, no sink,
    scale 1/sqrt(576).  The step's new token is the one at position 255."""
    cid, bs = 0, 64
    tables, total = _page_table(_rng(cid, 6, 0), [4])
    pos = _rng(cid, 4, rep).choice(256, size=64, replace=False)
    idx = (tables[0][pos // bs] * bs + pos % bs).reshape(1, 1, 64)
    new_slot = np.array([tables[0][255 // bs] * bs + 255 % bs])
    wl = _finish("tiny", cid, 1, 1, 16, 64, bs, total, 1.0 / 24.0, idx,
                 new_slot, False,
                 "tiny codec+decode: B1 S_q1 H16, pool 256, topk 64, no sink",
                 rep)
    wl.slots = np.sort((tables[0][:, None] * bs + np.arange(bs)[None, :]).reshape(-1))
    wl.latent, wl.rope = latents(cid, len(wl.slots), rep)
    return wl


def decode_h64(rep=0, batch=32, with_latents=True):
    """B 32, s_q 1, 64 heads, 32768 tokens per sequence in 64-token pages,
    random page table, 2048 distinct positions per query, 5 % invalid, sink."""
    cid, bs, seq, topk = 1, 64, 32768, 2048
    tables, total = _page_table(_rng(cid, 6, 0), [seq // bs] * batch)
    r4 = _rng(cid, 4, rep)
    idx = np.empty((batch, 1, topk), dtype=np.int64)
    new_slots = np.empty(batch, dtype=np.int64)
    for b in range(batch):
        pos = r4.choice(seq, size=topk, replace=False)
        idx[b, 0] = tables[b][pos // bs] * bs + pos % bs
        new_slots[b] = tables[b][(seq - 1) // bs] * bs + (seq - 1) % bs
    inval = r4.random(idx.shape) < 0.05
    idx[inval] = -1
    return _finish("decode_h64", cid, batch, 1, 64, topk, bs, total,
                   1.0 / 24.0, idx, new_slots, True,
                   f"h_q 64: B{batch} S_q1, 32768-token contexts, topk 2048, "
                   "5% invalid, sink", rep, with_latents=with_latents)


def decode_h64_ds_mla(rep=0, batch=32, with_latents=True):
    """decode_h64's inputs over a cache of 432-byte nvfp4_ds_mla records."""
    wl = decode_h64(rep=rep, batch=batch, with_latents=with_latents)
    wl.name = "decode_h64_ds_mla"
    wl.record_bytes = 432
    wl.description = wl.description.replace("h_q 64:", "h_q 64, 432-byte records:")
    return wl


def decode_h128_varlen(rep=0, batch=64, with_latents=True):
    """B 64, s_q 1, 128 heads, context length ~ U[4096, 131072], 64-token
    pages, topk = min(2048, len) distinct positions, 2 % invalid, sink."""
    cid, bs, topk = 2, 64, 2048
    r6 = _rng(cid, 6, 0)
    lens = r6.integers(4096, 131072, endpoint=True, size=batch)
    pages = [int(-(-int(n) // bs)) for n in lens]
    tables, total = _page_table(r6, pages)
    r4 = _rng(cid, 4, rep)
    idx = np.empty((batch, 1, topk), dtype=np.int64)
    new_slots = np.empty(batch, dtype=np.int64)
    for b in range(batch):
        n = int(lens[b])
        k = min(topk, n)
        pos = r4.choice(n, size=k, replace=False)
        row = np.full(topk, -1, dtype=np.int64)
        row[:k] = tables[b][pos // bs] * bs + pos % bs
        idx[b, 0] = row
        new_slots[b] = tables[b][(n - 1) // bs] * bs + (n - 1) % bs
    inval = r4.random(idx.shape) < 0.02
    idx[inval] = -1
    return _finish("decode_h128_varlen", cid, batch, 1, 128, topk, bs, total,
                   1.0 / 24.0, idx, new_slots, True,
                   f"h_q 128 varlen: B{batch} S_q1, lengths U[4096,131072], "
                   "topk 2048, 2% invalid, sink", rep,
                   extra={"lengths": lens}, with_latents=with_latents)


def decode_h16_mtp(rep=0, batch=256, with_latents=True):
    """B 256, s_q 2 (MTP), 16 heads, 65536-token contexts, 64-token pages.
    Query j sits at position L-2+j; its 640 indices are the 128-token window
    ending at that position followed by 512 distinct positions drawn from the
    older history; 3 % invalid; sink."""
    cid, bs, seq, s_q, win, extra_k = 4, 64, 65536, 2, 128, 512
    topk = win + extra_k
    tables, total = _page_table(_rng(cid, 6, 0), [seq // bs] * batch)
    r4 = _rng(cid, 4, rep)
    idx = np.empty((batch, s_q, topk), dtype=np.int64)
    new_slots = np.empty(batch * s_q, dtype=np.int64)
    for b in range(batch):
        for j in range(s_q):
            p = seq - s_q + j
            window = np.arange(p - win + 1, p + 1)
            hist = r4.choice(p - win + 1, size=extra_k, replace=False)
            pos = np.concatenate([window, hist])
            idx[b, j] = tables[b][pos // bs] * bs + pos % bs
            new_slots[b * s_q + j] = tables[b][p // bs] * bs + p % bs
    inval = r4.random(idx.shape) < 0.03
    idx[inval] = -1
    return _finish("decode_h16_mtp", cid, batch, s_q, 16, topk, bs, total,
                   1.0 / 24.0, idx, new_slots, True,
                   f"h_q 16 MTP: B{batch} S_q2, 65536-token contexts, topk 640 "
                   "(128 window + 512 history), 3% invalid, sink", rep,
                   with_latents=with_latents)


@dataclass
class AppendWorkload:
    """Quantize-append inputs: N new tokens scattered into a sentinel-filled
    cache of num_blocks pages by a slot mapping with -1 entries."""
    name: str
    num_tokens: int
    block_size: int
    num_blocks: int
    latent: torch.Tensor          # bf16 [N, 512]
    rope: torch.Tensor            # bf16 [N, 64]
    slot_mapping: np.ndarray      # int64 [N]
    sentinel: np.ndarray          # uint8 [num_blocks * block_size, 352]


def append_write(rep=0, num_tokens=16384, num_slots=262144, p_skip=0.10):
    """16384 tokens into a 262144-slot cache, 10 % of slots -1, the rest
    distinct uniform slots; the cache starts as random sentinel bytes."""
    cid, bs = 3, 64
    latent, rope = latents(cid, num_tokens, rep)
    r8 = _rng(cid, 8, rep)
    sm = r8.choice(num_slots, size=num_tokens, replace=False).astype(np.int64)
    sm[r8.random(num_tokens) < p_skip] = -1
    sentinel = _rng(cid, 7, rep).integers(0, 256, size=(num_slots, RECORD_BYTES),
                                          dtype=np.uint8)
    return AppendWorkload("append_write", num_tokens, bs, num_slots // bs,
                          latent, rope, sm, sentinel)


@dataclass
class NormRopeInputs:
    """The fused write path's extra inputs: an RMSNorm weight, a rotary table
    and each token's position."""
    norm_weight: torch.Tensor            # bf16 [512]
    eps: float
    cos_sin: torch.Tensor                # float32 [max_position, 64]: cos, then sin
    positions: np.ndarray                # int64 [num_tokens]


def rotary_table(max_position, base=10000.0):
    """The usual rotary angles pos * base^(-2i/64) for the 32 frequencies,
    as a float32 table [max_position, 64] of their cosines then sines (an
    input of the fused write path, drawn here the way models build it)."""
    inv = base ** (-np.arange(0, 64, 2, dtype=np.float64) / 64.0)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32))


def norm_rope_inputs(num_tokens, rep=0, max_position=8192, eps=1e-6, p_outside=0.0):
    """Seeded fused-path inputs for num_tokens tokens (config 3's stream 9):
    weight ~ U(0.5, 1.5) in bf16, positions uniform in [0, max_position),
    a fraction p_outside of them moved just outside the table."""
    r = _rng(3, 9, rep)
    weight = _bf16(r.uniform(0.5, 1.5, NOPE_DIM))
    pos = r.integers(0, max_position, size=num_tokens).astype(np.int64)
    out = r.random(num_tokens) < p_outside
    pos[out] = np.where(r.random(int(out.sum())) < 0.5, -1, max_position)
    return NormRopeInputs(weight, float(np.float32(eps)), rotary_table(max_position), pos)


@dataclass
class PagedPool:
    """One paged cache of a dual-cache workload: its geometry, and the
    sorted distinct slots its indices (and new tokens) use with those tokens'
    latents in that order."""
    block_size: int
    num_blocks: int
    slots: np.ndarray                    # int64 [n] sorted distinct
    latent: Optional[torch.Tensor]       # bf16 [n, 512] (None: not drawn)
    rope: Optional[torch.Tensor]         # bf16 [n, 64]

    @property
    def num_slots(self):
        return self.num_blocks * self.block_size

    def slot_rows(self, slots):
        slots = np.asarray(slots, dtype=np.int64)
        rows = np.searchsorted(self.slots, np.maximum(slots, 0))
        return np.where(slots < 0, -1, rows)


@dataclass
class DualDecodeWorkload:
    """One dual-cache decode step: `indices` are slot ids of the primary pool,
    `extra_indices` slot ids of the extra pool; one softmax covers both.  The
    step's new tokens (the queries themselves) go to the primary pool."""
    name: str
    config_id: int
    batch: int
    s_q: int
    h_q: int
    softmax_scale: float
    q: torch.Tensor                      # bf16 [B, S_q, H, 576]
    sink: Optional[np.ndarray]           # float32 [H]
    primary: PagedPool
    extra_pool: PagedPool
    indices: np.ndarray                  # int32 [B, S_q, topk0]
    extra_indices: np.ndarray            # int32 [B, S_q, topk1]
    new_slots: np.ndarray                # int64 [B * S_q], primary slots
    description: str = ""

    @property
    def topk(self):
        return self.indices.shape[2] + self.extra_indices.shape[2]


def decode_h16_mtp_dual(rep=0, batch=256, with_latents=True, extra_block_size=2):
    """The h_q 16 MTP decode with its two index kinds in two caches, as the
    DeepSeek-V4 pool keeps them: B 256, s_q 2, 16 heads, 65536-token
    contexts.  Query j sits at position L-2+j.  Primary (sliding-window)
    cache: each sequence's last 256 positions in four 64-token pages; its list
    is the 128-token window ending at the query.  Extra cache: the whole
    history in `extra_block_size`-token pages (2 by default); its list is 512
    distinct positions drawn from before the window.  3 % of each list
    invalid; sink."""
    cid, bs0, seq, s_q, win, extra_k = 5, 64, 65536, 2, 128, 512
    bs1 = extra_block_size
    recent = 256                                   # positions the primary pool keeps
    r6 = _rng(cid, 6, 0)
    t0, total0 = _page_table(r6, [recent // bs0] * batch)
    t1, total1 = _page_table(r6, [seq // bs1] * batch)
    r4 = _rng(cid, 4, rep)
    idx0 = np.empty((batch, s_q, win), dtype=np.int64)
    idx1 = np.empty((batch, s_q, extra_k), dtype=np.int64)
    new_slots = np.empty(batch * s_q, dtype=np.int64)
    base = seq - recent
    for b in range(batch):
        for j in range(s_q):
            p = seq - s_q + j
            window = np.arange(p - win + 1, p + 1) - base
            idx0[b, j] = t0[b][window // bs0] * bs0 + window % bs0
            hist = r4.choice(p - win + 1, size=extra_k, replace=False)
            idx1[b, j] = t1[b][hist // bs1] * bs1 + hist % bs1
            new_slots[b * s_q + j] = t0[b][(p - base) // bs0] * bs0 + (p - base) % bs0
    idx0[r4.random(idx0.shape) < 0.03] = -1
    idx1[r4.random(idx1.shape) < 0.03] = -1
    q = _bf16(_rng(cid, 3, rep).standard_normal((batch, s_q, 16, QK_DIM)))
    sink = _rng(cid, 5, 0).standard_normal(16).astype(np.float32)
    slots0 = np.unique(np.concatenate([idx0[idx0 >= 0], new_slots]))
    slots1 = np.unique(idx1[idx1 >= 0])
    lat0 = rope0 = lat1 = rope1 = None
    if with_latents:
        lat0, rope0 = latents(cid, len(slots0), rep)
        lat1, rope1 = latents(cid, len(slots1), rep, pool=1)
    return DualDecodeWorkload(
        "decode_h16_mtp_dual", cid, batch, s_q, 16, float(np.float32(1.0 / 24.0)), q, sink,
        PagedPool(bs0, total0, slots0, lat0, rope0), PagedPool(bs1, total1, slots1, lat1, rope1),
        idx0.astype(np.int32), idx1.astype(np.int32), new_slots,
        f"h_q 16 MTP dual cache: B{batch} S_q2, 65536-token contexts, primary 128-token "
        f"window (64-token pages) + extra 512 history ({bs1}-token pages), 3% invalid, sink")


def _distinct(r, n, k):
    """k distinct integers of [0, n) in random order (n >= k): a batch of
    draws with replacement, duplicates dropped, topped up until k remain;
    O(k) where choice(n, k, replace=False) is O(n)."""
    got = np.empty(0, dtype=np.int64)
    while len(got) < k:
        got = np.unique(np.concatenate([got, r.integers(0, n, size=k + k // 4 + 8)]))
    return got[r.permutation(len(got))[:k]]


def prefill_dual(rep=0, tokens=4096, h_q=64, seq=65536, with_latents=True, extra_block_size=64):
    """Sparse prefill as the pages benchmark it: one sequence of `seq` tokens
    whose last `tokens` positions are the query tokens (batch 1, s_q =
    tokens), each attending, with one softmax, to its 128-token sliding
    window (primary cache, 64-token pages) and to 512 distinct positions
    drawn from before its window (extra cache, the whole sequence in
    `extra_block_size`-token pages).  3 % of each list invalid; sink; Q
    N(0,1) for `h_q` heads."""
    cid, bs0, win, extra_k = 6, 64, 128, 512
    bs1 = extra_block_size
    first = seq - tokens                        # position of the first query token
    base = ((first - win + 1) // bs0) * bs0     # the primary pool starts at a page boundary
    r6 = _rng(cid, 6, 0)
    t0, total0 = _page_table(r6, [-(-(seq - base) // bs0)])
    t1, total1 = _page_table(r6, [-(-seq // bs1)])
    r4 = _rng(cid, 4, rep)
    idx0 = np.empty((1, tokens, win), dtype=np.int64)
    idx1 = np.empty((1, tokens, extra_k), dtype=np.int64)
    new_slots = np.empty(tokens, dtype=np.int64)
    for j in range(tokens):
        p = first + j
        window = np.arange(p - win + 1, p + 1) - base
        idx0[0, j] = t0[0][window // bs0] * bs0 + window % bs0
        hist = _distinct(r4, p - win + 1, extra_k)
        idx1[0, j] = t1[0][hist // bs1] * bs1 + hist % bs1
        new_slots[j] = t0[0][(p - base) // bs0] * bs0 + (p - base) % bs0
    idx0[r4.random(idx0.shape) < 0.03] = -1
    idx1[r4.random(idx1.shape) < 0.03] = -1
    # Q drawn in float32 directly (up to 8192 x 64 x 576 values)
    q = torch.from_numpy(_rng(cid, 3, rep).standard_normal((1, tokens, h_q, QK_DIM),
                                                           dtype=np.float32)).to(torch.bfloat16)
    sink = _rng(cid, 5, 0).standard_normal(h_q).astype(np.float32)
    slots0 = np.unique(np.concatenate([idx0[idx0 >= 0], new_slots]))
    slots1 = np.unique(idx1[idx1 >= 0])
    lat0 = rope0 = lat1 = rope1 = None
    if with_latents:
        lat0, rope0 = latents(cid, len(slots0), rep)
        lat1, rope1 = latents(cid, len(slots1), rep, pool=1)
    return DualDecodeWorkload(
        f"prefill_dual_h{h_q}_t{tokens}", cid, 1, tokens, h_q, float(np.float32(1.0 / 24.0)), q,
        sink, PagedPool(bs0, total0, slots0, lat0, rope0),
        PagedPool(bs1, total1, slots1, lat1, rope1), idx0.astype(np.int32),
        idx1.astype(np.int32), new_slots,
        f"sparse prefill: {tokens} query tokens of a {seq}-token sequence, h_q {h_q}, "
        f"primary 128-token window + extra 512 history ({bs1}-token pages), 3% invalid, sink")


DECODE_WORKLOADS = {
    "tiny": tiny,
    "decode_h64": decode_h64,
    "decode_h128_varlen": decode_h128_varlen,
    "decode_h16_mtp": decode_h16_mtp,
    "decode_h64_ds_mla": decode_h64_ds_mla,
}

DUAL_WORKLOADS = {
    "decode_h16_mtp_dual": decode_h16_mtp_dual,
    "prefill_dual_h64_t4096": prefill_dual,
}

# the pages' operator benchmark grid: heads per rank x query tokens
PREFILL_HEADS = (16, 32, 64)
PREFILL_TOKENS = (64, 1024, 2048, 4096, 8192)


def dual_workload(name):
    """Generator of a dual-cache workload by name: the entries above, or
    prefill_dual_h{H}_t{T} for any head count H and token count T."""
    if name in DUAL_WORKLOADS:
        return DUAL_WORKLOADS[name]
    if name.startswith("prefill_dual_h") and "_t" in name:
        h, t = name[len("prefill_dual_h"):].split("_t")
        return lambda rep=0, with_latents=True: prefill_dual(rep=rep, tokens=int(t), h_q=int(h),
                                                             with_latents=with_latents)
    return None
