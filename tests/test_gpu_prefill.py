"""GPU parity of the sparse prefill: many query tokens of one sequence (batch
1, s_q = tokens), each with its own 128-token sliding-window list into the
primary cache and 512-entry history list into the extra cache, one softmax
over both.  Small sequences are compared on every row; the pages' operator
shapes (4096 tokens at 64 heads, 1024 at 16) on sampled rows, in the
planner's launch configuration.  O within |d| <= 1e-2 + 2e-2 |ref|, LSE within
1e-3.
"""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import codec as OC
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import assert_decode_close, f64, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_prefill(lib, wl, rows):
    p0, p1 = wl.primary, wl.extra_pool
    note(f"{wl.name}: tokens={wl.s_q} h={wl.h_q} primary {p0.num_slots} slots, "
         f"extra {p1.num_slots} slots, checking {len(rows)} rows")
    c0 = lib.new_cache(p0.num_blocks, p0.block_size, DEV)
    c1 = lib.new_cache(p1.num_blocks, p1.block_size, DEV)
    lib.quantize_append(p0.latent.to(DEV), p0.rope.to(DEV), torch.from_numpy(p0.slots).to(DEV), c0)
    lib.quantize_append(p1.latent.to(DEV), p1.rope.to(DEV), torch.from_numpy(p1.slots).to(DEV), c1)
    splits = lib.plan(wl.batch, wl.s_q, wl.h_q, wl.topk)
    o, lse = lib.sparse_decode_dual(wl.q.to(DEV), c0, torch.from_numpy(wl.indices).to(DEV), c1,
                                    torch.from_numpy(wl.extra_indices).to(DEV), wl.softmax_scale,
                                    sink=torch.from_numpy(wl.sink).to(DEV), num_splits=splits)
    torch.cuda.synchronize()
    n = wl.s_q
    o = o.reshape(n, wl.h_q, 512).cpu()
    lse = lse.reshape(n, wl.h_q).cpu()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    # the oracle quantizes the records the checked rows use, from the same latents
    parts = []
    for pool, ids in ((p0, wl.indices.reshape(n, -1)[rows]), (p1, wl.extra_indices.reshape(n, -1)[rows])):
        need = np.unique(ids[ids >= 0])
        pr = pool.slot_rows(need)
        recs = OC.quantize_records(f64(pool.latent[pr]), f64(pool.rope[pr]))
        local = np.where(ids >= 0, np.searchsorted(need, np.maximum(ids, 0)), -1)
        parts.append((recs, local[None]))
    q = f64(wl.q.reshape(n, wl.h_q, 576)[rows])[None]
    o_ref, l_ref = OA.sparse_decode_dual(q, parts[0][0], parts[0][1], parts[1][0], parts[1][1],
                                         wl.softmax_scale, sink=wl.sink.astype(np.float64))
    worst = assert_decode_close(o[rows], lse[rows], o_ref[0], l_ref[0], wl.name)
    note(f"{wl.name}: splits={splits}, worst error/bound = {worst:.3f}")
    del c0, c1
    torch.cuda.empty_cache()


@pytest.mark.parametrize("h", [16, 32, 64])
def test_prefill_64_tokens_every_row(lib, h):
    """64 query tokens: the size at which the pages see an operator
    regression; every row checked."""
    wl = W.prefill_dual(tokens=64, h_q=h, seq=4096)
    run_prefill(lib, wl, list(range(64)))


def test_prefill_ragged_token_count_every_row(lib):
    wl = W.prefill_dual(tokens=77, h_q=48, seq=2048, extra_block_size=2)
    run_prefill(lib, wl, list(range(77)))


@pytest.mark.parametrize("h,tokens,rows", [
    (64, 4096, [0, 1, 63, 64, 1000, 2047, 2048, 4094, 4095]),
    (16, 1024, [0, 5, 511, 512, 1022, 1023]),
])
def test_prefill_operator_shapes(lib, h, tokens, rows):
    wl = W.prefill_dual(tokens=tokens, h_q=h)
    run_prefill(lib, wl, rows)
