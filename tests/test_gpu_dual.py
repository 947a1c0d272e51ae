"""GPU parity of the dual-cache decode (one softmax over a primary list of
slot ids into one paged cache and an extra list into a second cache with its
own page size) against the fp64 oracle: O within |d| <= 1e-2 + 2e-2 |ref|,
LSE within 1e-3, -inf rows exact.  Small cases cover both kernels (16- and
32-head groups), lists whose boundary falls inside a 16-token chunk and a
64-token tile, empty lists, power-of-two, odd and one-token pages, split
counts, and indices that are valid in one cache but beyond the other.  The
full-size MTP workload runs in the planner's launch configuration and is
compared on every row.  Since the kernels' arithmetic depends only on the joined token order,
a dual decode must also equal, bit for bit, the plain decode over one cache
holding both pools' records with the lists concatenated.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import sparse_mla_decode_nvfp4_amd as M
from oracle import attention as OA
from oracle import codec as OC
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import ORACLE_THREADS, assert_decode_close, f64, nan_outputs, note, oracle_record_table

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 1.0 / 24


def dual_case(seed, b, s_q, h, k0, k1, bs0, nb0, bs1, nb1, p_inval=0.1, oob=False):
    rng = np.random.default_rng(seed)
    n0, n1 = nb0 * bs0, nb1 * bs1
    lat0, rope0 = W.latents(0, n0, rep=seed)
    lat1, rope1 = W.latents(0, n1, rep=seed, pool=1)
    r0 = OC.quantize_records(f64(lat0), f64(rope0))
    r1 = OC.quantize_records(f64(lat1), f64(rope1))
    q = torch.from_numpy(rng.standard_normal((b, s_q, h, 576)).astype(np.float32)).to(torch.bfloat16)
    i0 = rng.integers(0, n0, size=(b, s_q, k0)).astype(np.int32)
    i1 = rng.integers(0, n1, size=(b, s_q, k1)).astype(np.int32)
    i0[rng.random(i0.shape) < p_inval] = -1
    i1[rng.random(i1.shape) < p_inval] = -1
    if oob:
        # each beyond its own cache but inside the other one
        if k0:
            i0[..., 0] = n0 + 1
        if k1:
            i1[..., -1] = n1 + 2
    sink = rng.standard_normal(h).astype(np.float32)
    return r0, r1, q, i0, i1, sink


def run_dual(lib, case, bs0, bs1, splits):
    r0, r1, q, i0, i1, sink = case
    c0 = torch.from_numpy(r0.reshape(-1, bs0, 352)).to(DEV)
    c1 = torch.from_numpy(r1.reshape(-1, bs1, 352)).to(DEV)
    o, lse = lib.sparse_decode_dual(q.to(DEV), c0, torch.from_numpy(i0).to(DEV), c1,
                                    torch.from_numpy(i1).to(DEV), SCALE,
                                    sink=torch.from_numpy(sink).to(DEV), num_splits=splits)
    torch.cuda.synchronize()
    j0 = np.where(i0 >= r0.shape[0], -1, i0)
    j1 = np.where(i1 >= r1.shape[0], -1, i1)
    o_ref, l_ref = OA.sparse_decode_dual(f64(q), r0, j0, r1, j1, SCALE,
                                         sink=sink.astype(np.float64))
    return o, lse, o_ref, l_ref


CASES = [
    # b, s_q, h, topk0, topk1, bs0, nb0, bs1, nb1, splits
    (2, 2, 16, 128, 512, 64, 8, 2, 600, 1),      # the MTP shape at small batch
    (1, 2, 16, 128, 512, 64, 8, 2, 600, 0),
    (2, 1, 32, 100, 37, 64, 4, 64, 3, 1),        # boundary inside a chunk / tile
    (1, 1, 64, 7, 300, 48, 2, 2, 200, 3),        # odd primary pages
    (1, 1, 16, 0, 200, 64, 2, 2, 150, 1),        # empty primary list
    (2, 1, 32, 150, 0, 64, 4, 2, 10, 2),         # empty extra list
    (1, 1, 128, 64, 64, 64, 2, 3, 50, 4),        # three-token extra pages
    (3, 1, 16, 17, 33, 64, 2, 1, 90, 2),         # one-token extra pages
    (1, 1, 48, 1, 1, 64, 1, 2, 1, 1),            # one token each
]


@pytest.mark.parametrize("b,s_q,h,k0,k1,bs0,nb0,bs1,nb1,splits", CASES)
def test_dual_small_cases(lib, b, s_q, h, k0, k1, bs0, nb0, bs1, nb1, splits):
    what = f"dual b{b} s{s_q} h{h} k{k0}+{k1} pages {bs0}/{bs1} sp{splits}"
    note(what)
    case = dual_case(b * 977 + k0 + 3 * k1, b, s_q, h, k0, k1, bs0, nb0, bs1, nb1)
    o, lse, o_ref, l_ref = run_dual(lib, case, bs0, bs1, splits)
    assert_decode_close(o, lse, o_ref, l_ref, what)


@pytest.mark.parametrize("h", [16, 32])
def test_dual_index_ranges_are_per_cache(lib, h):
    """An index beyond its own cache is invalid even where the other cache
    has that slot; an all-invalid row gives O = 0, LSE = -inf."""
    note(f"dual per-cache ranges h={h}")
    case = dual_case(31 + h, 2, 1, h, 70, 90, 64, 2, 2, 200, oob=True)
    r0, r1, q, i0, i1, sink = case
    i0[1] = -1
    i1[1] = -1
    o, lse, o_ref, l_ref = run_dual(lib, (r0, r1, q, i0, i1, sink), 64, 2, 2)
    assert_decode_close(o, lse, o_ref, l_ref, "per-cache ranges")
    assert bool((o[1] == 0).all()) and bool(torch.isneginf(lse[1]).all())


@pytest.mark.parametrize("h,splits", [(16, 1), (16, 3), (64, 1), (64, 4)])
def test_dual_equals_plain_decode_over_joined_cache(lib, h, splits):
    note(f"dual vs joined cache h={h} splits={splits}")
    case = dual_case(400 + h + splits, 2, 2, h, 90, 230, 64, 2, 2, 150)
    r0, r1, q, i0, i1, sink = case
    o, lse, _, _ = run_dual(lib, case, 64, 2, splits)
    joined = torch.from_numpy(np.concatenate([r0, r1]).reshape(-1, 1, 352)).to(DEV)
    ji = np.concatenate([i0, np.where(i1 >= 0, i1 + r0.shape[0], -1)], axis=-1).astype(np.int32)
    o2, l2 = lib.sparse_decode(q.to(DEV), joined, torch.from_numpy(ji).to(DEV), SCALE,
                               sink=torch.from_numpy(sink).to(DEV), num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_dual_full_size_mtp_workload_every_row(lib):
    wl = W.decode_h16_mtp_dual()
    p0, p1 = wl.primary, wl.extra_pool
    rows = wl.batch * wl.s_q
    note(f"{wl.name}: rows={rows} topk={wl.topk} primary {p0.num_slots} slots, "
         f"extra {p1.num_slots} slots in {p1.block_size}-token pages")
    c0 = lib.new_cache(p0.num_blocks, p0.block_size, DEV)
    c1 = lib.new_cache(p1.num_blocks, p1.block_size, DEV)
    lib.quantize_append(p0.latent.to(DEV), p0.rope.to(DEV), torch.from_numpy(p0.slots).to(DEV), c0)
    lib.quantize_append(p1.latent.to(DEV), p1.rope.to(DEV), torch.from_numpy(p1.slots).to(DEV), c1)
    splits = lib.plan(wl.batch, wl.s_q, wl.h_q, wl.topk)
    o, lse = nan_outputs((wl.batch, wl.s_q, wl.h_q), DEV)
    lib.sparse_decode_dual(wl.q.to(DEV), c0, torch.from_numpy(wl.indices).to(DEV), c1,
                           torch.from_numpy(wl.extra_indices).to(DEV), wl.softmax_scale,
                           sink=torch.from_numpy(wl.sink).to(DEV), num_splits=splits,
                           out=o, lse=lse)
    torch.cuda.synchronize()
    o = o.reshape(rows, wl.h_q, 512).cpu()
    lse = lse.reshape(rows, wl.h_q).cpu()
    del c0, c1
    torch.cuda.empty_cache()
    note(f"{wl.name}: oracle records of both pools")
    tables = [oracle_record_table(p0.latent, p0.rope), oracle_record_table(p1.latent, p1.rope)]
    note(f"{wl.name}: oracle decode of all {rows} rows")
    q = wl.q.reshape(rows, wl.h_q, 576)
    i0 = wl.indices.reshape(rows, -1)
    i1 = wl.extra_indices.reshape(rows, -1)
    sink = wl.sink.astype(np.float64)

    def one(r):
        parts = []
        for pool, table, ids in ((p0, tables[0], i0[r]), (p1, tables[1], i1[r])):
            uniq = np.unique(ids[ids >= 0])
            recs = table[pool.slot_rows(uniq)]
            local = np.where(ids >= 0, np.searchsorted(uniq, np.maximum(ids, 0)), -1)
            parts.append((recs, local[None, None]))
        orr, lr = OA.sparse_decode_dual(f64(q[r])[None, None], parts[0][0], parts[0][1],
                                        parts[1][0], parts[1][1], wl.softmax_scale, sink=sink)
        return orr[0, 0], lr[0, 0]

    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        res = list(ex.map(one, range(rows)))
    o_ref = np.stack([x for x, _ in res])
    l_ref = np.stack([y for _, y in res])
    worst = assert_decode_close(o, lse, o_ref, l_ref, wl.name)
    note(f"{wl.name}: splits={splits}, worst error/bound over all {rows} rows = {worst:.3f}")


def test_dual_many_workgroups_every_row(lib):
    # >= 1024 workgroups: the 32-head kernel's two-pair shape over two caches
    note("dual many workgroups")
    case = dual_case(91, 512, 1, 64, 64, 100, 64, 8, 2, 300)
    o, lse, o_ref, l_ref = run_dual(lib, case, 64, 2, 1)
    assert_decode_close(o, lse, o_ref, l_ref, "dual many workgroups")
