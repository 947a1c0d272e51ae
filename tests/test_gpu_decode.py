"""GPU parity of the sparse decode and the split-KV combine against the fp64
oracle: O within |d| <= 1e-2 + 2e-2 |ref| elementwise, LSE within 1e-3, -inf
rows exact.  Small cases span several 16-token blocks, several head groups,
ragged tails, splits, invalid and out-of-range indices; the four decode
workloads run at full size with the planner's split choice (the launch
configuration the benchmark times) and are compared with the oracle on every
row (outputs start as NaN, so an unwritten row fails).  Rows with a single valid token pin the
decode's own dequant bit for bit over every (code, scale) product.
"""

import numpy as np
import pytest
import torch

import sparse_mla_decode_nvfp4_amd as M
from oracle import attention as OA
from oracle import codec as OC
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import (assert_decode_close, f64, nan_outputs, note, oracle_record_table,
                             oracle_rows, table_lookup)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def small_case(seed, b, s_q, h, topk, nblocks=24, bs=64, p_inval=0.1, with_sink=True,
               dup=False, oob=False):
    rng = np.random.default_rng(seed)
    nblocks = max(nblocks, -(-topk // bs) + 4)     # room for topk distinct slots
    n_slots = nblocks * bs
    lat, rope = W.latents(0, n_slots, rep=seed)
    recs = OC.quantize_records(f64(lat), f64(rope))
    q = torch.from_numpy(rng.standard_normal((b, s_q, h, 576)).astype(np.float32)).to(torch.bfloat16)
    idx = np.stack([rng.choice(n_slots, size=topk, replace=dup) for _ in range(b * s_q)])
    idx = idx.reshape(b, s_q, topk).astype(np.int32)
    idx[rng.random(idx.shape) < p_inval] = -1
    if oob:
        idx[..., 0] = n_slots + 5          # beyond the cache: treated as invalid
    sink = rng.standard_normal(h).astype(np.float32) if with_sink else None
    return recs, q, idx, sink, nblocks, bs


def run_small(lib, recs, q, idx, sink, nblocks, bs, splits, scale=1.0 / 24):
    cache = torch.from_numpy(recs.reshape(nblocks, bs, 352)).to(DEV)
    o, lse = lib.sparse_decode(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), scale,
                               sink=None if sink is None else torch.from_numpy(sink).to(DEV),
                               num_splits=splits)
    torch.cuda.synchronize()
    oob = idx >= recs.shape[0]
    idx_o = np.where(oob, -1, idx)
    o_ref, l_ref = OA.sparse_decode(f64(q), recs, idx_o, scale,
                                    sink=None if sink is None else sink.astype(np.float64))
    return o, lse, o_ref, l_ref


@pytest.mark.parametrize("b,s_q,h,topk,splits", [
    (1, 1, 16, 64, 1), (2, 1, 16, 1, 1), (3, 2, 16, 17, 1), (2, 2, 32, 100, 1),
    (1, 1, 64, 333, 1), (1, 2, 128, 200, 1), (2, 1, 16, 1000, 3), (1, 1, 64, 512, 0),
    (2, 1, 128, 700, 4), (1, 1, 16, 2048, 0), (1, 1, 16, 31, 2), (1, 1, 48, 129, 5),
    (3, 1, 96, 150, 2), (1, 3, 160, 90, 1),
])
def test_small_cases(lib, b, s_q, h, topk, splits):
    note(f"small case b={b} s_q={s_q} h={h} topk={topk} splits={splits}")
    recs, q, idx, sink, nb, bs = small_case(b * 1000 + topk, b, s_q, h, topk)
    o, lse, o_ref, l_ref = run_small(lib, recs, q, idx, sink, nb, bs, splits)
    assert_decode_close(o, lse, o_ref, l_ref, f"b{b} s{s_q} h{h} k{topk} sp{splits}")


def test_no_sink_duplicates_out_of_range_and_odd_pages(lib):
    recs, q, idx, sink, nb, bs = small_case(5, 2, 1, 32, 150, nblocks=30, bs=48, dup=True,
                                            oob=True, with_sink=False)
    o, lse, o_ref, l_ref = run_small(lib, recs, q, idx, sink, nb, bs, 2)
    assert_decode_close(o, lse, o_ref, l_ref, "dup/oob/bs48")


@pytest.mark.parametrize("h", [16, 32, 64])
def test_empty_rows_single_token_and_zero_query(lib, h):
    note(f"edge rows h={h}")
    recs, q, idx, sink, nb, bs = small_case(9, 4, 1, h, 40, p_inval=0.0)
    idx[0, 0, :] = -1                     # a row with no valid index
    idx[1, 0, :] = -1
    idx[1, 0, 13] = 77                    # exactly one valid token
    q[2] = 0                              # zero query: the plain mean
    for splits in (1, 3):
        o, lse, o_ref, l_ref = run_small(lib, recs, q, idx, sink, nb, bs, splits)
        assert_decode_close(o, lse, o_ref, l_ref, f"edge rows sp{splits}")
        o = o.cpu()
        assert bool((o[0] == 0).all()) and bool(torch.isneginf(lse[0]).all())
    # no sink: a single valid token returns its value row exactly (weight 1)
    o, lse, o_ref, l_ref = run_small(lib, recs, q, idx, None, nb, bs, 1)
    v = torch.from_numpy(OC.dequantize_records(recs[77:78])[0, :512]).to(torch.bfloat16)
    assert torch.equal(o[1, 0].cpu(), v[None].expand(h, 512))


@pytest.mark.parametrize("h,splits", [(16, 1), (32, 1), (64, 3)])
def test_large_scores_raise_the_running_max(lib, h, splits):
    # scores spread over tens of log2 units: the online max is raised (and
    # the accumulators rescaled) many times along the index list
    note(f"large scores h={h} splits={splits}")
    recs, q, idx, sink, nb, bs = small_case(31, 2, 1, h, 900)
    q = (q.float() * 24.0).to(torch.bfloat16)
    o, lse, o_ref, l_ref = run_small(lib, recs, q, idx, sink, nb, bs, splits)
    assert_decode_close(o, lse, o_ref, l_ref, f"large scores h{h}")


@pytest.mark.parametrize("h,splits", [(16, 1), (48, 1), (32, 1), (64, 2)])
def test_scores_rising_along_the_list_raise_the_max_in_every_tile(lib, h, splits):
    # the index list ordered by head 0's score, lowest first, with scores
    # spread over hundreds of log2 units: head 0's running max is raised in
    # nearly every tile (16-head kernel) or chunk (32-head kernel), so the
    # raise path (rescale and, in the 16-head kernel, P redone behind a
    # second barrier) runs all along the list
    note(f"rising scores h={h} splits={splits}")
    recs, q, idx, sink, nb, bs = small_case(47, 1, 2, h, 700, p_inval=0.0)
    q = (q.float() * 24.0).to(torch.bfloat16)
    k = OC.dequantize_records(recs)                       # [slots, 576] fp64
    for r in range(idx.shape[1]):
        s0 = k[idx[0, r]] @ f64(q)[0, r, 0]
        idx[0, r] = idx[0, r][np.argsort(s0, kind="stable")]
    o, lse, o_ref, l_ref = run_small(lib, recs, q, idx, sink, nb, bs, splits)
    assert_decode_close(o, lse, o_ref, l_ref, f"rising scores h{h}")


def test_split_counts_agree(lib):
    recs, q, idx, sink, nb, bs = small_case(21, 1, 2, 64, 1024)
    outs = []
    for splits in (1, 2, 7, 16):
        o, lse, o_ref, l_ref = run_small(lib, recs, q, idx, sink, nb, bs, splits)
        assert_decode_close(o, lse, o_ref, l_ref, f"splits {splits}")
        outs.append(o.float().cpu())
    # different split counts differ only by rounding: within the same bound
    for o in outs[1:]:
        assert bool(((o - outs[0]).abs() <= 1e-2 + 2e-2 * outs[0].abs()).all())


def test_workspace_too_small_is_reported(lib):
    recs, q, idx, sink, nb, bs = small_case(3, 1, 1, 16, 256)
    cache = torch.from_numpy(recs.reshape(nb, bs, 352)).to(DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(M.Nvfp4MlaError) as e:
        lib.sparse_decode(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), 0.04,
                          num_splits=4, workspace=ws)
    assert e.value.code == M.ERR_WORKSPACE_TOO_SMALL


def test_combine_matches_oracle(lib):
    rng = np.random.default_rng(4)
    p, r, h = 5, 7, 32
    o_part = rng.standard_normal((p, r, h, 512)).astype(np.float32)
    lse_part = (rng.standard_normal((p, r, h)) * 3).astype(np.float32)
    lse_part[rng.random((p, r, h)) < 0.2] = -np.inf
    lse_part[:, 3, 5] = -np.inf                 # fully empty (row, head)
    o_part[np.isneginf(lse_part)] = 0
    sink = rng.standard_normal(h).astype(np.float32)
    for s in (None, sink):
        o, lse = lib.combine(torch.from_numpy(o_part).to(DEV), torch.from_numpy(lse_part).to(DEV),
                             sink=None if s is None else torch.from_numpy(s).to(DEV))
        torch.cuda.synchronize()
        o_ref, l_ref = OA.combine(o_part.astype(np.float64), lse_part.astype(np.float64),
                                  sink=None if s is None else s.astype(np.float64))
        assert_decode_close(o, lse, o_ref, l_ref, "combine")


def test_combine_turns_a_nan_partial_lse_into_a_nan_row(lib):
    # a decode workgroup whose bounded wait ran out marks its partial with a
    # NaN LSE; the merge must not hide it behind the other splits' maxima
    rng = np.random.default_rng(5)
    p, r, h = 6, 5, 16
    o_part = rng.standard_normal((p, r, h, 512)).astype(np.float32)
    lse_part = (rng.standard_normal((p, r, h)) * 3).astype(np.float32)
    marked = [(0, 1, 3), (5, 4, 0), (2, 2, 15)]      # (split, row, head); split 5 is in the tail group
    for s, i, j in marked:
        lse_part[s, i, j] = np.nan
    lse_part[:, 3, 7] = -np.inf
    lse_part[4, 3, 7] = np.nan                      # NaN among empty partials
    o_part[np.isneginf(lse_part)] = 0
    o, lse = lib.combine(torch.from_numpy(o_part).to(DEV), torch.from_numpy(lse_part).to(DEV),
                         sink=torch.from_numpy(rng.standard_normal(h).astype(np.float32)).to(DEV))
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    bad = np.isnan(lse_part).any(axis=0)
    assert np.isnan(lse[bad]).all() and np.isnan(o[bad]).all()
    assert np.isfinite(o[~bad]).all() and not np.isnan(lse[~bad]).any()


def full_workload(lib, wl):
    """GPU pool filled by the HIP quantize-append from the workload latents;
    expected values from the oracle quantizing the same latents.  Every row
    is compared; O and LSE start as NaN, so a row the kernels never write
    fails."""
    rows = wl.batch * wl.s_q
    note(f"{wl.name}: rows={rows} h={wl.h_q} topk={wl.topk} "
         f"slots={wl.num_slots} filled={len(wl.slots)}")
    cache = lib.new_cache(wl.num_blocks, wl.block_size, DEV, record_bytes=wl.record_bytes)
    lib.quantize_append(wl.latent.to(DEV), wl.rope.to(DEV),
                        torch.from_numpy(wl.slots).to(DEV), cache)
    splits = lib.plan(wl.batch, wl.s_q, wl.h_q, wl.topk)
    o, lse = nan_outputs((wl.batch, wl.s_q, wl.h_q), DEV)
    lib.sparse_decode(wl.q.to(DEV), cache, torch.from_numpy(wl.indices).to(DEV),
                      wl.softmax_scale,
                      sink=None if wl.sink is None else torch.from_numpy(wl.sink).to(DEV),
                      num_splits=splits, out=o, lse=lse)
    torch.cuda.synchronize()
    o = o.reshape(rows, wl.h_q, 512).cpu()
    lse = lse.reshape(rows, wl.h_q).cpu()
    del cache
    torch.cuda.empty_cache()
    note(f"{wl.name}: decoded with {splits} splits; oracle over {len(wl.slots)} records")
    table = oracle_record_table(wl.latent, wl.rope, wl.record_bytes)
    note(f"{wl.name}: oracle records done; oracle decode of all {rows} rows")
    o_ref, l_ref = oracle_rows(wl, range(rows), table_lookup(wl, table))
    worst = assert_decode_close(o, lse, o_ref, l_ref, wl.name)
    note(f"{wl.name}: splits={splits}, worst error/bound over all {rows} rows = {worst:.3f}")


def test_tiny_workload_all_rows(lib):
    wl = W.tiny()
    full_workload(lib, wl)


@pytest.mark.parametrize("name", ["decode_h64", "decode_h128_varlen", "decode_h16_mtp",
                                  "decode_h64_ds_mla"])
def test_full_size_workloads_every_row(lib, name):
    wl = W.DECODE_WORKLOADS[name]()
    full_workload(lib, wl)


def test_workspace_reuse_and_garbage_workspace(lib):
    """The workspace needs no initialisation and keeps nothing between calls:
    one filled with garbage serves repeated decodes of a shape (both kernels),
    each giving the same bits."""
    for h in (16, 32):
        recs, q, idx, sink, nb, bs = small_case(17 + h, 3, 2, h, 600)
        cache = torch.from_numpy(recs.reshape(nb, bs, 352)).to(DEV)
        splits = 5
        need = lib.workspace_size(3, 2, h, 600, splits)
        ws = torch.full((need,), 0xC3, dtype=torch.uint8, device=DEV)
        qd, idd = q.to(DEV), torch.from_numpy(idx).to(DEV)
        sk = torch.from_numpy(sink).to(DEV)
        outs = []
        for _ in range(3):
            o, l = lib.sparse_decode(qd, cache, idd, 1.0 / 24, sink=sk, num_splits=splits,
                                     workspace=ws)
            torch.cuda.synchronize()
            outs.append((o.clone(), l.clone()))
        for o, l in outs[1:]:
            assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
        _, _, o_ref, l_ref = run_small(lib, recs, q, idx, sink, nb, bs, splits)
        assert_decode_close(outs[0][0], outs[0][1], o_ref, l_ref, f"reused workspace h{h}")


def crafted_code_scale_records(record_bytes, seed=5):
    """127 records that together hold every E2M1 code under every finite E4M3
    scale byte (0 and the subnormals included): record r gives block s the
    scale byte (r + 5s) mod 127 and element i the code (i + r) mod 16, so
    each block holds all 16 codes.  RoPE bytes are small finite values."""
    rng = np.random.default_rng(seed)
    n = 127
    rec = np.zeros((n, record_bytes), np.uint8)
    i = np.arange(512)
    for r in range(n):
        codes = (i + r) % 16
        rec[r, :256] = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
        rec[r, OC._scale_positions(record_bytes)] = (r + 5 * np.arange(32)) % 127
    if record_bytes == 352:
        # E4M3 bytes with exponent field <= 9: |value| < 8
        rec[:, 256:320] = (rng.integers(0, 80, (n, 64)) | (rng.integers(0, 2, (n, 64)) << 7)).astype(np.uint8)
    else:
        rope = rng.standard_normal((n, 64)).astype(np.float32)
        rec[:, 304:432] = (rope.view(np.uint32) >> 16).astype(np.uint16).view(np.uint8).reshape(n, 128)
    return rec


@pytest.mark.parametrize("h,splits,rb", [(16, 1, 352), (32, 1, 352), (64, 3, 352), (128, 1, 352),
                                         (16, 2, 432), (64, 1, 432)])
def test_single_valid_token_returns_every_code_scale_product_exactly(lib, h, splits, rb):
    # each row has one valid token among invalid ones, so its weight is 1 and
    # O is that record's dequantized NoPE row, bit for bit in bf16; the
    # records cover all 16 x 127 (code, scale) products
    note(f"code x scale through the decode h={h} splits={splits} record={rb}")
    recs = crafted_code_scale_records(rb)
    n = recs.shape[0]
    bs = 64
    nb = -(-n // bs)
    full = np.zeros((nb * bs, rb), np.uint8)
    full[:n] = recs
    rng = np.random.default_rng(h + splits)
    topk = 37
    idx = np.full((n, 1, topk), -1, np.int32)
    idx[np.arange(n), 0, rng.integers(0, topk, n)] = np.arange(n)
    q = torch.from_numpy(rng.standard_normal((n, 1, h, 576)).astype(np.float32)).to(torch.bfloat16)
    cache = torch.from_numpy(full.reshape(nb, bs, rb)).to(DEV)
    o, lse = lib.sparse_decode(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), 1.0 / 24,
                               num_splits=splits)
    torch.cuda.synchronize()
    v = torch.from_numpy(OC.dequantize_records(recs)[:, :512]).to(torch.bfloat16)
    assert torch.equal(o[:, 0].cpu(), v[:, None, :].expand(n, h, 512))
    o_ref, l_ref = OA.sparse_decode(f64(q), recs, idx, 1.0 / 24)
    assert_decode_close(o, lse, o_ref, l_ref, f"code x scale h={h}")


# Launches of at least four workgroups per CU (a prefill's many query rows)
# run the 32-head kernel with two pairs per workgroup, two workgroups per CU.
# These cases are large enough to take that path (>= 1024 workgroups on 256
# CUs) and small enough to check every row: odd chunk counts give the two
# pairs different numbers of chunks.
@pytest.mark.parametrize("b,h,topk,splits,p_inval", [
    (512, 64, 100, 1, 0.1), (256, 128, 77, 1, 0.3), (512, 32, 300, 2, 0.05), (1024, 32, 33, 1, 0.5),
])
def test_many_workgroups_every_row(lib, b, h, topk, splits, p_inval):
    note(f"many workgroups b={b} h={h} topk={topk} splits={splits}")
    recs, q, idx, sink, nb, bs = small_case(41 + h, b, 1, h, topk, nblocks=40, p_inval=p_inval, dup=True)
    idx[3, 0, :] = -1                       # an empty row
    o, lse, o_ref, l_ref = run_small(lib, recs, q, idx, sink, nb, bs, splits)
    assert_decode_close(o, lse, o_ref, l_ref, f"many workgroups h={h} splits={splits}")
    assert bool((o[3].cpu() == 0).all()) and bool(torch.isneginf(lse[3]).all())


@pytest.mark.parametrize("b,s_q,h,topk,splits", [
    (8, 2, 16, 100, 1), (16, 3, 48, 70, 2), (8, 4, 16, 33, 1),
    (8, 2, 64, 100, 3), (8, 3, 32, 70, 1), (512, 2, 32, 40, 1),
])
def test_sequences_of_several_rows_every_row(lib, b, s_q, h, topk, splits):
    # at least 8 sequences of several query rows: both kernels place
    # workgroups by sequence (the last case also takes the 32-head kernel's
    # two-pair shape)
    note(f"sequences b={b} s_q={s_q} h={h} topk={topk} splits={splits}")
    recs, q, idx, sink, nb, bs = small_case(57 + s_q, b, s_q, h, topk)
    o, lse, o_ref, l_ref = run_small(lib, recs, q, idx, sink, nb, bs, splits)
    assert_decode_close(o, lse, o_ref, l_ref, f"sequences s_q={s_q}")
