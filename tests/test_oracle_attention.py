"""Pins of the oracle's sparse decode, dual-cache decode and split-KV combine.

Pinned against: torch's scaled_dot_product_attention and logsumexp in float64
(dense attention over the whole pool is the special case top-k = pool with no
invalid index and no sink), closed forms (one token, zero query, sink
algebra, empty rows) and invariants (index order, inserted -1, duplicates,
splitting then combining).  The dual-cache decode is pinned by a dense
softmax with the sink as an extra zero-valued logit column, by combining the
two lists' separate decodes, by moving a token from one cache to the other,
and by its one-list special cases.
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import codec as C
from sparse_mla_decode_nvfp4_amd import workloads as W


@pytest.fixture(scope="module")
def tiny():
    wl = W.tiny()
    recs = C.quantize_records(wl.latent.to(torch.float64).numpy(),
                              wl.rope.to(torch.float64).numpy())
    q = wl.q.to(torch.float64).numpy()
    return wl, recs, q


def test_dense_special_case_matches_torch_sdpa(tiny):
    wl, recs, q = tiny
    n = recs.shape[0]
    idx = np.arange(n).reshape(1, 1, n)
    o, lse = A.sparse_decode(q, recs, idx, wl.softmax_scale)
    kv = torch.from_numpy(C.dequantize_records(recs))
    qt = torch.from_numpy(q[0, 0])[None, :, None, :]          # [1, H, 1, 576]
    k = kv[None, None].expand(1, qt.shape[1], n, 576)
    v = kv[None, None, :, :512].expand(1, qt.shape[1], n, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=wl.softmax_scale)
    assert np.allclose(o[0, 0], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    z = wl.softmax_scale * (qt[0, :, 0] @ kv.T)
    assert np.allclose(lse[0, 0], torch.logsumexp(z, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_single_token_returns_its_value_row(tiny):
    wl, recs, q = tiny
    idx = np.full((1, 1, 5), -1)
    idx[0, 0, 3] = 17
    o, lse = A.sparse_decode(q, recs, idx, wl.softmax_scale)
    kv = C.dequantize_records(recs)
    assert np.array_equal(o[0, 0], np.broadcast_to(kv[17, :512], (16, 512)))
    z = np.float64(np.float32(wl.softmax_scale)) * (q[0, 0] @ kv[17])
    assert np.allclose(lse[0, 0], z, atol=1e-12)


def test_zero_query_is_a_plain_mean_and_sink_algebra(tiny):
    wl, recs, _ = tiny
    q0 = np.zeros((1, 1, 16, 576))
    idx = np.array([[[3, 9, -1, 40, 41, 200]]])
    kv = C.dequantize_records(recs)
    mean = kv[[3, 9, 40, 41, 200], :512].mean(0)
    o, lse = A.sparse_decode(q0, recs, idx, wl.softmax_scale)
    assert np.allclose(o[0, 0], mean, atol=1e-12) and np.allclose(lse, np.log(5))
    sink = np.linspace(-2, 3, 16)
    o2, lse2 = A.sparse_decode(q0, recs, idx, wl.softmax_scale, sink=sink)
    assert np.allclose(o2[0, 0], mean[None] * (5 / (5 + np.exp(sink)))[:, None], atol=1e-12)
    assert np.allclose(lse2, np.log(5))                     # LSE excludes the sink
    o3, _ = A.sparse_decode(q0, recs, idx, wl.softmax_scale, sink=np.full(16, -np.inf))
    assert np.array_equal(o3, o)                            # sink -inf == no sink


def test_all_invalid_row_gives_zero_and_minus_inf(tiny):
    wl, recs, q = tiny
    idx = np.full((1, 1, 8), -1)
    o, lse = A.sparse_decode(q, recs, idx, wl.softmax_scale, sink=np.zeros(16))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_order_invalid_entries_and_duplicates(tiny):
    wl, recs, q = tiny
    idx = wl.slot_rows(wl.indices)                          # rows into recs
    o, lse = A.sparse_decode(q, recs, idx, wl.softmax_scale)
    rng = np.random.default_rng(0)
    perm = idx[:, :, rng.permutation(idx.shape[-1])]
    pad = np.concatenate([perm, np.full((1, 1, 7), -1)], axis=-1)[:, :, rng.permutation(71)]
    o2, lse2 = A.sparse_decode(q, recs, pad, wl.softmax_scale)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)
    # a duplicated index counts twice: same as weighting that token by 2
    dup = np.concatenate([idx, idx[:, :, :1]], axis=-1)
    o3, lse3 = A.sparse_decode(q, recs, dup, wl.softmax_scale)
    kv = C.dequantize_records(recs)
    t = idx[0, 0]
    z = np.float64(np.float32(wl.softmax_scale)) * (q[0, 0] @ kv[t].T)
    w = np.exp(z - z.max(1, keepdims=True))
    w[:, 0] *= 2
    ref = (w @ kv[t, :512]) / w.sum(1, keepdims=True)
    assert np.allclose(o3[0, 0], ref, atol=1e-12)
    assert np.allclose(lse3[0, 0], z.max(1) + np.log(w.sum(1)), atol=1e-12)


@pytest.mark.parametrize("parts", [1, 2, 3, 7])
def test_split_then_combine_equals_unsplit(tiny, parts):
    wl, recs, q = tiny
    idx = wl.slot_rows(wl.indices)
    idx[0, 0, 5] = -1
    sink = np.linspace(-1, 1, 16)
    o, lse = A.sparse_decode(q, recs, idx, wl.softmax_scale, sink=sink)
    bounds = np.linspace(0, idx.shape[-1], parts + 1).astype(int)
    po, pl = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        oi, li = A.partial_decode(q, recs, idx[:, :, a:b], wl.softmax_scale)
        po.append(oi)
        pl.append(li)
    # an extra empty split must not change anything
    po.append(np.zeros_like(po[0]))
    pl.append(np.full_like(pl[0], -np.inf))
    oc, lc = A.combine(np.stack(po), np.stack(pl), sink=sink)
    assert np.allclose(oc, o, atol=1e-12) and np.allclose(lc, lse, atol=1e-12)


def test_combine_of_nothing_is_empty():
    o, l = A.combine(np.zeros((3, 2, 4, 512)), np.full((3, 2, 4), -np.inf), sink=np.zeros(4))
    assert np.all(o == 0) and np.all(np.isneginf(l))


@pytest.fixture(scope="module")
def two_pools():
    """A primary pool of 40 and an extra pool of 30 records, quantized by the
    oracle from differently seeded latents, and two query rows of 16 heads."""
    lat0, rope0 = W.latents(0, 40, rep=7)
    lat1, rope1 = W.latents(0, 30, rep=7, pool=1)
    r0 = C.quantize_records(lat0.to(torch.float64).numpy(), rope0.to(torch.float64).numpy())
    r1 = C.quantize_records(lat1.to(torch.float64).numpy(), rope1.to(torch.float64).numpy())
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 2, 16, 576))
    i0 = np.array([[[3, 9, -1, 39, 0, 12, 3]], [[5, -1, -1, 1, 2, 30, 31]]]).reshape(1, 2, 7)
    i1 = np.array([[[29, -1, 0, 7, 8]], [[4, 4, 17, -1, 22]]]).reshape(1, 2, 5)
    sink = np.linspace(-2, 1.5, 16)
    return r0, r1, q, i0, i1, sink


def test_dual_matches_dense_softmax_with_sink_column(two_pools):
    r0, r1, q, i0, i1, sink = two_pools
    scale = float(np.float32(1.0 / 24.0))      # the decode's scale is a float32
    o, lse = A.sparse_decode_dual(q, r0, i0, r1, i1, scale, sink=sink)
    k0 = torch.from_numpy(C.dequantize_records(r0))
    k1 = torch.from_numpy(C.dequantize_records(r1))
    for s in range(2):
        keys = torch.cat([k0[[t for t in i0[0, s] if t >= 0]], k1[[t for t in i1[0, s] if t >= 0]]])
        z = scale * (torch.from_numpy(q[0, s]) @ keys.T)                   # [16, n]
        zs = torch.cat([z, torch.from_numpy(sink)[:, None]], dim=1)        # sink as a logit
        vals = torch.cat([keys[:, :512], torch.zeros(1, 512, dtype=torch.float64)])
        ref = torch.softmax(zs, dim=1) @ vals
        assert np.allclose(o[0, s], ref.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[0, s], torch.logsumexp(z, dim=1).numpy(), rtol=0, atol=1e-12)


def test_dual_is_the_combine_of_its_two_lists(two_pools):
    r0, r1, q, i0, i1, sink = two_pools
    o, lse = A.sparse_decode_dual(q, r0, i0, r1, i1, 0.07, sink=sink)
    oa, la = A.partial_decode(q, r0, i0, 0.07)
    ob, lb = A.partial_decode(q, r1, i1, 0.07)
    oc, lc = A.combine(np.stack([oa, ob]), np.stack([la, lb]), sink=sink)
    assert np.allclose(o, oc, atol=1e-12) and np.allclose(lse, lc, atol=1e-12)


def test_dual_token_moves_between_caches(two_pools):
    """A primary entry served from a copy of its record in the extra pool
    (and the reverse) gives the same result."""
    r0, r1, q, i0, i1, sink = two_pools
    o, lse = A.sparse_decode_dual(q, r0, i0, r1, i1, 0.05, sink=sink)
    # primary entry 39 of row 0 becomes extra row 30 (a copy of primary record 39)
    r1b = np.concatenate([r1, r0[39:40]])
    i0b, i1b = i0.copy(), i1.copy()
    i0b[0, 0, 3] = -1
    i1b[0, 0, 1] = 30
    ob, lb = A.sparse_decode_dual(q, r0, i0b, r1b, i1b, 0.05, sink=sink)
    assert np.allclose(o, ob, atol=1e-12) and np.allclose(lse, lb, atol=1e-12)


def test_dual_with_one_empty_list_is_the_plain_decode(two_pools):
    r0, r1, q, i0, i1, sink = two_pools
    none = np.zeros((1, 2, 0), dtype=np.int64)
    o, lse = A.sparse_decode_dual(q, r0, i0, r1, none, 0.05, sink=sink)
    o0, l0 = A.sparse_decode(q, r0, i0, 0.05, sink=sink)
    assert np.array_equal(o, o0) and np.array_equal(lse, l0)
    o, lse = A.sparse_decode_dual(q, r0, none, r1, i1, 0.05, sink=sink)
    o1, l1 = A.sparse_decode(q, r1, i1, 0.05, sink=sink)
    assert np.allclose(o, o1, atol=1e-14) and np.allclose(lse, l1, atol=1e-14)
    allinv = np.full((1, 2, 3), -1)
    o, lse = A.sparse_decode_dual(q, r0, allinv, r1, allinv, 0.05, sink=sink)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
