"""Pins of the oracle's sparse decode and split-KV combine.

Pinned against: torch's scaled_dot_product_attention and logsumexp in float64
(dense attention over the whole pool is the special case top-k = pool with no
invalid index and no sink), closed forms (one token, zero query, sink
algebra, empty rows) and invariants (index order, inserted -1, duplicates,
splitting then combining).
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
