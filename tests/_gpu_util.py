"""Shared helpers for the GPU parity tests (test infrastructure)."""

import sys

import numpy as np
import torch

from oracle import attention as OA
from oracle import codec as OC

O_ATOL = 1e-2
O_RTOL = 2e-2
LSE_ATOL = 1e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.to(torch.float64).cpu().numpy()


def upload_records(kv_cache, slots, records):
    """Write oracle records at the given slots of a [blocks, bs, 352] GPU cache."""
    flat = kv_cache.view(-1, 352) if kv_cache.is_contiguous() else None
    assert flat is not None
    idx = torch.from_numpy(np.asarray(slots, dtype=np.int64)).to(kv_cache.device)
    flat[idx] = torch.from_numpy(np.ascontiguousarray(records)).to(kv_cache.device)


def oracle_rows(wl, rows, records_for_slots):
    """Oracle O, LSE for the listed query rows (flattened b*s_q + s).

    records_for_slots(slots) -> uint8 [len(slots), 352] computed by the oracle.
    """
    b_ = wl.batch
    s_ = wl.s_q
    out_o, out_l = [], []
    q = wl.q.reshape(b_ * s_, wl.h_q, 576)
    idx = wl.indices.reshape(b_ * s_, wl.topk)
    for r in rows:
        ids = idx[r].astype(np.int64)
        valid = ids[ids >= 0]
        uniq = np.unique(valid)
        recs = records_for_slots(uniq) if len(uniq) else np.zeros((0, 352), np.uint8)
        local = np.where(ids >= 0, np.searchsorted(uniq, np.maximum(ids, 0)), -1)
        o, l = OA.sparse_decode(f64(q[r])[None, None], recs, local[None, None],
                                wl.softmax_scale, sink=None if wl.sink is None
                                else wl.sink.astype(np.float64))
        out_o.append(o[0, 0])
        out_l.append(l[0, 0])
    return np.stack(out_o), np.stack(out_l)


def oracle_records_from_workload(wl):
    """records_for_slots() quantizing the workload's own latents with the oracle."""
    lat = wl.latent
    rope = wl.rope

    def fn(slots):
        rows = wl.slot_rows(slots)
        return OC.quantize_records(f64(lat[rows]), f64(rope[rows]), wl.record_bytes)
    return fn


def assert_decode_close(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    o = o_gpu.to(torch.float64).cpu().numpy() if torch.is_tensor(o_gpu) else o_gpu
    lse = lse_gpu.to(torch.float64).cpu().numpy() if torch.is_tensor(lse_gpu) else lse_gpu
    err = np.abs(o - o_ref)
    bound = O_ATOL + O_RTOL * np.abs(o_ref)
    bad = err > bound
    assert not np.any(np.isnan(o)), f"{what}: NaN in O"
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} O elements out of "
                           f"tolerance; worst ratio {(err / bound).max():.3f}")
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), inf_ref), f"{what}: -inf LSE pattern differs"
    fin = ~inf_ref
    if fin.any():
        lerr = np.abs(lse[fin] - lse_ref[fin]).max()
        assert lerr <= LSE_ATOL, f"{what}: LSE max error {lerr:.2e}"
    return float((err / bound).max()) if err.size else 0.0
