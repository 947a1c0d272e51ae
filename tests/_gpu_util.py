"""Shared helpers for the GPU parity tests (test infrastructure)."""

import sys
from concurrent.futures import ThreadPoolExecutor

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


# host threads for oracle work (numpy releases the GIL inside its array loops)
ORACLE_THREADS = 8


def oracle_rows(wl, rows, records_for_slots):
    """Oracle O, LSE for the listed query rows (flattened b*s_q + s), the rows
    spread over host threads.

    records_for_slots(slots) -> uint8 [len(slots), record_bytes] computed by
    the oracle.
    """
    b_ = wl.batch
    s_ = wl.s_q
    q = wl.q.reshape(b_ * s_, wl.h_q, 576)
    idx = wl.indices.reshape(b_ * s_, wl.topk)
    sink = None if wl.sink is None else wl.sink.astype(np.float64)

    def one(r):
        ids = idx[r].astype(np.int64)
        valid = ids[ids >= 0]
        uniq = np.unique(valid)
        recs = (records_for_slots(uniq) if len(uniq)
                else np.zeros((0, wl.record_bytes), np.uint8))
        local = np.where(ids >= 0, np.searchsorted(uniq, np.maximum(ids, 0)), -1)
        o, l = OA.sparse_decode(f64(q[r])[None, None], recs, local[None, None],
                                wl.softmax_scale, sink=sink)
        return o[0, 0], l[0, 0]

    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        res = list(ex.map(one, list(rows)))
    return np.stack([o for o, _ in res]), np.stack([l for _, l in res])


def oracle_record_table(latent, rope, record_bytes=352, chunk=8192):
    """The oracle's records for every row of latent/rope (bf16 tensors),
    quantized in chunks spread over host threads."""
    n = latent.shape[0]

    def part(i):
        return OC.quantize_records(f64(latent[i:i + chunk]), f64(rope[i:i + chunk]), record_bytes)

    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        parts = list(ex.map(part, range(0, n, chunk)))
    return np.concatenate(parts) if parts else np.zeros((0, record_bytes), np.uint8)


def table_lookup(wl, table):
    """records_for_slots() reading a workload's precomputed record table
    (one row per entry of wl.slots)."""
    return lambda slots: table[wl.slot_rows(slots)]


def nan_outputs(shape, device):
    """O (bf16) and LSE (fp32) filled with NaN, so rows a kernel never writes
    cannot pass as stale finite values."""
    o = torch.full((*shape, 512), float("nan"), dtype=torch.bfloat16, device=device)
    lse = torch.full(shape, float("nan"), dtype=torch.float32, device=device)
    return o, lse


GUARD = 4096
GUARD_BYTE = 0xA7


class Guarded:
    """A device buffer of `nbytes` between two GUARD-byte canary regions of
    GUARD_BYTE: a kernel writing past either end of the buffer shows up as
    a changed canary byte."""

    def __init__(self, nbytes, device, fill=None):
        self.nbytes = int(nbytes)
        self.buf = torch.full((GUARD + self.nbytes + GUARD,), GUARD_BYTE, dtype=torch.uint8,
                              device=device)
        self.inner = self.buf[GUARD:GUARD + self.nbytes]
        if fill is not None:
            self.inner.fill_(fill)

    def view(self, dtype, shape):
        return self.inner.view(dtype).view(shape)

    def check(self, what=""):
        head = self.buf[:GUARD].cpu().numpy()
        tail = self.buf[GUARD + self.nbytes:].cpu().numpy()
        bad_h = np.nonzero(head != GUARD_BYTE)[0]
        bad_t = np.nonzero(tail != GUARD_BYTE)[0]
        assert bad_h.size == 0, f"{what}: {bad_h.size} canary bytes before the buffer changed"
        assert bad_t.size == 0, (f"{what}: {bad_t.size} canary bytes after the buffer changed, "
                                 f"first at +{bad_t[0]}")


def padded_cache(records, block_size, pad_bytes, seed, device):
    """A paged cache [num_blocks, block_size, R] whose pages sit pad_bytes
    apart beyond block_size * R (block_stride_bytes = block_size * R +
    pad_bytes), built with as_strided over random backing bytes: the
    records of slot s = p * block_size + j at page p, offset j * R.
    Returns (cache view, backing tensor, the backing bytes as uploaded)."""
    n, r = records.shape
    nb = -(-n // block_size)
    stride = block_size * r + pad_bytes
    assert stride % 16 == 0
    rng = np.random.default_rng(seed)
    backing = rng.integers(0, 256, size=nb * stride, dtype=np.uint8)
    full = np.zeros((nb * block_size, r), np.uint8)
    full[:n] = records
    for p in range(nb):
        backing[p * stride:p * stride + block_size * r] = full[p * block_size:(p + 1) * block_size].reshape(-1)
    back = torch.from_numpy(backing.copy()).to(device)
    cache = torch.as_strided(back, (nb, block_size, r), (stride, r, 1))
    return cache, back, backing


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
