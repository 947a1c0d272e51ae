"""GPU parity of the 432-byte "nvfp4_ds_mla" record: the write path must give
the oracle's bytes exactly (codes, block-order scales, zero pad, verbatim bf16
RoPE) and leave unmapped slots untouched; the gather must return the oracle's
values bit for bit; the decode (both kernels, single and dual cache) must match
the fp64 oracle to |d| <= 1e-2 + 2e-2 |ref| in O and 1e-3 in LSE.
"""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import codec as OC
from oracle import formats as OF
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import assert_decode_close, f64, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
R = 432


def bf16_from_f64(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16)


def gpu_quantize_ds(lib, lat_b, rope_b, bs=64):
    n = lat_b.shape[0]
    nb = (n + bs - 1) // bs
    cache = lib.new_cache(nb, bs, DEV, fill=0xA5, record_bytes=R)
    sm = torch.arange(n, dtype=torch.int64, device=DEV)
    lib.quantize_append(lat_b.to(DEV), rope_b.to(DEV), sm, cache)
    torch.cuda.synchronize()
    return cache.view(-1, R)[:n].cpu().numpy()


def test_ds_mla_append_workload_is_byte_exact(lib):
    wl = W.append_write()
    n_slots = wl.num_blocks * wl.block_size
    note(f"append_write into 432-byte records: N={wl.num_tokens} slots={n_slots}")
    sentinel = np.random.default_rng(21).integers(0, 256, size=(n_slots, R), dtype=np.uint8)
    cache = torch.from_numpy(sentinel.reshape(wl.num_blocks, wl.block_size, R)).to(DEV)
    lib.quantize_append(wl.latent.to(DEV), wl.rope.to(DEV),
                        torch.from_numpy(wl.slot_mapping).to(DEV), cache)
    torch.cuda.synchronize()
    got = cache.view(-1, R).cpu().numpy()
    ref = OC.quantize_append(sentinel, f64(wl.latent), f64(wl.rope), wl.slot_mapping)
    diff = np.nonzero(np.any(got != ref, axis=1))[0]
    assert diff.size == 0, f"{diff.size} slots differ, first {diff[:5]}"


def test_ds_mla_every_bf16_amax_and_every_finite_rope(lib):
    """Every positive finite bf16 value as a block amax (its scale byte lands
    at 256 + block), and every finite bf16 value through the RoPE lane."""
    bits = torch.arange(1, 0x7F80, dtype=torch.int32).to(torch.int16)
    amax = bits.view(torch.bfloat16).to(torch.float64).numpy()
    n = len(amax)
    lat = np.zeros((n, 512))
    lat[:, 3] = amax
    lat[:, 100] = -amax * 0.6
    lat[:, 496:512] = np.linspace(-1, 1, 16)[None, :] * amax[:, None]
    allv = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    allv = allv[torch.isfinite(allv.to(torch.float32))]
    rope = torch.zeros(n * 64, dtype=torch.bfloat16)
    k = min(len(allv), n * 64)
    rope[:k] = allv[:k]
    rope = rope.reshape(n, 64)
    lat_b = bf16_from_f64(lat)
    got = gpu_quantize_ds(lib, lat_b, rope)
    ref = OC.quantize_records(f64(lat_b), f64(rope), R)
    bad = np.any(got != ref, axis=1)
    assert not bad.any(), f"{int(bad.sum())} records differ, first {np.nonzero(bad)[0][:3]}"
    assert np.all(got[:, 288:304] == 0)


def test_ds_mla_gather_bit_exact_on_arbitrary_records(lib):
    """Random NoPE and scale bytes (scales avoid the NaN code), arbitrary
    RoPE bits returned verbatim; negative and out-of-range slots give zero
    rows."""
    rng = np.random.default_rng(12)
    n = 4096
    recs = rng.integers(0, 256, size=(n, R), dtype=np.uint8)
    sc = recs[:, 256:288]
    sc[(sc & 0x7F) == 0x7F] ^= 1
    cache = torch.from_numpy(recs.reshape(n // 64, 64, R)).to(DEV)
    slots = np.arange(n, dtype=np.int32)
    rng.shuffle(slots)
    slots[::89] = -1
    slots[7] = n + 1
    out = lib.dequantize_gather(cache, torch.from_numpy(slots).to(DEV))
    got = out.view(torch.int16).cpu().numpy()
    ok = (slots >= 0) & (slots < n)
    nope = np.zeros((n, 512))
    nope[ok] = OC.dequantize_records(recs[slots[ok]])[:, :512]
    assert np.array_equal(got[:, :512], bf16_from_f64(nope).view(torch.int16).numpy())
    rope_bits = np.zeros((n, 128), dtype=np.uint8)
    rope_bits[ok] = recs[slots[ok], 304:432]
    assert np.array_equal(got[:, 512:].view(np.uint8), rope_bits)


def ds_case(seed, b, s_q, h, topk, nb, bs, p_inval=0.1):
    rng = np.random.default_rng(seed)
    n_slots = nb * bs
    lat, rope = W.latents(0, n_slots, rep=seed)
    recs = OC.quantize_records(f64(lat), f64(rope), R)
    q = torch.from_numpy(rng.standard_normal((b, s_q, h, 576)).astype(np.float32)).to(torch.bfloat16)
    idx = np.stack([rng.choice(n_slots, size=topk, replace=False) for _ in range(b * s_q)])
    idx = idx.reshape(b, s_q, topk).astype(np.int32)
    idx[rng.random(idx.shape) < p_inval] = -1
    sink = rng.standard_normal(h).astype(np.float32)
    return recs, q, idx, sink


@pytest.mark.parametrize("b,s_q,h,topk,bs,splits", [
    (2, 1, 16, 200, 64, 1), (1, 2, 16, 1000, 64, 3), (2, 1, 32, 100, 48, 1),
    (1, 1, 64, 640, 64, 0), (1, 1, 128, 333, 64, 4), (3, 1, 48, 17, 2, 2),
])
def test_ds_mla_decode_small_cases(lib, b, s_q, h, topk, bs, splits):
    what = f"432-byte decode b{b} s{s_q} h{h} k{topk} page {bs} sp{splits}"
    note(what)
    nb = -(-topk // bs) + 3
    recs, q, idx, sink = ds_case(b * 31 + topk + h, b, s_q, h, topk, nb, bs)
    cache = torch.from_numpy(recs.reshape(nb, bs, R)).to(DEV)
    o, lse = lib.sparse_decode(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), 1.0 / 24,
                               sink=torch.from_numpy(sink).to(DEV), num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.sparse_decode(f64(q), recs, idx, 1.0 / 24, sink=sink.astype(np.float64))
    assert_decode_close(o, lse, o_ref, l_ref, what)


@pytest.mark.parametrize("h", [16, 64])
def test_ds_mla_dual_cache_decode(lib, h):
    note(f"432-byte dual decode h={h}")
    rng = np.random.default_rng(70 + h)
    r0, q, i0, sink = ds_case(80 + h, 2, 1, h, 128, 4, 64)
    lat1, rope1 = W.latents(0, 400, rep=9, pool=1)
    r1 = OC.quantize_records(f64(lat1), f64(rope1), R)
    i1 = rng.integers(0, 400, size=(2, 1, 300)).astype(np.int32)
    i1[rng.random(i1.shape) < 0.05] = -1
    c0 = torch.from_numpy(r0.reshape(4, 64, R)).to(DEV)
    c1 = torch.from_numpy(r1.reshape(200, 2, R)).to(DEV)
    o, lse = lib.sparse_decode_dual(q.to(DEV), c0, torch.from_numpy(i0).to(DEV), c1,
                                    torch.from_numpy(i1).to(DEV), 1.0 / 24,
                                    sink=torch.from_numpy(sink).to(DEV), num_splits=0)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.sparse_decode_dual(f64(q), r0, i0, r1, i1, 1.0 / 24,
                                         sink=sink.astype(np.float64))
    assert_decode_close(o, lse, o_ref, l_ref, f"432-byte dual h{h}")


def test_ds_mla_many_workgroups_every_row(lib):
    # >= 1024 workgroups: the 32-head kernel's two-pair shape on 432-byte records
    note("ds_mla many workgroups")
    h, b, topk = 64, 512, 90
    rng = np.random.default_rng(77)
    n = 40 * 64
    lat, rope = W.latents(0, n, rep=77)
    recs = OC.quantize_records(f64(lat), f64(rope), 432)
    q = torch.from_numpy(rng.standard_normal((b, 1, h, 576)).astype(np.float32)).to(torch.bfloat16)
    idx = rng.integers(0, n, size=(b, 1, topk)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    sink = rng.standard_normal(h).astype(np.float32)
    cache = torch.from_numpy(recs.reshape(40, 64, 432)).to(DEV)
    o, lse = lib.sparse_decode(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), 1.0 / 24,
                               sink=torch.from_numpy(sink).to(DEV), num_splits=1)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.sparse_decode(f64(q), recs, idx, 1.0 / 24, sink=sink.astype(np.float64))
    assert_decode_close(o, lse, o_ref, l_ref, "ds_mla many workgroups")
