"""GPU parity of the write path and of the decode's dequantization.

The HIP quantize-append must produce the oracle's bytes exactly (every code,
every scale byte, every RoPE byte) and leave unmapped slots untouched; the
dequantize-gather export (the decode's own dequant routine) must return the
oracle's values bit for bit in bf16.
"""

import numpy as np
import pytest
import torch

from oracle import codec as OC
from oracle import formats as OF
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import f64, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bf16_from_f64(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16)


def gpu_quantize(lib, latent_bf16, rope_bf16, num_slots=None, bs=64, sentinel=None):
    """Quantize-append of bf16 (or fp16) rows to slots 0..N-1 on the GPU."""
    n = latent_bf16.shape[0]
    if num_slots is None:
        num_slots = ((n + bs - 1) // bs) * bs
    nb = num_slots // bs
    if sentinel is None:
        cache = lib.new_cache(nb, bs, DEV)
    else:
        cache = torch.from_numpy(sentinel.reshape(nb, bs, 352)).to(DEV)
    sm = torch.arange(n, dtype=torch.int64, device=DEV)
    lib.quantize_append(latent_bf16.to(DEV), rope_bf16.to(DEV), sm, cache)
    torch.cuda.synchronize()
    return cache.view(-1, 352)[:n].cpu().numpy()


def test_append_workload_is_byte_exact_and_leaves_unmapped_slots(lib):
    wl = W.append_write()
    note(f"append_write: N={wl.num_tokens} slots={wl.num_blocks * wl.block_size}")
    cache = torch.from_numpy(wl.sentinel.reshape(wl.num_blocks, wl.block_size, 352)).to(DEV)
    lib.quantize_append(wl.latent.to(DEV), wl.rope.to(DEV),
                        torch.from_numpy(wl.slot_mapping).to(DEV), cache)
    torch.cuda.synchronize()
    got = cache.view(-1, 352).cpu().numpy()
    ref = OC.quantize_append(wl.sentinel, f64(wl.latent), f64(wl.rope), wl.slot_mapping)
    diff = np.nonzero(np.any(got != ref, axis=1))[0]
    assert diff.size == 0, f"{diff.size} slots differ, first {diff[:5]}"


def test_every_bf16_amax_gives_the_oracle_scale(lib):
    """All positive finite bf16 values as a block amax (block 0), the other
    elements of the block spread below it."""
    bits = torch.arange(1, 0x7F80, dtype=torch.int32).to(torch.int16)
    amax = bits.view(torch.bfloat16).to(torch.float64).numpy()
    n = len(amax)
    lat = np.zeros((n, 512))
    lat[:, 3] = amax
    lat[:, 4] = -amax * 0.3
    lat[:, 7] = amax * 0.74
    lat[:, 16:32] = -np.linspace(0, 1, 16)[None, :] * amax[:, None]
    lat_b = bf16_from_f64(lat)
    rope_b = bf16_from_f64(np.zeros((n, 64)))
    got = gpu_quantize(lib, lat_b, rope_b)
    ref = OC.quantize_records(f64(lat_b), f64(rope_b))
    assert np.array_equal(got, ref), f"{int(np.any(got != ref, axis=1).sum())} records differ"


def test_every_code_under_every_scale(lib):
    """For each E4M3 scale code S (amax = 6*value(S) exactly), every bf16 x
    with |x| <= amax in the other lanes of the block."""
    allb = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    pos = allb.to(torch.float64).numpy()
    rows = []
    for s in range(1, 0x7F):
        sv = OF.e4m3_decode(s)
        amax = 6.0 * sv
        xs = pos[pos <= amax]
        xs = np.concatenate([xs, -xs])
        per = 15
        ng = (len(xs) + per - 1) // per
        blk = np.zeros((ng, 16))
        flat = np.zeros(ng * per)
        flat[:len(xs)] = xs
        blk[:, :15] = flat.reshape(ng, per)
        blk[:, 15] = amax
        rows.append(blk)
    blocks = np.concatenate(rows)
    nt = (len(blocks) + 31) // 32
    pad = np.zeros((nt * 32 - len(blocks), 16))
    lat = np.concatenate([blocks, pad]).reshape(nt, 512)
    note(f"code sweep: {len(blocks)} blocks in {nt} tokens")
    lat_b = bf16_from_f64(lat)
    rope_b = bf16_from_f64(np.zeros((nt, 64)))
    got = gpu_quantize(lib, lat_b, rope_b)
    ref = OC.quantize_records(f64(lat_b), f64(rope_b))
    bad = np.any(got != ref, axis=1)
    assert not bad.any(), f"{int(bad.sum())} records differ, first token {np.nonzero(bad)[0][:3]}"


def test_every_finite_bf16_as_rope(lib):
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    v = bits.view(torch.bfloat16)
    v = v[torch.isfinite(v.to(torch.float32))]
    n = (len(v) + 63) // 64
    rope = torch.zeros(n * 64, dtype=torch.bfloat16)
    rope[:len(v)] = v
    rope = rope.reshape(n, 64)
    lat_b = torch.zeros((n, 512), dtype=torch.bfloat16)
    got = gpu_quantize(lib, lat_b, rope)
    ref = OC.quantize_records(f64(lat_b), f64(rope))
    assert np.array_equal(got[:, 256:320], ref[:, 256:320])
    assert np.array_equal(got, ref)


def test_edge_groups(lib):
    """Ties at every E2M1 midpoint, zero and signed-zero blocks, saturation,
    sub-normal scales, maximum-magnitude values."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows = []
    for s in [1, 2, 7, 8, 9, 0x30, 0x38, 0x3B, 0x55, 0x7D, 0x7E]:
        sv = OF.e4m3_decode(s)
        blk = np.zeros(16)
        blk[15] = 6 * sv
        for i, mdl in enumerate(mids):
            blk[i] = mdl * sv
            blk[7 + i] = -mdl * sv
        rows.append(blk)
    rows.append(np.zeros(16))
    rows.append(-np.zeros(16))
    rows.append(np.full(16, 3e38))              # saturated scale, codes 7
    rows.append(np.full(16, -1e5))
    rows.append(np.array([1e-30] * 8 + [-1e-30] * 8))   # amax/6 rounds to scale 0
    rows.append(np.linspace(-2688, 2688, 16))
    blocks = np.stack(rows)
    nt = (len(blocks) + 31) // 32
    lat = np.zeros((nt * 32, 16))
    lat[:len(blocks)] = blocks
    lat = lat.reshape(nt, 512)
    lat_b = bf16_from_f64(lat)
    rope_b = bf16_from_f64(np.tile(np.array([0.0, -0.0, 448, -448, 464, 1e4, -1e4, 2.0 ** -10]),
                                   (nt, 8)))
    got = gpu_quantize(lib, lat_b, rope_b)
    ref = OC.quantize_records(f64(lat_b), f64(rope_b))
    assert np.array_equal(got, ref)


def test_padded_pages_and_odd_block_size(lib):
    """Non-power-of-two page size and a padded page stride: records land at
    page*stride + offset*352 and nothing else changes."""
    bs, nb, pad = 48, 7, 16 * 5
    stride = bs * 352 + pad
    backing = torch.randint(0, 256, (nb * stride,), dtype=torch.uint8, device=DEV)
    before = backing.clone()
    cache = torch.as_strided(backing, (nb, bs, 352), (stride, 352, 1))
    lat, rope = W.latents(0, 40)
    sm = np.full(40, -1, dtype=np.int64)
    sm[:10] = [0, 47, 48, 49, 300, 100, -1, 200, 7 * 48 - 1, 150]   # distinct slots
    lib.quantize_append(lat.to(DEV), rope.to(DEV), torch.from_numpy(sm).to(DEV), cache)
    torch.cuda.synchronize()
    ref_rec = OC.quantize_records(f64(lat[:10]), f64(rope[:10]))
    after = backing.cpu().numpy()
    exp = before.cpu().numpy().copy()
    for i in range(10):
        s = int(sm[i])
        if s < 0:
            continue
        off = (s // bs) * stride + (s % bs) * 352
        exp[off:off + 352] = ref_rec[i]
    assert np.array_equal(after, exp)
    # the gather reads back through the same addressing
    slots = torch.from_numpy(sm[:10].astype(np.int32)).to(DEV)
    deq = lib.dequantize_gather(cache, slots)
    ref = OC.dequantize_records(ref_rec)
    ref[sm[:10] < 0] = 0.0
    assert np.array_equal(deq.view(torch.int16).cpu().numpy(),
                          bf16_from_f64(ref).view(torch.int16).numpy())


def test_dequantize_gather_bit_exact_on_arbitrary_records(lib):
    """Random record bytes (scale and RoPE bytes avoid the NaN code): every
    (code, scale) pair, signs and zeros; negative and out-of-range slots give
    zero rows."""
    rng = np.random.default_rng(11)
    n = 4096
    recs = rng.integers(0, 256, size=(n, 352), dtype=np.uint8)
    tail = recs[:, 256:]
    tail[(tail & 0x7F) == 0x7F] ^= 1
    recs[:, 320:352] &= 0x7F | (rng.integers(0, 2, size=(n, 32), dtype=np.uint8) << 7)
    recs[:, 320:352][(recs[:, 320:352] & 0x7F) == 0x7F] ^= 1
    cache = torch.from_numpy(recs.reshape(n // 64, 64, 352)).to(DEV)
    slots = np.arange(n, dtype=np.int32)
    rng.shuffle(slots)
    slots[::97] = -1
    slots[5] = n + 3
    out = lib.dequantize_gather(cache, torch.from_numpy(slots).to(DEV))
    got = out.view(torch.int16).cpu().numpy()
    ok = (slots >= 0) & (slots < n)
    ref_vals = np.zeros((n, 576))
    ref_vals[ok] = OC.dequantize_records(recs[slots[ok]])
    ref = bf16_from_f64(ref_vals).view(torch.int16).numpy()
    assert np.array_equal(got, ref)


def test_zero_tokens_is_a_no_op(lib):
    cache = lib.new_cache(2, 64, DEV, fill=7)
    lib.quantize_append(torch.zeros((0, 512), dtype=torch.bfloat16, device=DEV),
                        torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV),
                        torch.zeros((0,), dtype=torch.int64, device=DEV), cache)
    torch.cuda.synchronize()
    assert bool((cache == 7).all())


# ---- fp16 input (the write kernel's other 16-bit input type)

def fp16_from_f64(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float16)


def test_fp16_every_amax_gives_the_oracle_scale(lib):
    """All positive finite fp16 values as a block amax, through the fp16
    export, with companions below it in the block."""
    bits = torch.arange(1, 0x7C00, dtype=torch.int32).to(torch.int16)
    amax = bits.view(torch.float16).to(torch.float64).numpy()
    n = len(amax)
    lat = np.zeros((n, 512))
    lat[:, 3] = amax
    lat[:, 4] = -amax * 0.3
    lat[:, 7] = amax * 0.74
    lat[:, 16:32] = -np.linspace(0, 1, 16)[None, :] * amax[:, None]
    lat_h = fp16_from_f64(lat)
    rope_h = fp16_from_f64(np.zeros((n, 64)))
    got = gpu_quantize(lib, lat_h, rope_h)
    ref = OC.quantize_records(f64(lat_h), f64(rope_h))
    assert np.array_equal(got, ref), f"{int(np.any(got != ref, axis=1).sum())} records differ"


def test_fp16_every_code_under_every_scale(lib):
    """For each E4M3 scale code S (amax = 6*value(S), exact in fp16 where it
    fits), every fp16 x with |x| <= amax in the other lanes of the block."""
    pos = torch.arange(0, 0x7C00, dtype=torch.int32).to(torch.int16).view(torch.float16)
    pos = pos.to(torch.float64).numpy()
    rows = []
    for s in range(1, 0x7F):
        amax = 6.0 * OF.e4m3_decode(s)
        xs = pos[pos <= amax]
        xs = np.concatenate([xs, -xs])
        per = 15
        ng = (len(xs) + per - 1) // per
        blk = np.zeros((ng, 16))
        flat = np.zeros(ng * per)
        flat[:len(xs)] = xs
        blk[:, :15] = flat.reshape(ng, per)
        blk[:, 15] = amax
        rows.append(blk)
    blocks = np.concatenate(rows)
    nt = (len(blocks) + 31) // 32
    pad = np.zeros((nt * 32 - len(blocks), 16))
    lat = np.concatenate([blocks, pad]).reshape(nt, 512)
    note(f"fp16 code sweep: {len(blocks)} blocks in {nt} tokens")
    lat_h = fp16_from_f64(lat)
    rope_h = fp16_from_f64(np.zeros((nt, 64)))
    got = gpu_quantize(lib, lat_h, rope_h)
    ref = OC.quantize_records(f64(lat_h), f64(rope_h))
    bad = np.any(got != ref, axis=1)
    assert not bad.any(), f"{int(bad.sum())} records differ, first token {np.nonzero(bad)[0][:3]}"


def test_fp16_every_finite_value_as_rope(lib):
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    v = bits.view(torch.float16)
    v = v[torch.isfinite(v.to(torch.float32))]
    n = (len(v) + 63) // 64
    rope = torch.zeros(n * 64, dtype=torch.float16)
    rope[:len(v)] = v
    rope = rope.reshape(n, 64)
    lat_h = torch.zeros((n, 512), dtype=torch.float16)
    got = gpu_quantize(lib, lat_h, rope)
    ref = OC.quantize_records(f64(lat_h), f64(rope))
    assert np.array_equal(got, ref)


def test_fp16_workload_over_sentinel_bytes(lib):
    """Seeded fp16 latents (the append workload's recipe, cast to fp16, plus
    values beyond bf16 precision and near the fp16 range) scattered into a
    sentinel cache through a slot map with -1 entries."""
    wl = W.append_write(num_tokens=2048, num_slots=8192)
    g = np.random.default_rng([3, 9, 0])
    lat = wl.latent.to(torch.float64).numpy() * (1 + g.uniform(-1e-3, 1e-3, size=(2048, 512)))
    lat[::97] = np.clip(lat[::97] * 3000.0, -65000.0, 65000.0)   # rows near the fp16 range top
    rope = wl.rope.to(torch.float64).numpy()
    lat_h, rope_h = fp16_from_f64(lat), fp16_from_f64(rope)
    cache = torch.from_numpy(wl.sentinel.reshape(wl.num_blocks, wl.block_size, 352)).to(DEV)
    lib.quantize_append(lat_h.to(DEV), rope_h.to(DEV), torch.from_numpy(wl.slot_mapping).to(DEV), cache)
    torch.cuda.synchronize()
    got = cache.view(-1, 352).cpu().numpy()
    ref = OC.quantize_append(wl.sentinel, f64(lat_h), f64(rope_h), wl.slot_mapping)
    diff = np.nonzero(np.any(got != ref, axis=1))[0]
    assert diff.size == 0, f"{diff.size} slots differ, first {diff[:5]}"
