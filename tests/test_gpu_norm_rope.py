"""GPU parity of the fused write path (RMSNorm + rotary turn + bf16 rounding +
quantize-append in one pass) against the oracle (oracle/norm_rope.py).

  * The fp32 values before the bf16 rounding (the test export) equal the
    oracle's binary32 steps bit for bit: on the append_write latents with a
    random weight and positions (both pair layouts), and on a sweep of one
    nonzero element over every bf16 magnitude from 2^-40 to 2^40, which puts
    the square root and the division through about 10000 different inputs.
  * The records written over random sentinel bytes equal the oracle's bytes
    over the whole append_write cache (352- and 432-byte records, both pair
    layouts, slots -1 and positions outside the table skipped).
  * The fused records equal the plain quantize-append of the bf16
    intermediate: rounding the test export's values to bf16 and appending
    them gives the same cache bytes.
"""

import numpy as np
import pytest
import torch

from oracle import norm_rope as NR
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import f64, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gpu_f32(lib, lat, rope, nr, neox):
    out = lib.norm_rope_f32(lat.to(DEV), rope.to(DEV), nr.norm_weight.to(DEV), nr.eps,
                            nr.cos_sin.to(DEV), torch.from_numpy(nr.positions).to(DEV), neox=neox)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_f32(lat, rope, nr, neox):
    pos = nr.positions
    inside = (pos >= 0) & (pos < nr.cos_sin.shape[0])
    c, s = NR.table_rows(nr.cos_sin.numpy(), np.where(inside, pos, 0))
    y = NR.rms_norm_f32(f64(lat), f64(nr.norm_weight), nr.eps)
    k = NR.rotate_f32(f64(rope), c, s, neox)
    k[~inside] = np.nan
    return np.concatenate([y, k], axis=1)


def assert_bits_equal(got, ref, what):
    g = got.view(np.uint32)
    r = ref.astype(np.float32).view(np.uint32)
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN pattern differs"
    bad = (g != r) & ~nan_r
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} values differ, first at "
                           f"{np.argwhere(bad)[0]}")


@pytest.mark.parametrize("neox", [False, True])
def test_fp32_prologue_is_bit_exact_on_the_append_workload(lib, neox):
    note(f"fused prologue fp32, append_write latents, neox={neox}")
    wl = W.append_write()
    nr = W.norm_rope_inputs(wl.num_tokens, p_outside=0.01)
    got = gpu_f32(lib, wl.latent, wl.rope, nr, neox)
    assert_bits_equal(got, oracle_f32(wl.latent, wl.rope, nr, neox), "append_write prologue")


@pytest.mark.parametrize("eps", [0.0, 1e-6])
def test_fp32_norm_is_bit_exact_over_a_sweep_of_magnitudes(lib, eps):
    # one nonzero element a per token: the mean square is a^2 / 512, so the
    # square root and the division see every bf16 magnitude in the range
    bits = np.arange(0x2B80, 0x53C0, dtype=np.uint32)          # 2^-40 .. 2^40
    a = (bits << 16).view(np.float32)
    n = len(a)
    note(f"fused norm sweep over {n} magnitudes, eps={eps}")
    lat = np.zeros((n, 512), np.float32)
    lat[np.arange(n), np.arange(n) % 512] = a * np.where(np.arange(n) % 3 == 0, -1, 1)
    lat[np.arange(n), (np.arange(n) + 100) % 512] = a * 0.75         # a second element
    rng = np.random.default_rng(3)
    rope = rng.standard_normal((n, 64)).astype(np.float32)
    lat_b = torch.from_numpy(lat).to(torch.bfloat16)
    rope_b = torch.from_numpy(rope).to(torch.bfloat16)
    nr = W.norm_rope_inputs(n, rep=1, eps=eps)
    got = gpu_f32(lib, lat_b, rope_b, nr, False)
    assert_bits_equal(got, oracle_f32(lat_b, rope_b, nr, False), f"sweep eps={eps}")


@pytest.mark.parametrize("rb,neox", [(352, False), (352, True), (432, False)])
def test_fused_append_is_byte_exact_on_the_append_workload(lib, rb, neox):
    wl = W.append_write()
    nr = W.norm_rope_inputs(wl.num_tokens, p_outside=0.01)
    n_slots = wl.num_blocks * wl.block_size
    note(f"fused append_write R={rb} neox={neox}: {wl.num_tokens} tokens into {n_slots} slots")
    sentinel = (wl.sentinel if rb == 352 else
                np.random.default_rng(21).integers(0, 256, size=(n_slots, rb), dtype=np.uint8))
    cache = torch.from_numpy(sentinel.reshape(wl.num_blocks, wl.block_size, rb)).to(DEV)
    lib.norm_rope_quantize_append(wl.latent.to(DEV), wl.rope.to(DEV), nr.norm_weight.to(DEV),
                                  nr.eps, nr.cos_sin.to(DEV), torch.from_numpy(nr.positions).to(DEV),
                                  torch.from_numpy(wl.slot_mapping).to(DEV), cache, neox=neox)
    torch.cuda.synchronize()
    got = cache.view(-1, rb).cpu().numpy()
    ref = NR.fused_append(sentinel, f64(wl.latent), f64(wl.rope), f64(nr.norm_weight), nr.eps,
                          nr.cos_sin.numpy(), nr.positions, wl.slot_mapping, neox)
    diff = np.nonzero(np.any(got != ref, axis=1))[0]
    assert diff.size == 0, f"{diff.size} slots differ, first {diff[:5]}"


def test_fused_append_equals_the_plain_append_of_the_bf16_intermediate(lib):
    wl = W.append_write(num_tokens=4096, num_slots=8192)
    nr = W.norm_rope_inputs(wl.num_tokens, rep=2)
    note("fused append vs plain append of the rounded prologue")
    f32 = lib.norm_rope_f32(wl.latent.to(DEV), wl.rope.to(DEV), nr.norm_weight.to(DEV), nr.eps,
                            nr.cos_sin.to(DEV), torch.from_numpy(nr.positions).to(DEV))
    inter = f32.to(torch.bfloat16)                  # round to nearest even
    sm = torch.from_numpy(wl.slot_mapping).to(DEV)
    c1 = torch.from_numpy(wl.sentinel.reshape(wl.num_blocks, wl.block_size, 352)).to(DEV)
    c2 = c1.clone()
    lib.quantize_append(inter[:, :512].contiguous(), inter[:, 512:].contiguous(), sm, c1)
    lib.norm_rope_quantize_append(wl.latent.to(DEV), wl.rope.to(DEV), nr.norm_weight.to(DEV),
                                  nr.eps, nr.cos_sin.to(DEV), torch.from_numpy(nr.positions).to(DEV),
                                  sm, c2)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
