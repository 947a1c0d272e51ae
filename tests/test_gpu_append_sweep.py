"""A seeded random sweep of the write path against the oracle, byte for byte.

Each case draws, from one fixed seed: the entry point (bf16 or fp16 input
into 352-byte records, bf16 into 432-byte records, or the fused norm +
rotary path into either, with either pair layout), a token count that is
rarely a multiple of a workgroup's tokens, row strides wider than the rows,
a page size (1 to 256 tokens) with or without padding between pages, slot
ids that are distinct and scattered with a fraction -1 and a few at or past
the cache's end (skipped), input magnitudes from tiny (subnormal scales) to
huge (saturated scales), and for the fused path positions partly outside
the table.  The cache is a view over random backing bytes: every written
record must equal the oracle's bytes and every other byte, page padding
included, must be unchanged.
"""

import numpy as np
import pytest
import torch

from oracle import codec as OC
from oracle import norm_rope as NR
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import f64, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KINDS = ["bf16", "fp16", "bf16_432", "fused", "fused_432"]
PAGES = [1, 3, 16, 48, 64, 256]
PADS = [0, 0, 16, 208]
MAGNITUDES = [1.0, 1.0, 1.0, 2.0 ** -12, 2.0 ** 9]


def draw_cases(n_cases=40, seed=77123):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        kind = str(rng.choice(KINDS))
        n = int(np.exp(rng.uniform(0, np.log(3000))))
        cases.append(dict(
            i=i, kind=kind, n=n, bs=int(rng.choice(PAGES)), pad=int(rng.choice(PADS)),
            lextra=8 * int(rng.integers(0, 5)), rextra=int(rng.integers(0, 9)),
            p_skip=float(rng.choice([0.0, 0.1, 0.5])), oob=bool(rng.random() < 0.3),
            mag=float(rng.choice(MAGNITUDES)), neox=bool(rng.random() < 0.5),
            seed=int(rng.integers(1 << 30))))
    return cases


CASES = draw_cases()


def strided_rows(x, extra, dtype):
    """x [n, d] as rows of a wider [n, d + extra] tensor (row stride d + extra)."""
    n, d = x.shape
    wide = torch.zeros((n, d + extra), dtype=dtype)
    wide[:, :d] = x.to(dtype)
    return wide.to(DEV)[:, :d]


@pytest.mark.parametrize("case", CASES, ids=[f"a{c['i']}" for c in CASES])
def test_random_append_is_byte_exact(lib, case):
    c = case
    rb = 432 if c["kind"].endswith("432") else 352
    fused = c["kind"].startswith("fused")
    what = (f"append sweep a{c['i']}: {c['kind']} N={c['n']} pages {c['bs']}+{c['pad']} "
            f"strides +{c['lextra']}/+{c['rextra']} skip{c['p_skip']} oob{c['oob']} mag{c['mag']} "
            f"neox{c['neox']}")
    note(what)
    rng = np.random.default_rng(c["seed"])
    n, bs, pad = c["n"], c["bs"], c["pad"]
    # the token latents, scaled by a power of two (exact in bf16 and fp16;
    # fp16 inputs are not scaled up, which could overflow its range)
    dtype = torch.float16 if c["kind"] == "fp16" else torch.bfloat16
    mag = min(c["mag"], 1.0) if dtype == torch.float16 else c["mag"]
    lat, rope = W.latents(3, n, rep=c["seed"] % 1000)
    lat = (lat.to(torch.float64) * mag).to(torch.bfloat16)
    rope = (rope.to(torch.float64) * mag).to(torch.bfloat16)
    if dtype == torch.float16:
        lat, rope = lat.to(torch.float16), rope.to(torch.float16)

    # paged cache over random backing bytes; distinct slots, some skipped
    nb = -(-(n + 5) // bs) + 2
    num_slots = nb * bs
    stride = bs * rb + pad
    backing = rng.integers(0, 256, size=nb * stride, dtype=np.uint8)
    back = torch.from_numpy(backing.copy()).to(DEV)
    cache = torch.as_strided(back, (nb, bs, rb), (stride, rb, 1))
    slots = rng.permutation(num_slots)[:n].astype(np.int64)
    slots[rng.random(n) < c["p_skip"]] = -1
    if c["oob"]:
        sel = rng.random(n) < 0.05
        slots[sel] = num_slots + rng.integers(0, 100, size=int(sel.sum()))
    sm = torch.from_numpy(slots).to(DEV)
    slots_ref = np.where(slots >= num_slots, -1, slots)

    # the logical records [num_slots, rb] the backing holds before the call
    def logical(bytes_):
        pages = bytes_.reshape(nb, stride)[:, :bs * rb]
        return pages.reshape(num_slots, rb)

    sentinel = logical(backing).copy()
    lat_d = strided_rows(lat, c["lextra"], dtype)
    rope_d = strided_rows(rope, c["rextra"], dtype)
    if fused:
        nr = W.norm_rope_inputs(n, rep=c["seed"] % 97, max_position=4096, p_outside=0.05)
        lib.norm_rope_quantize_append(lat_d, rope_d, nr.norm_weight.to(DEV), nr.eps,
                                      nr.cos_sin.to(DEV), torch.from_numpy(nr.positions).to(DEV),
                                      sm, cache, neox=c["neox"])
        ref = NR.fused_append(sentinel, f64(lat), f64(rope), f64(nr.norm_weight), nr.eps,
                              nr.cos_sin.numpy(), nr.positions, slots_ref, c["neox"])
    else:
        lib.quantize_append(lat_d, rope_d, sm, cache)
        ref = OC.quantize_append(sentinel, f64(lat), f64(rope), slots_ref)
    torch.cuda.synchronize()
    after = back.cpu().numpy()
    expect = backing.copy()
    exp_pages = expect.reshape(nb, stride)
    exp_pages[:, :bs * rb] = ref.reshape(nb, bs * rb)
    bad = np.nonzero(after != expect)[0]
    assert bad.size == 0, (f"{what}: {bad.size} bytes differ, first at byte {bad[0]} "
                           f"(page {bad[0] // stride}, offset {bad[0] % stride})")
