"""Pins of the oracle's element encodings and record layout.

Each check compares the oracle with something other than itself: the facts
the pages print (tests/golden/record_layout.txt), torch's float8_e4m3fn
conversions (a library routine), literal tables written from the format
definitions, and exact rational brute force.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "record_layout.txt")
GOLDEN_DS = os.path.join(os.path.dirname(__file__), "golden", "record_layout_ds_mla.txt")


def golden(path=GOLDEN):
    out = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (t.strip() for t in line.split("=", 1))
            out[k] = v
    return out


def test_record_layout_matches_pages():
    g = golden()
    assert int(g["d_qk"]) == F.QK_DIM
    assert int(g["d_v"]) == F.V_DIM
    assert int(g["record_bytes"]) == F.RECORD_BYTES
    assert [int(t) for t in g["nope_region"].split()] == [F.NOPE_OFFSET, F.NOPE_OFFSET + F.NOPE_BYTES]
    assert int(g["nope_values"]) == F.NOPE_DIM
    assert int(g["nope_values"]) // int(g["nope_values_per_byte"]) == F.NOPE_BYTES
    assert [int(t) for t in g["rope_region"].split()] == [F.ROPE_OFFSET, F.ROPE_OFFSET + F.ROPE_DIM]
    assert int(g["rope_values"]) == F.ROPE_DIM
    assert [int(t) for t in g["scale_region"].split()] == [F.SCALE_OFFSET, F.RECORD_BYTES]
    assert int(g["scale_count"]) == F.N_GROUPS
    assert int(g["scale_group_elements"]) == F.GROUP
    # the capacity figures the page prints follow from the sizes
    ratio = int(g["fp8_record_bytes"]) / F.RECORD_BYTES
    assert round(ratio, 1) == float(g["capacity_ratio_vs_fp8"])
    bits = F.RECORD_BYTES * 8 / F.QK_DIM
    assert round(bits, 2) == float(g["effective_bits_per_value"])


def test_scale_permutation_is_the_pages_transpose():
    g = golden()
    assert g["scale_byte_formula"] == "8*(s&3)+(s>>2)"
    s = np.arange(32)
    pos = F.scale_byte_position(s)
    assert sorted(pos.tolist()) == list(range(32))                 # bijection
    # inverse of the 8x4 -> 4x8 transpose: byte j holds block 4*(j&7) + (j>>3)
    for j in range(32):
        assert pos[4 * (j & 7) + (j >> 3)] == j
    # for a fixed q the blocks {4c+q : c = 0..7} fill 8 contiguous bytes, in c order
    for q in range(4):
        blocks = [4 * c + q for c in range(int(g["thread_blocks_per_q"]))]
        assert F.scale_byte_position(np.array(blocks)).tolist() == list(range(8 * q, 8 * q + 8))


def test_e2m1_decode_table():
    # OCP E2M1 value table written out from the format definition
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = F.e2m1_decode(np.arange(16))
    assert got[:8].tolist() == expect
    assert got[8:].tolist() == [-v for v in expect]
    assert np.signbit(got[8])                                      # code 8 is -0.0
    assert got.max() == float(golden()["e2m1_max"])


def test_e4m3_decode_matches_torch_all_256():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert F.E4M3_GRID[-1] == 448.0 and F.E4M3_GRID[1] == 2.0 ** -9


def all_finite_bf16():
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    v = bits.view(torch.bfloat16).to(torch.float64)
    return v[torch.isfinite(v)].numpy()


def test_e4m3_encode_matches_torch_rne_on_every_bf16():
    x = all_finite_bf16()
    got = F.e4m3_encode_satfinite(x)
    inrange = np.abs(x) < 464.0          # torch's RNE overflows to NaN at 464+
    ref = torch.from_numpy(x[inrange]).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[inrange], ref)
    # beyond: saturates to the largest finite value, sign kept
    big = x[~inrange]
    assert np.all(got[~inrange] == np.where(np.signbit(big), 0xFE, 0x7E))
    assert F.e4m3_encode_satfinite(np.array([-0.0]))[0] == 0x80
    assert not np.any((got & 0x7F) == 0x7F)


def brute_nearest(a, step, grid):
    """Exact rational nearest-code search, ties to the even code."""
    a = Fraction(a)
    step = Fraction(step)
    if step == 0:
        return 0
    d = [abs(a - step * Fraction(g)) for g in grid]
    best = min(d)
    c = [k for k in range(len(grid)) if d[k] == best]
    if len(c) == 1:
        return c[0]
    return [k for k in c if k % 2 == 0][0]


def test_nearest_code_against_rational_brute_force():
    rng = np.random.default_rng(7)
    bf = all_finite_bf16()
    bf = bf[bf >= 0]
    scales = F.E4M3_GRID
    a = rng.choice(bf[(bf < 5000)], 3000)
    st = rng.choice(scales, 3000)
    got = F.nearest_code(a, st, F.E2M1_GRID)
    for i in range(3000):
        assert got[i] == brute_nearest(a[i], st[i], F.E2M1_GRID), (a[i], st[i])
    # scale grid: every bf16 amax up to well past saturation
    amax = bf[bf < 4000][::7]
    got = F.nearest_code(amax, 6.0, F.E4M3_GRID)
    for i in range(len(amax)):
        assert got[i] == brute_nearest(amax[i], 6, F.E4M3_GRID), amax[i]


def test_e2m1_ties_go_to_even_codes():
    # quotient -> expected code at each midpoint of the E2M1 grid
    table = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for sv in [2.0 ** -9, 0.875, 1.0, 1.5, 448.0, 13.0 / 8]:
        for r, code in table.items():
            assert F.nearest_code(np.array([r * sv]), sv, F.E2M1_GRID)[0] == code
    # above 6 saturates; exactly 6 is code 7
    assert F.nearest_code(np.array([7.0]), 1.0, F.E2M1_GRID)[0] == 7
    assert F.nearest_code(np.array([6.0]), 1.0, F.E2M1_GRID)[0] == 7


def test_ds_mla_record_layout_matches_pages():
    g = golden(GOLDEN_DS)
    sizes = dict(nope=int(g["nope_bytes"]), scales=int(g["scale_bytes"]),
                 pad=int(g["pad_bytes"]), rope=int(g["rope_bytes"]))
    assert sum(sizes.values()) == int(g["record_bytes"]) == F.DS_RECORD_BYTES
    starts, off = {}, 0
    for name in g["region_order"].split():
        starts[name] = off
        off += sizes[name]
    assert starts["nope"] == F.NOPE_OFFSET and sizes["nope"] == F.NOPE_BYTES
    assert starts["scales"] == F.DS_SCALE_OFFSET and sizes["scales"] == F.N_GROUPS
    assert starts["pad"] == F.DS_PAD_OFFSET and sizes["pad"] == F.DS_PAD_BYTES
    assert starts["rope"] == F.DS_ROPE_OFFSET and sizes["rope"] == 2 * F.ROPE_DIM
    assert int(g["scale_group_elements"]) == F.GROUP
    assert sum(int(t) for t in g["fp8_ds_mla_regions"].split()) == int(g["fp8_ds_mla_record_bytes"])


def test_bf16_decode_matches_torch_all_65536():
    bits = np.arange(1 << 16, dtype=np.int64)
    ours = F.bf16_decode(bits)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref, equal_nan=True)
    num = ~np.isnan(ref)                       # a NaN's sign carries nothing
    assert np.array_equal(np.signbit(ours[num]), np.signbit(ref[num]))
    fin = np.isfinite(ref)
    assert np.array_equal(F.bf16_bits(ref[fin]).astype(np.int64), bits[fin])
