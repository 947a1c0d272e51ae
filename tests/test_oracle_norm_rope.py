"""Pins of the fused write path's oracle (oracle/norm_rope.py) against what the
mathematics fixes, independently of the oracle's own code:

  * RMSNorm: inputs whose mean square is a power of four normalise exactly
    to x / rms; scaling x by a power of two changes nothing (bit for bit);
    against x * w / sqrt(mean(x^2) + eps) evaluated in float64 the binary32
    steps stay within a few units in the last place, with eps making a
    visible difference;
  * rotary: angle 0 is the identity, 90 degrees maps (a, b) to (-b, a), 180
    degrees negates, and against complex multiplication by e^{i theta} in
    float64 the result stays within rounding; the half-split ("neox")
    layout is the interleaved one on permuted dims;
  * bf16 rounding: ties go to the even pattern, and it agrees with torch's
    float32 -> bfloat16 conversion;
  * the fused records equal the plain write rule on the intermediate, and
    the append skips negative slots and positions outside the table.
"""

import numpy as np
import pytest
import torch

from oracle import codec as OC
from oracle import norm_rope as NR


def bf16_values(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(np.maximum(x, np.float32(1e-30))).astype(np.float64)


def test_power_of_four_mean_square_normalises_exactly():
    rng = np.random.default_rng(1)
    for k in (-6, 0, 3):
        c = 2.0 ** k
        x = np.where(rng.random((5, 512)) < 0.5, -c, c)          # mean square c^2
        y = NR.rms_norm_f32(x, np.ones(512), 0.0)
        assert np.array_equal(y.astype(np.float64), x / c)       # r = 1/c exactly
    # with unit weight, zero eps and a zero angle the records are those of
    # the plain write rule on x / rms
    x = np.where(rng.random((3, 512)) < 0.5, -4.0, 4.0)
    rope = bf16_values(rng.standard_normal((3, 64)))
    cos, sin = np.ones((3, 32), np.float32), np.zeros((3, 32), np.float32)
    got = NR.fused_records(x, rope, np.ones(512), 0.0, cos, sin)
    assert np.array_equal(got, OC.quantize_records(x / 4.0, rope))


def test_scaling_by_a_power_of_two_leaves_the_norm_unchanged():
    rng = np.random.default_rng(2)
    x = bf16_values(rng.standard_normal((16, 512)) * 3)
    w = bf16_values(rng.uniform(0.5, 1.5, 512))
    y = NR.rms_norm_f32(x, w, 0.0)
    for k in (-9, -2, 5, 12):
        assert np.array_equal(NR.rms_norm_f32(x * 2.0 ** k, w, 0.0), y)


@pytest.mark.parametrize("rms,eps", [(1.0, 1e-6), (0.01, 1e-4), (5.0, 0.0), (0.003, 1e-5)])
def test_norm_matches_the_float64_definition(rms, eps):
    rng = np.random.default_rng(int(rms * 1000) + 7)
    x = bf16_values(rng.standard_normal((64, 512)) * rms)
    w = bf16_values(rng.uniform(-2, 2, 512))
    eps32 = float(np.float32(eps))
    y = NR.rms_norm_f32(x, w, eps32).astype(np.float64)
    ref = x * w / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps32)
    # squares exact, 63 additions, sqrt, divide, two products: a few ulps
    assert np.all(np.abs(y - ref) <= 8 * ulp32(ref) + 1e-38)
    if eps > 0 and rms < 0.05:
        # eps is in the denominator: dropping it moves the result
        no_eps = x * w / np.sqrt(np.mean(x * x, axis=1, keepdims=True))
        assert np.max(np.abs(no_eps - ref) / (np.abs(ref) + 1e-30)) > 1e-3


def test_rotation_closed_forms():
    rng = np.random.default_rng(3)
    x = bf16_values(rng.standard_normal((4, 64)))
    one, zero = np.ones((4, 32), np.float32), np.zeros((4, 32), np.float32)
    for neox in (False, True):
        assert np.array_equal(NR.rotate_f32(x, one, zero, neox), x.astype(np.float32))
        assert np.array_equal(NR.rotate_f32(x, -one, zero, neox), -x.astype(np.float32))
    r90 = NR.rotate_f32(x, zero, one, neox=False)
    assert np.array_equal(r90[:, 0::2], -x[:, 1::2]) and np.array_equal(r90[:, 1::2], x[:, 0::2])
    r90n = NR.rotate_f32(x, zero, one, neox=True)
    assert np.array_equal(r90n[:, :32], -x[:, 32:]) and np.array_equal(r90n[:, 32:], x[:, :32])


def test_rotation_is_complex_multiplication_by_the_angle():
    rng = np.random.default_rng(4)
    x = bf16_values(rng.standard_normal((32, 64)) * 2)
    theta = rng.uniform(-np.pi, np.pi, (32, 32))
    cos, sin = np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)
    got = NR.rotate_f32(x, cos, sin, neox=False).astype(np.float64)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * (cos.astype(np.float64) + 1j * sin.astype(np.float64))
    mag = np.abs(x[:, 0::2]) + np.abs(x[:, 1::2])
    tol = 4 * ulp32(mag)
    assert np.all(np.abs(got[:, 0::2] - z.real) <= tol)
    assert np.all(np.abs(got[:, 1::2] - z.imag) <= tol)
    # the pair's length is kept (cos^2 + sin^2 = 1 up to float32 rounding)
    n0 = np.hypot(x[:, 0::2], x[:, 1::2])
    n1 = np.hypot(got[:, 0::2], got[:, 1::2])
    assert np.all(np.abs(n1 - n0) <= 1e-5 * (n0 + 1e-30) + 8 * ulp32(n0))


def test_neox_layout_is_the_interleaved_one_on_permuted_dims():
    rng = np.random.default_rng(5)
    x = bf16_values(rng.standard_normal((8, 64)))
    theta = rng.uniform(-3, 3, (8, 32))
    cos, sin = np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)
    perm = np.empty(64, np.int64)
    perm[0::2], perm[1::2] = np.arange(32), np.arange(32) + 32     # (i, i+32) -> (2i, 2i+1)
    a = NR.rotate_f32(x, cos, sin, neox=True)
    b = NR.rotate_f32(x[:, perm], cos, sin, neox=False)
    assert np.array_equal(a[:, perm], b)


def test_bf16_rounding_ties_to_even_and_agrees_with_torch():
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -100 * (1 + 2 ** -8),
                     1 + 2 ** -8 + 2 ** -20], np.float32)
    want = np.array([1.0, 1 + 2 ** -6, -1.0, 2 ** -100, 1 + 2 ** -7])
    assert np.array_equal(NR.bf16_round(vals), want)
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    assert np.array_equal(NR.bf16_round(x), bf16_values(x))


def test_fused_records_are_the_write_rule_on_the_bf16_intermediate():
    rng = np.random.default_rng(7)
    x = bf16_values(rng.standard_normal((20, 512)) * 2)
    r = bf16_values(rng.standard_normal((20, 64)))
    w = bf16_values(rng.uniform(0.2, 2.0, 512))
    theta = rng.uniform(-3, 3, (20, 32))
    cos, sin = np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)
    for rb, neox in ((352, False), (432, True)):
        y, rr = NR.norm_rope_bf16(x, r, w, 1e-6, cos, sin, neox)
        assert np.array_equal(NR.fused_records(x, r, w, 1e-6, cos, sin, neox, rb),
                              OC.quantize_records(y, rr, rb))


def test_fused_append_skips_negative_slots_and_positions_outside_the_table():
    rng = np.random.default_rng(8)
    n, slots_total, max_pos = 12, 40, 100
    x = bf16_values(rng.standard_normal((n, 512)))
    r = bf16_values(rng.standard_normal((n, 64)))
    w = bf16_values(rng.uniform(0.5, 1.5, 512))
    ang = np.arange(max_pos)[:, None] * 0.01 * np.arange(1, 33)[None, :]
    table = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    pos = rng.integers(0, max_pos, n)
    pos[3], pos[7] = max_pos, -1                      # outside the table
    slot = rng.permutation(slots_total)[:n].astype(np.int64)
    slot[5] = -1
    cache = rng.integers(0, 256, (slots_total, 352), dtype=np.uint8)
    out = NR.fused_append(cache, x, r, w, 1e-6, table, pos, slot)
    keep = np.ones(n, bool)
    keep[[3, 5, 7]] = False
    untouched = np.setdiff1d(np.arange(slots_total), slot[keep])
    assert np.array_equal(out[untouched], cache[untouched])
    c, s = NR.table_rows(table, pos[keep])
    assert np.array_equal(out[slot[keep]], NR.fused_records(x[keep], r[keep], w, 1e-6, c, s))
