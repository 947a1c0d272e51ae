"""Pins of the oracle's quantize-append and dequantization.

Pinned against: torch's float8_e4m3fn rounding of amax/6 (the pages' literal
definition of the block scale, evaluated by a library routine), a record whose
bytes follow in closed form from a crafted token, exact rational brute force
over all 16 codes, the invariants the pages' write-path test states, and
exhaustive enumeration of the dequantized products.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codec as C
from oracle import formats as F
from sparse_mla_decode_nvfp4_amd import workloads as W


def bf16_values(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def positive_finite_bf16():
    bits = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16)
    return bits.view(torch.bfloat16).to(torch.float64).numpy()


def test_block_scale_is_e4m3_of_amax_over_6_for_every_bf16_amax():
    """[vLLM-82] test commit: stored scales equal E4M3(group_amax / 6)."""
    amax = positive_finite_bf16()
    lat = np.zeros((len(amax), 512))
    lat[:, 5] = amax                       # one element per token sets block 0's amax
    got = C.block_scales(lat)[:, 0]
    q = torch.from_numpy(amax).to(torch.float32) / 6.0   # IEEE, correctly rounded
    inrange = (q < 464.0).numpy()
    ref = q[inrange].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[inrange], ref)
    assert np.all(got[~inrange] == 0x7E)   # saturates, never NaN
    assert np.all(C.block_scales(np.zeros((1, 512))) == 0)


def test_block_scale_is_e4m3_of_amax_over_6_for_every_fp16_amax():
    """The fp16-input write path uses the same rule: for every positive
    finite fp16 amax the oracle's exact-quotient scale equals torch's
    float8_e4m3fn rounding of the correctly rounded fp32 quotient (so fp32
    division is exact enough for fp16 inputs too)."""
    bits = torch.arange(1, 0x7C00, dtype=torch.int32).to(torch.int16)
    amax = bits.view(torch.float16).to(torch.float64).numpy()
    lat = np.zeros((len(amax), 512))
    lat[:, 9] = -amax
    got = C.block_scales(lat)[:, 0]
    q = torch.from_numpy(amax).to(torch.float32) / 6.0
    inrange = (q < 464.0).numpy()
    ref = q[inrange].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[inrange], ref)
    assert np.all(got[~inrange] == 0x7E)


def crafted_token():
    """Block s: elements i = 0..14 are sign(i) * grid[i % 8] * v_s with the
    sign negative for i >= 8, element 15 is 6 * v_s (the amax), where v_s is
    the value of E4M3 code 0x20 + s.  RoPE k is +-value(E4M3 code 0x30 + k//2),
    negative for odd k."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    lat = np.zeros(512)
    for s in range(32):
        code = 0x20 + s
        e, m = code >> 3, code & 7
        v = 2.0 ** (e - 7) * (1 + m / 8)
        for i in range(15):
            val = grid[i % 8] * v
            lat[16 * s + i] = -val if i >= 8 else val
        lat[16 * s + 8] = -0.0
        lat[16 * s + 15] = 6 * v
    rope = np.zeros(64)
    for k in range(64):
        code = 0x30 + k // 2
        e, m = code >> 3, code & 7
        v = 2.0 ** (e - 7) * (1 + m / 8)
        rope[k] = -v if k % 2 else v
    return lat, rope


def test_crafted_record_bytes_in_closed_form():
    lat, rope = crafted_token()
    rec = C.quantize_records(lat[None], rope[None])[0]
    # NoPE: codes per block are 0..7, 8..14 (negative), 7 -> nibble pairs
    block_bytes = [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0x7E]
    assert rec[:256].tolist() == block_bytes * 32
    # RoPE: code 0x30 + k//2 with the sign bit on odd k
    assert rec[256:320].tolist() == [(0x30 + k // 2) | (0x80 if k % 2 else 0) for k in range(64)]
    # scales: byte j of the scale area holds block 4*(j&7) + (j>>3)
    assert rec[320:352].tolist() == [0x20 + 4 * (j & 7) + (j >> 3) for j in range(32)]
    # and dequantization returns the token exactly, signed zeros included
    back = C.dequantize_records(rec[None])[0]
    assert np.array_equal(back[:512], lat) and np.array_equal(back[512:], rope)
    assert np.array_equal(np.signbit(back[:512]), np.signbit(lat))


def brute_code(x, sv):
    """Exact search over all 16 codes: nearest value, ties to the even
    magnitude code, sign taken from x."""
    vals = F.e2m1_decode(np.arange(8))
    if sv == 0:
        mag = 0
    else:
        d = [abs(Fraction(abs(x)) - Fraction(sv) * Fraction(v)) for v in vals]
        best = min(d)
        cand = [k for k in range(8) if d[k] == best]
        mag = cand[0] if len(cand) == 1 else [k for k in cand if k % 2 == 0][0]
    return (8 if np.signbit(x) else 0) | mag


def test_nope_codes_against_brute_force():
    lat, _ = W.latents(0, 40)
    x = lat.to(torch.float64).numpy()
    x[0, :16] = 0.0
    x[1, :16] = -0.0
    x[2, :16] = 1e-8                       # amax/6 below the smallest scale
    s = C.block_scales(x)
    codes = C.nope_codes(x, s)
    sv = F.e4m3_decode(s)
    for n in range(40):
        for d in range(0, 512, 3):
            assert codes[n, d] == brute_code(x[n, d], sv[n, d // 16]), (n, d)


def test_write_path_invariants_on_synthetic_latents():
    """[vLLM-82] test commit: scale within half a mantissa step of amax/6,
    per-element NoPE error at most 1.25x the group scale (for normal E4M3
    scales), RoPE verbatim where representable."""
    lat, rope = W.latents(0, 256)
    x = lat.to(torch.float64).numpy()
    r = rope.to(torch.float64).numpy()
    rec = C.quantize_records(x, r)
    s = C.record_scale_bytes(rec)
    sv = F.e4m3_decode(s)
    amax = np.abs(x.reshape(-1, 32, 16)).max(-1)
    # half a mantissa step (relative 1/16) of amax/6 for normal scales
    normal = sv >= 2.0 ** -6
    assert np.all(np.abs(sv - amax / 6)[normal] <= (amax / 6)[normal] / 16 + 1e-300)
    deq = C.dequantize_records(rec)
    err = np.abs(deq[:, :512] - x).reshape(-1, 32, 16).max(-1)
    assert np.all(err[normal] <= 1.25 * sv[normal])
    # RoPE lane: unscaled RNE E4M3, so an E4M3-representable value round-trips
    assert np.array_equal(deq[:, 512:], F.e4m3_decode(F.e4m3_encode_satfinite(r)))
    rep = F.e4m3_decode(np.arange(0x7F))
    rr = np.concatenate([rep, -rep])[:128].reshape(2, 64)
    rec2 = C.quantize_records(np.zeros((2, 512)), rr)
    assert np.array_equal(C.dequantize_records(rec2)[:, 512:], rr)


def test_saturation_and_zero_groups():
    x = np.zeros((1, 512))
    x[0, 0:16] = 1e6                       # amax/6 >> 448
    x[0, 16:32] = -1e6
    x[0, 32] = -0.0
    rec = C.quantize_records(x, np.zeros((1, 64)))
    s = C.record_scale_bytes(rec)[0]
    codes = C.record_nope_codes(rec)[0]
    assert s[0] == 0x7E and s[1] == 0x7E and s[2] == 0
    assert np.all(codes[0:16] == 7) and np.all(codes[16:32] == 15)
    assert codes[32] == 8 and np.all(codes[33:48] == 0)


def test_every_dequantized_product_is_exact_in_bf16():
    """NoPE products e2m1 * e4m3 (16 codes x 127 finite scales) and all finite
    E4M3 RoPE values survive a round trip through bfloat16 unchanged."""
    prods = np.outer(F.e2m1_decode(np.arange(16)), F.e4m3_decode(np.arange(0x7F))).reshape(-1)
    rope = F.e4m3_decode(np.array([b for b in range(256) if b & 0x7F != 0x7F]))
    for v in (prods, rope):
        back = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(back, v) and np.array_equal(np.signbit(back), np.signbit(v))


def test_quantize_append_leaves_unmapped_slots_untouched():
    rng = np.random.default_rng(3)
    cache = rng.integers(0, 256, size=(64, 352), dtype=np.uint8)
    lat, rope = W.latents(0, 10)
    x = lat.to(torch.float64).numpy()
    r = rope.to(torch.float64).numpy()
    sm = np.array([5, -1, 17, 63, -1, 0, 2, 40, 41, -1])
    out = C.quantize_append(cache, x, r, sm)
    keep = sm >= 0
    assert np.array_equal(out[sm[keep]], C.quantize_records(x[keep], r[keep]))
    untouched = np.setdiff1d(np.arange(64), sm[keep])
    assert np.array_equal(out[untouched], cache[untouched])


def ds_tokens(n=64, rep=0):
    lat, rope = W.latents(0, n, rep=rep)
    return lat, rope, lat.to(torch.float64).numpy(), rope.to(torch.float64).numpy()


def test_ds_mla_record_meets_the_pages_test_invariants():
    """[vLLM-82] test commit, on the 432-byte record itself: scales within half
    a mantissa step of amax/6, NoPE error at most 1.25x the group scale
    (normal scales), the 16-byte pad zero, the RoPE lane the input's bf16 bits
    verbatim (compared with torch's own bf16 bit patterns)."""
    lat, rope, x, r = ds_tokens(256)
    rec = C.quantize_records(x, r, F.DS_RECORD_BYTES)
    assert rec.shape == (256, 432)
    sv = F.e4m3_decode(C.record_scale_bytes(rec))
    amax = np.abs(x.reshape(-1, 32, 16)).max(-1)
    normal = sv >= 2.0 ** -6
    assert np.all(np.abs(sv - amax / 6)[normal] <= (amax / 6)[normal] / 16 + 1e-300)
    deq = C.dequantize_records(rec)
    err = np.abs(deq[:, :512] - x).reshape(-1, 32, 16).max(-1)
    assert np.all(err[normal] <= 1.25 * sv[normal])
    assert np.all(rec[:, 288:304] == 0)
    torch_bits = rope.contiguous().view(torch.int16).numpy().view(np.uint8).reshape(256, 128)
    assert np.array_equal(rec[:, 304:432], torch_bits)
    assert np.array_equal(deq[:, 512:], r)


def test_ds_mla_and_352_records_share_codes_and_scales():
    """The two records differ only in where the scales sit and how RoPE is
    stored: the NoPE bytes are identical and the 432-byte record's scale byte
    256 + s equals the 352-byte record's byte 320 + 8(s&3) + (s>>2)."""
    _, _, x, r = ds_tokens(64, rep=3)
    a = C.quantize_records(x, r)
    b = C.quantize_records(x, r, F.DS_RECORD_BYTES)
    assert np.array_equal(a[:, :256], b[:, :256])
    for s in range(32):
        assert np.array_equal(b[:, 256 + s], a[:, 320 + 8 * (s & 3) + (s >> 2)])
    assert np.array_equal(C.dequantize_records(a)[:, :512], C.dequantize_records(b)[:, :512])


def test_ds_mla_append_leaves_unmapped_slots_untouched():
    rng = np.random.default_rng(5)
    cache = rng.integers(0, 256, size=(50, 432), dtype=np.uint8)
    _, _, x, r = ds_tokens(8, rep=4)
    sm = np.array([3, -1, 49, 0, 7, -1, 20, 21])
    out = C.quantize_append(cache, x, r, sm)
    keep = sm >= 0
    assert np.array_equal(out[sm[keep]], C.quantize_records(x[keep], r[keep], F.DS_RECORD_BYTES))
    untouched = np.setdiff1d(np.arange(50), sm[keep])
    assert np.array_equal(out[untouched], cache[untouched])
