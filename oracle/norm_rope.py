"""The fused write path: RMSNorm of the latent, rotary embedding of the RoPE
part, then the quantize-append of the two rounded to bfloat16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[sglang-38646] Limitations: without a fused NVFP4 store the path pays a bf16
intermediate plus a separate quantize kernel per layer; the fused kernel
normalises, rotates, quantizes and stores in one pass.  The pages name the
three steps and nothing more, so the readings here are the plainest ones:

  RMSNorm   y_i = x_i * w_i / sqrt(mean_j x_j^2 + eps)   over the 512 NoPE dims
  rotary    pairs of RoPE dims turned by the token position's angle:
              interleaved pairs (2i, 2i+1) (the DeepSeek layout), or
              half-split pairs (i, i+32) ("neox" layout),
            with a caller-supplied table row [cos_0..cos_31 | sin_0..sin_31]:
              a' = a*cos_i - b*sin_i,   b' = b*cos_i + a*sin_i
  then both are rounded to bf16 (the intermediate the unfused path stores)
  and quantized by the ordinary write rule (oracle.codec.quantize_records).

The rounding of the bf16 intermediate decides codes, so the oracle takes the
same single-precision steps as the kernel, each an IEEE binary32 operation
rounded to nearest even (numpy float32 arithmetic, no fused multiply-add):
  * squares x_i*x_i; a partial sum of elements 8l..8l+7 for l = 0..63, added
    in element order; the 64 partials added pairwise in a balanced tree
    (neighbours first: (0,1), (2,3), ..., then those sums pairwise, ...);
  * mean = sum / 512 (exact), v = mean + eps, s = sqrt(v), r = 1 / s;
  * y_i = (x_i * r) * w_i;
  * rotary: each product, then the difference or sum;
  * bf16 = round-to-nearest-even of the binary32 value.
"""

import numpy as np

from .codec import quantize_records
from .formats import NOPE_DIM, ROPE_DIM

HALF = ROPE_DIM // 2       # 32 frequencies


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def rms_norm_f32(latent, weight, eps):
    """Normalised latent before its bf16 rounding, float32 [N, 512].

    latent: [N, 512] values that are exact in float32 (bf16 inputs);
    weight: [512] (bf16 values); eps: a float32 value.
    """
    x = _f32(latent)
    n = x.shape[0]
    assert x.shape == (n, NOPE_DIM)
    w = _f32(weight)
    assert w.shape == (NOPE_DIM,)
    sq = x * x                                        # float32 products
    part = sq.reshape(n, 64, 8)
    acc = part[:, :, 0].copy()
    for k in range(1, 8):                             # element order within a lane
        acc = acc + part[:, :, k]
    while acc.shape[1] > 1:                           # neighbours first
        acc = acc[:, 0::2] + acc[:, 1::2]
    total = acc[:, 0]
    mean = total * np.float32(1.0 / NOPE_DIM)         # exact: a power of two
    v = mean + np.float32(eps)
    s = np.sqrt(v)                                    # IEEE sqrt, rounded
    r = np.float32(1.0) / s                           # IEEE division, rounded
    return (x * r[:, None]) * w[None, :]


def rotate_f32(rope, cos, sin, neox=False):
    """Rotated RoPE part before its bf16 rounding, float32 [N, 64].

    rope: [N, 64] (bf16 values); cos, sin: [N, 32] float32, the table row
    of each token's position.  Interleaved pairs (2i, 2i+1) unless neox,
    which pairs (i, i+32).
    """
    x = _f32(rope)
    c = _f32(cos)
    s = _f32(sin)
    n = x.shape[0]
    assert x.shape == (n, ROPE_DIM) and c.shape == (n, HALF) and s.shape == (n, HALF)
    if neox:
        a, b = x[:, :HALF], x[:, HALF:]
    else:
        a, b = x[:, 0::2], x[:, 1::2]
    a2 = a * c - b * s                                # products, then the difference
    b2 = b * c + a * s
    out = np.empty_like(x)
    if neox:
        out[:, :HALF], out[:, HALF:] = a2, b2
    else:
        out[:, 0::2], out[:, 1::2] = a2, b2
    return out


def bf16_round(x):
    """Round-to-nearest-even of float32 values to bfloat16, returned as
    float64 (finite inputs)."""
    u = _f32(x).view(np.uint32).astype(np.uint64)
    assert np.all(np.isfinite(_f32(x)))
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def table_rows(cos_sin_cache, positions):
    """(cos, sin) [N, 32] of each token from a [max_position, 64] table
    holding [cos_0..cos_31 | sin_0..sin_31] per position."""
    t = _f32(cos_sin_cache)[np.asarray(positions, dtype=np.int64)]
    return t[:, :HALF], t[:, HALF:]


def norm_rope_bf16(latent, rope, weight, eps, cos, sin, neox=False):
    """The bf16 intermediate: (normalised latent, rotated RoPE) as float64
    values of bfloat16 numbers."""
    return (bf16_round(rms_norm_f32(latent, weight, eps)),
            bf16_round(rotate_f32(rope, cos, sin, neox)))


def fused_records(latent, rope, weight, eps, cos, sin, neox=False, record_bytes=352):
    """Records written by the fused path: the write rule applied to the bf16
    intermediate."""
    y, r = norm_rope_bf16(latent, rope, weight, eps, cos, sin, neox)
    return quantize_records(y, r, record_bytes)


def fused_append(cache, latent, rope, weight, eps, cos_sin_cache, positions, slot_mapping,
                 neox=False):
    """Write path on a flat cache copy ([num_slots, 352 or 432]): tokens with a
    negative slot, or a position outside the table, are skipped; every other
    byte is left as it was."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    slots = np.asarray(slot_mapping).astype(np.int64)
    pos = np.asarray(positions).astype(np.int64)
    keep = (slots >= 0) & (pos >= 0) & (pos < np.asarray(cos_sin_cache).shape[0])
    assert len(np.unique(slots[keep])) == int(keep.sum()), "slots must be distinct"
    c, s = table_rows(cos_sin_cache, pos[keep])
    rec = fused_records(np.asarray(latent)[keep], np.asarray(rope)[keep], weight, eps, c, s,
                        neox, out.shape[1])
    out[slots[keep]] = rec
    return out
