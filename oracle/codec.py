"""Quantize-append (write path) and record dequantization, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Write path ([vLLM-82] Fix section and test commit message; [FlashMLA-18] PR
description for the 352-byte record):
  for every NoPE block of 16 latent elements
      amax  = max |x_i|
      S     = E4M3(amax / 6)                 (block scale byte, RNE, saturating)
      code  = sign(x_i) | RNE_e2m1(|x_i| / value(S))   (0 when value(S) == 0)
  two codes per byte (even element in the low nibble).  In the 352-byte
  record the scale of block s sits at scale byte 8*(s&3) + (s>>2) and RoPE is
  stored as unscaled E4M3 (RNE, sign kept).  In the 432-byte record
  ([vLLM-82] summary, Fix and test commit) the scales follow in block order,
  a 16-byte pad is zero and the bf16 RoPE bits are copied verbatim.
  A token whose slot is negative is skipped; every other byte of the cache is
  left as it was ([vLLM-82] Tests: unmapped slots stay untouched).

Dequantization ([FlashMLA-18] PR description, "dequantizes to bf16"): NoPE
element = e2m1(code) * e4m3(scale of its block), RoPE element = e4m3(byte)
or the stored bf16 value; the token's key is [NoPE 512 | RoPE 64] and its
value is the NoPE part.  The record width (352 or 432) selects the layout.
"""

import numpy as np

from .formats import (NOPE_DIM, ROPE_DIM, GROUP, N_GROUPS, NOPE_BYTES,
                      ROPE_OFFSET, SCALE_OFFSET, RECORD_BYTES, DS_SCALE_OFFSET,
                      DS_ROPE_OFFSET, DS_RECORD_BYTES, E2M1_GRID, E4M3_GRID,
                      bf16_bits, bf16_decode, e2m1_decode, e4m3_decode,
                      e4m3_encode_satfinite, nearest_code,
                      scale_byte_position)


def block_scales(latent):
    """E4M3 scale byte of every 16-element NoPE block: E4M3(amax/6).

    latent: float64 [N, 512] (finite).  Returns uint8 [N, 32].  The nearest
    E4M3 value to amax/6 is the one whose sextuple is nearest to amax; that
    comparison is exact, so no quotient is ever rounded.
    """
    x = np.asarray(latent, dtype=np.float64)
    assert x.shape[-1] == NOPE_DIM and np.all(np.isfinite(x))
    amax = np.abs(x.reshape(x.shape[0], N_GROUPS, GROUP)).max(axis=-1)
    return nearest_code(amax, 6.0, E4M3_GRID).astype(np.uint8)


def nope_codes(latent, scales):
    """4-bit E2M1 codes of the NoPE elements given their block scale bytes.

    Magnitude = nearest grid point of |x| / value(S), ties to the even code,
    saturating at 6; a zero scale gives magnitude 0.  The sign bit is copied
    from x (so -0.0 and small negatives that round to 0 keep it).
    """
    x = np.asarray(latent, dtype=np.float64)
    sv = e4m3_decode(scales).astype(np.float64)          # [N, 32]
    step = np.repeat(sv, GROUP, axis=1)                  # [N, 512]
    mag = nearest_code(np.abs(x), step, E2M1_GRID)
    return (np.signbit(x).astype(np.int64) << 3 | mag).astype(np.uint8)


def _scale_positions(record_bytes):
    """Byte of each block's scale within a record of this width."""
    s = np.arange(N_GROUPS)
    if record_bytes == DS_RECORD_BYTES:
        return DS_SCALE_OFFSET + s
    assert record_bytes == RECORD_BYTES
    return SCALE_OFFSET + scale_byte_position(s)


def quantize_records(latent, rope, record_bytes=RECORD_BYTES):
    """352- (default) or 432-byte records for N tokens.  latent [N,512],
    rope [N,64] float64 (bf16 values for the 432-byte record)."""
    latent = np.asarray(latent, dtype=np.float64)
    rope = np.asarray(rope, dtype=np.float64)
    n = latent.shape[0]
    assert latent.shape == (n, NOPE_DIM) and rope.shape == (n, ROPE_DIM)
    scales = block_scales(latent)
    codes = nope_codes(latent, scales)
    rec = np.zeros((n, record_bytes), dtype=np.uint8)      # the pad stays zero
    rec[:, :NOPE_BYTES] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    if record_bytes == DS_RECORD_BYTES:
        bits = bf16_bits(rope)
        rec[:, DS_ROPE_OFFSET:DS_ROPE_OFFSET + 2 * ROPE_DIM:2] = bits & 0xFF
        rec[:, DS_ROPE_OFFSET + 1:DS_ROPE_OFFSET + 2 * ROPE_DIM:2] = bits >> 8
    else:
        rec[:, ROPE_OFFSET:ROPE_OFFSET + ROPE_DIM] = e4m3_encode_satfinite(rope)
    rec[:, _scale_positions(record_bytes)] = scales
    return rec


def quantize_append(cache, latent, rope, slot_mapping):
    """Write path on a flat cache copy.

    cache: uint8 [num_slots, 352 or 432] (returned modified copy; its width
    selects the record).  slot_mapping: int [N]; a negative slot skips that
    token.  Slots are distinct.
    """
    out = np.array(cache, dtype=np.uint8, copy=True)
    slots = np.asarray(slot_mapping).astype(np.int64)
    keep = slots >= 0
    assert len(np.unique(slots[keep])) == int(keep.sum()), "slots must be distinct"
    rec = quantize_records(np.asarray(latent)[keep], np.asarray(rope)[keep], out.shape[1])
    out[slots[keep]] = rec
    return out


def record_scale_bytes(records):
    """Scale byte of block s for every record (undoing the 352-byte record's
    permutation)."""
    rec = np.asarray(records, dtype=np.uint8)
    return rec[:, _scale_positions(rec.shape[1])]


def record_nope_codes(records):
    """The 512 4-bit codes of every record, in element order."""
    rec = np.asarray(records, dtype=np.uint8)
    nib = rec[:, :NOPE_BYTES]
    codes = np.empty((rec.shape[0], NOPE_DIM), dtype=np.uint8)
    codes[:, 0::2] = nib & 0xF
    codes[:, 1::2] = nib >> 4
    return codes


def dequantize_records(records):
    """float64 [N, 576] keys: [e2m1 * scale (512) | e4m3 RoPE (64)]."""
    rec = np.asarray(records, dtype=np.uint8)
    codes = record_nope_codes(rec)
    sv = np.repeat(e4m3_decode(record_scale_bytes(rec)), GROUP, axis=1)
    nope = e2m1_decode(codes) * sv
    if rec.shape[1] == DS_RECORD_BYTES:
        lo = rec[:, DS_ROPE_OFFSET:DS_ROPE_OFFSET + 2 * ROPE_DIM:2].astype(np.uint16)
        hi = rec[:, DS_ROPE_OFFSET + 1:DS_ROPE_OFFSET + 2 * ROPE_DIM:2].astype(np.uint16)
        rope = bf16_decode(lo | (hi << 8))
    else:
        rope = e4m3_decode(rec[:, ROPE_OFFSET:ROPE_OFFSET + ROPE_DIM])
    return np.concatenate([nope, rope], axis=1)
