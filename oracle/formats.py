"""Element encodings and the 352- and 432-byte token records, restated from
the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Record layout ("nvfp4.fp8rope", [FlashMLA-18] PR description):
  bytes [0, 256)    512 E2M1 NoPE codes, two per byte
  bytes [256, 320)  64 E4M3 RoPE values, no block scale
  bytes [320, 352)  32 E4M3 NoPE block scales, one per 16 elements, permuted:
                    the scale of element block s sits at byte 8*(s&3) + (s>>2)
                    of this area (an 8x4 -> 4x8 transpose).

Record layout ("nvfp4_ds_mla", 432 bytes, [vLLM-82] summary and Fix: 256 B
FP4 NoPE + 32 B E4M3 scales + 16 B alignment pad + 128 B BF16 RoPE):
  bytes [0, 256)    the same 512 E2M1 NoPE codes
  bytes [256, 288)  32 E4M3 block scales
  bytes [288, 304)  zero pad
  bytes [304, 432)  64 bf16 RoPE values, the input's 16-bit pattern verbatim

Readings where the page is silent (each listed in the design notes):
  * Nibble order of "packed 2/byte": element 2j is the LOW nibble of byte j,
    element 2j+1 the high nibble.
  * E4M3 is the OCP FP8 E4M3 ("fn") variant: bias 7, no infinities, the
    all-ones pattern 0x7F/0xFF is NaN, largest finite 448.
  * Rounding to either grid is round-to-nearest, ties to the even code, on the
    finite grid; magnitudes beyond the largest finite value saturate to it.
  * The 432-byte record's regions lie in the order the page lists them; its
    scales are in block order (the page names no permutation for it); its
    NoPE bytes pack nibbles as the 352-byte record does; bf16 is stored
    little-endian.

Every decoder is written from the bit fields; the grids used for encoding are
produced by those decoders.  Encoding never divides: "nearest to a/b" is
decided by comparing a with b*g for every grid value g, products that are
exact in float64 for these operands (b has at most 4 significant bits and g at
most 4), so every rounding decision is exact.
"""

import numpy as np

NOPE_DIM = 512
ROPE_DIM = 64
QK_DIM = NOPE_DIM + ROPE_DIM       # d_qk = 576
V_DIM = NOPE_DIM                   # d_v = 512
GROUP = 16                         # elements per NoPE block scale
N_GROUPS = NOPE_DIM // GROUP       # 32
NOPE_OFFSET = 0
NOPE_BYTES = NOPE_DIM // 2         # 256
ROPE_OFFSET = NOPE_OFFSET + NOPE_BYTES   # 256
SCALE_OFFSET = ROPE_OFFSET + ROPE_DIM    # 320
RECORD_BYTES = SCALE_OFFSET + N_GROUPS   # 352

# the 432-byte "nvfp4_ds_mla" record
DS_SCALE_OFFSET = NOPE_OFFSET + NOPE_BYTES       # 256
DS_PAD_OFFSET = DS_SCALE_OFFSET + N_GROUPS       # 288
DS_PAD_BYTES = 16
DS_ROPE_OFFSET = DS_PAD_OFFSET + DS_PAD_BYTES    # 304
DS_RECORD_BYTES = DS_ROPE_OFFSET + 2 * ROPE_DIM  # 432

E2M1_MAX = 6.0


def scale_byte_position(s):
    """Byte (relative to the scale area) holding the scale of NoPE block s.

    [FlashMLA-18] PR description: block s is stored at 8*(s & 3) + (s >> 2).
    """
    s = np.asarray(s)
    return 8 * (s & 3) + (s >> 2)


def e2m1_decode(code):
    """Value of a 4-bit E2M1 code: 1 sign, 2 exponent (bias 1), 1 mantissa bit.

    Exponent field 0 is subnormal: value = M * 0.5.  Otherwise
    value = 2**(E-1) * (1 + M/2).  Largest magnitude 6 ([FlashMLA-18]:
    "2 exponent bits, max 6").
    """
    code = np.asarray(code).astype(np.int64)
    sign = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(sign == 1, -mag, mag)


def e4m3_decode(byte):
    """Value of an OCP E4M3 byte: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal: value = 2**-6 * M/8.  Exponent 15 with
    mantissa 7 is NaN (no infinities).  Sign applies to zero too (-0.0).
    """
    b = np.asarray(byte).astype(np.int64)
    sign = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# Non-negative finite grids, indexed by magnitude code (monotone increasing).
E2M1_GRID = e2m1_decode(np.arange(8))            # [0, .5, 1, 1.5, 2, 3, 4, 6]
E4M3_GRID = e4m3_decode(np.arange(0x7F))         # codes 0x00..0x7E, max 448


def nearest_code(a, step, grid):
    """Code k minimising |a - step*grid[k]|, ties to the even code.

    a, step: broadcastable non-negative float64 arrays.  grid: increasing
    non-negative grid (index = code).  Values beyond step*grid[-1] saturate to
    the last code.  step == 0 gives code 0.  The candidate products step*g are
    exact in float64 for the encodings used here, so the comparison is exact.
    """
    a = np.asarray(a, dtype=np.float64)
    step = np.asarray(step, dtype=np.float64)
    a, step = np.broadcast_arrays(a, step)
    flat_a = a.reshape(-1)
    flat_s = step.reshape(-1)
    out = np.zeros(flat_a.shape, dtype=np.int64)
    nz = np.nonzero(flat_s > 0)[0]
    chunk = 1 << 16
    for c0 in range(0, len(nz), chunk):
        sel = nz[c0:c0 + chunk]
        out[sel] = _nearest_rows(flat_a[sel], flat_s[sel], grid)
    return out.reshape(a.shape)


def _nearest_rows(aa, ss, grid):
    n = len(grid)
    cand = ss[:, None] * grid[None, :]          # exact products
    # index of the last grid point <= a (grid[0] = 0 <= a always)
    lo = np.sum(cand <= aa[:, None], axis=1) - 1
    hi = np.minimum(lo + 1, n - 1)
    rows = np.arange(len(aa))
    # a is nearer to cand[lo] iff 2a < cand[lo] + cand[hi]; both sides are
    # exact in float64 (adjacent grid products have few significant bits).
    twice_mid = cand[rows, lo] + cand[rows, hi]
    twice_a = 2.0 * aa
    pick = np.where(twice_a < twice_mid, lo, np.where(twice_a > twice_mid, hi,
                    np.where(lo % 2 == 0, lo, hi)))
    return np.where(lo == n - 1, n - 1, pick)   # saturate past the top


def e4m3_encode_satfinite(x):
    """E4M3 byte of a finite float64 x: RNE on the finite grid, saturating.

    The sign bit is kept (so -0.0 encodes to 0x80); 0x7F/0xFF never appear.
    """
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), "E4M3 encode needs finite input"
    mag = nearest_code(np.abs(x), 1.0, E4M3_GRID)
    return (np.signbit(x).astype(np.int64) << 7 | mag).astype(np.uint8)


def bf16_decode(bits):
    """Value of bfloat16 bit patterns (uint16), from the fields: sign, 8-bit
    exponent (bias 127), 7-bit fraction; exponent 255 gives inf/NaN."""
    b = np.asarray(bits).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(np.float64)
    with np.errstate(over="ignore"):
        mag = np.where(e == 0, f * 2.0 ** -133, (1.0 + f / 128.0) * np.exp2(e - 127.0))
    mag = np.where(e == 255, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def bf16_bits(x):
    """bfloat16 bit patterns of values that bfloat16 represents exactly (the
    16-bit inputs of the write path); anything else is an error."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64), equal_nan=True)
    u = x32.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "not a bfloat16 value"
    return (u >> 16).astype(np.uint16)
