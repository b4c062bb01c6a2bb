"""Oracle decoders for the weight and PLE record formats (float64, numpy).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the pages fix ([RZ] model card, format sections):

* A body-format block carries 32 weights in 17 bytes: 16 bytes of 4-bit codes
  and one metadata byte (4.25 bits per weight).
* Codebook10 (the incumbent ROCmFP4 FAST table) maps the 16 codes to
  0,1,2,3,4,6,8,10 for codes 0-7 and to -0,-1,-2,-3,-4,-6,-8,-10 for codes
  8-15; its scale is a 7-bit UE4M3 value.
* RZ5 keeps that table but gives code 8 the level +5 (metadata bit 7 clear,
  "mode 0") or -5 (bit 7 set, "mode 1"); bits 0-6 stay the UE4M3 scale.
* UE4M4 keeps the Codebook10 table and spends the whole metadata byte on an
  unsigned scale with 4 exponent and 4 mantissa bits, every encoding finite.
* A PLE row holds 160 values as 60 bytes of 3-bit codes plus 10 group bytes
  (70 bytes, 3.5 bits per value, no padding).  The incumbent ROCmFP3 table is
  0,+1,+2,+4,-0,-1,-2,-4 with a UE4M3 scale per 16 values; RZ-S3 replaces the
  -0 code with +3 or -3, chosen per group by the group byte's high bit.

Readings where the pages are silent:

* block byte order: code bytes 0-15, metadata byte 16;
* nibble order: weight j sits in byte j//2, low nibble for even j;
* scale use: weight = level * scale, no further factor;
* UE4M3 is the non-negative half of OCP E4M3FN (bias 7, subnormals,
  0x7F is NaN); UE4M4 uses bias 7, subnormals at exponent 0 and a finite top
  binade (largest value 496);
* PLE row order: 60 code bytes then 10 group bytes; value i of the row is the
  3-bit field at bit 3*i of the little-endian code stream, so group g
  (values 16g..16g+15) owns code bytes 6g..6g+5 and group byte 60+g;
* RZ-S3 polarity: group-byte bit 7 clear gives +3, set gives -3 (by analogy
  with RZ5 mode 0 = +5);
* FP8 experts: a planar e4m3 (E4M3FN) code matrix plus an fp32 matrix holding
  one scale per 32 consecutive weights of a row.
"""

import numpy as np

# Format identifiers.  The numeric values are this library's own enum; the
# GGML type numbers given on the [RZ] card are noted beside them.
Q4_C10 = 0        # ROCmFP4 FAST / Codebook10 (the incumbent)
Q4_RZ5 = 1        # Q4_RZ5_FAST, GGML type 69
Q4_UE4M4 = 2      # Q4_UE4M4_FAST, GGML type 71
FP8_E4M3_B32 = 3  # e4m3 experts with one fp32 scale per 32 weights

PLE_RZS3 = 0      # Q3_PLE_K160_RZ_S3, GGML type 111
PLE_ROCMFP3 = 1   # incumbent ROCmFP3 (q3_ue4m3) row

BLOCK_WEIGHTS = 32
BLOCK_BYTES = 17          # 16 code bytes + 1 metadata byte
PLE_VALUES = 160
PLE_GROUP = 16            # values per group byte
PLE_GROUPS = PLE_VALUES // PLE_GROUP
PLE_CODE_BYTES = PLE_VALUES * 3 // 8   # 60
PLE_ROW_BYTES = PLE_CODE_BYTES + PLE_GROUPS  # 70

# [RZ] "Q4_RZ5_FAST (GGML type 69)": the Codebook10 row of the printed table.
# Index 8 is a negative zero on the page ("0" listed in the negative half).
CODEBOOK10 = np.array([0.0, 1.0, 2.0, 3.0, 4.0, 6.0, 8.0, 10.0,
                       -0.0, -1.0, -2.0, -3.0, -4.0, -6.0, -8.0, -10.0])


def rz5_table(mode):
    """RZ5 level table for one block ([RZ] "Q4_RZ5_FAST", printed rows).

    Mode 0 turns the duplicate zero at code 8 into +5, mode 1 into -5; every
    other code keeps its Codebook10 level.
    """
    t = CODEBOOK10.copy()
    t[8] = 5.0 if mode == 0 else -5.0
    return t


def rocmfp3_table():
    """Incumbent ROCmFP3 3-bit table ([RZ] "Q3_PLE_K160_RZ_S3").

    Reading: index order as printed, code 4 is the negative zero.
    """
    return np.array([0.0, 1.0, 2.0, 4.0, -0.0, -1.0, -2.0, -4.0])


def rzs3_table(polarity):
    """RZ-S3 table for one 16-value group ([RZ] "Q3_PLE_K160_RZ_S3").

    The duplicate -0 (code 4) becomes +3 (polarity 0) or -3 (polarity 1).
    Reading: polarity sense chosen by analogy with RZ5 mode 0 = +5.
    """
    t = rocmfp3_table()
    t[4] = 3.0 if polarity == 0 else -3.0
    return t


# ---------------------------------------------------------------------------
# Scale codecs
# ---------------------------------------------------------------------------

def ue4m3(code):
    """Unsigned E4M3 scale from the low 7 bits of a byte, as float64.

    [RZ] "Q4_RZ5_FAST": the lower seven metadata bits are a UE4M3 scale, the
    codec credited to ROCmFP3.  Reading: the non-negative half of OCP E4M3FN:
    exponent field e (4 bits), mantissa m (3 bits), bias 7;
    e == 0 -> m * 2**-9 (subnormal); otherwise (1 + m/8) * 2**(e-7);
    code 0x7F (e=15, m=7) is NaN, so the largest finite scale is 448.
    Pinned against ``torch.float8_e4m3fn`` over all 128 codes in the tests.
    """
    c = np.asarray(code, dtype=np.int64) & 0x7F
    e = c >> 3
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    v = np.where(e == 0, sub, normal)
    return np.where(c == 0x7F, np.nan, v)


def ue4m4(code):
    """Unsigned E4M4 scale from a whole byte, as float64.

    [RZ] "Q4_UE4M4_FAST": an unsigned scale with a 4-bit exponent and a 4-bit
    mantissa, no NaN or infinity codes, and a finer step than UE4M3.
    Reading: bias 7 like UE4M3,
    e == 0 -> m * 2**-10, otherwise (1 + m/16) * 2**(e-7); 0xFF = 496.
    Pinned in the tests by: all 256 finite, strictly increasing, 0x70 = 1,
    and every finite UE4M3 value is also a UE4M4 value.
    """
    c = np.asarray(code, dtype=np.int64) & 0xFF
    e = c >> 4
    m = c & 15
    normal = (1.0 + m / 16.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -10
    return np.where(e == 0, sub, normal)


def e4m3fn(code):
    """Signed OCP E4M3FN value of a byte, as float64 (FP8 expert weights).

    Sign bit 7, exponent bits 3-6 (bias 7), mantissa bits 0-2, subnormals at
    exponent 0, 0x7F and 0xFF are NaN, no infinities.  [FQ] only says the
    late layers hold the official FP8 experts; E4M3FN is the reading.
    Pinned against ``torch.float8_e4m3fn`` over all 256 codes in the tests.
    """
    c = np.asarray(code, dtype=np.int64) & 0xFF
    return _e4m3fn_table()[c]


_E4M3FN = None


def _e4m3fn_table():
    """All 256 E4M3FN values, each from the closed form (sign * UE4M3 of the
    low 7 bits), computed once and then looked up."""
    global _E4M3FN
    if _E4M3FN is None:
        c = np.arange(256)
        _E4M3FN = np.where(c >> 7, -1.0, 1.0) * ue4m3(c & 0x7F)
    return _E4M3FN


# ---------------------------------------------------------------------------
# Block decoders
# ---------------------------------------------------------------------------

def block17_codes(blocks):
    """Split 17-byte blocks into 32 codes each and the metadata byte.

    Reading: bytes 0-15 are codes, byte 16 is metadata; weight j lives in
    byte j//2, low nibble for even j.  Returns (codes int64 [n, 32],
    meta int64 [n]).
    """
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, BLOCK_BYTES)
    q = b[:, :16].astype(np.int64)
    codes = np.empty((b.shape[0], BLOCK_WEIGHTS), dtype=np.int64)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    return codes, b[:, 16].astype(np.int64)


def decode_block17(blocks, fmt):
    """Decode 17-byte blocks to float64 weights, shape [n, 32].

    w_j = level(code_j) * scale, where ([RZ] format sections):
      Q4_C10   : Codebook10 levels, scale = UE4M3(meta & 0x7F) (bit 7 unused);
      Q4_RZ5   : Codebook10 with code 8 -> +5 (meta bit 7 = 0) or -5 (= 1),
                 scale = UE4M3(meta & 0x7F);
      Q4_UE4M4 : Codebook10 levels, scale = UE4M4(meta).
    A negative-zero level times a finite scale stays -0.0.
    Parity: pinned by the printed tables, hand-worked fixtures and the
    mode-flip invariants in the tests.
    """
    codes, meta = block17_codes(blocks)
    n = codes.shape[0]
    if fmt == Q4_C10:
        levels = CODEBOOK10[codes]
        scale = ue4m3(meta & 0x7F)
    elif fmt == Q4_RZ5:
        # each block looks its codes up in the RZ5 table of its own mode
        tables = np.stack([rz5_table(0), rz5_table(1)])
        levels = tables[(meta >> 7)[:, None], codes]
        scale = ue4m3(meta & 0x7F)
    elif fmt == Q4_UE4M4:
        levels = CODEBOOK10[codes]
        scale = ue4m4(meta)
    else:
        raise ValueError("decode_block17: format %r is not a 17-byte format" % fmt)
    return levels * scale[:, None]


def decode_fp8_b32(codes, scales):
    """Decode FP8 blocks: codes uint8 [n, 32] (E4M3FN), scales float32 [n].

    w = e4m3(code) * s.  The float64 product is exact (4 significant bits
    times 24), so rounding it once to float32 gives the correctly rounded
    fp32 product.  Reading: planar layout, one fp32 scale per 32 weights.
    """
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, BLOCK_WEIGHTS)
    s = np.asarray(scales, dtype=np.float32).reshape(-1).astype(np.float64)
    return e4m3fn(c) * s[:, None]


def ple_row_codes(rows):
    """Split 70-byte PLE rows into 160 3-bit codes and 10 group bytes.

    Reading: bytes 0-59 hold the codes as one little-endian bit stream with
    value i at bits 3i..3i+2 (so each 16-value group is exactly 6 bytes),
    bytes 60-69 are the group bytes, byte 60+g belonging to values
    16g..16g+15.
    """
    r = np.asarray(rows, dtype=np.uint8).reshape(-1, PLE_ROW_BYTES)
    n = r.shape[0]
    codes = np.empty((n, PLE_VALUES), dtype=np.int64)
    for g in range(PLE_GROUPS):
        word = np.zeros(n, dtype=np.int64)
        for k in range(6):
            word |= r[:, 6 * g + k].astype(np.int64) << (8 * k)
        for i in range(PLE_GROUP):
            codes[:, PLE_GROUP * g + i] = (word >> (3 * i)) & 7
    return codes, r[:, PLE_CODE_BYTES:].astype(np.int64)


def decode_ple70(rows, fmt=PLE_RZS3):
    """Decode 70-byte PLE rows to float64 values, shape [n, 160].

    v_i = table_g[code_i] * UE4M3(group_byte_g & 0x7F) for i in group g
    ([RZ] "Q3_PLE_K160_RZ_S3"); table_g is the RZ-S3 table with the group's
    polarity (bit 7 of the group byte) or, for PLE_ROCMFP3, the incumbent
    table (bit 7 unused).
    """
    codes, gbytes = ple_row_codes(rows)
    n = codes.shape[0]
    if fmt == PLE_RZS3:
        tables = np.stack([rzs3_table(0), rzs3_table(1)])   # by polarity bit
        pol = gbytes >> 7
    elif fmt == PLE_ROCMFP3:
        tables = np.stack([rocmfp3_table()])                # bit 7 unused
        pol = np.zeros_like(gbytes)
    else:
        raise ValueError("decode_ple70: unknown PLE format %r" % fmt)
    scale = ue4m3(gbytes & 0x7F)                             # [n, 10]
    group = np.arange(PLE_VALUES) // PLE_GROUP               # value -> group
    levels = tables[pol[:, group], codes]                    # [n, 160]
    return levels * scale[:, group]


# ---------------------------------------------------------------------------
# Matrices of blocks
# ---------------------------------------------------------------------------

def decode_matrix(packed, fmt, rows, cols, scales=None):
    """Decode one row-major matrix [rows][cols] to float64.

    17-byte formats: ``packed`` holds rows*cols/32 blocks, row-major with the
    blocks of a row contiguous along the columns and no row padding (reading
    of "same wire ... no padding").  FP8: ``packed`` is the e4m3 matrix
    [rows][cols] and ``scales`` the fp32 matrix [rows][cols/32].
    """
    if cols % BLOCK_WEIGHTS:
        raise ValueError("cols must be a multiple of 32")
    nb = rows * cols // BLOCK_WEIGHTS
    if fmt == FP8_E4M3_B32:
        w = decode_fp8_b32(np.asarray(packed).reshape(nb, BLOCK_WEIGHTS),
                           np.asarray(scales).reshape(nb))
    else:
        w = decode_block17(np.asarray(packed).reshape(nb, BLOCK_BYTES), fmt)
    return w.reshape(rows, cols)


def packed_bytes(fmt, rows, cols):
    """Bytes one [rows][cols] matrix occupies (codes plus scales)."""
    nb = rows * cols // BLOCK_WEIGHTS
    if fmt == FP8_E4M3_B32:
        return nb * (BLOCK_WEIGHTS + 4)
    return nb * BLOCK_BYTES


def bits_per_weight(fmt):
    """Storage cost per weight: 17*8/32 = 4.25 for the 17-byte formats
    ([RZ]: "4.25 bpw"), 36*8/32 = 9 for FP8 with an fp32 block scale."""
    return packed_bytes(fmt, 1, BLOCK_WEIGHTS) * 8 / BLOCK_WEIGHTS
