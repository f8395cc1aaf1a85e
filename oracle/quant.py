"""Block decoding by definition (float64).  Test infrastructure only.

Source: the "Engine and kernels" page, the paragraph under "What it runs"
(weights are GGUF Q4_0 or Q8_0 blocks of 32 weights plus one f16 scale) and
the "Reading weights" table (nibbles unpacked from u32 words and scaled; f16
scales; load-time repacking into separate nibble and scale arrays).  The byte
order inside a block is the public GGUF one:

* Q4_0 (18 B): bytes 0-1 the scale d as little-endian IEEE binary16; bytes
  2..17 = qs[0..15]; weight j = (qs[j] & 15) - 8 and weight j+16 =
  (qs[j] >> 4) - 8 for j = 0..15; value = weight * d.
* Q8_0 (34 B): bytes 0-1 the scale d; weight j = signed byte 2+j; value =
  weight * d.

Every f16 scale and every small integer is exactly representable in float64,
so `dequantize` is exact.
"""
from __future__ import annotations

import numpy as np

Q4_0 = 2
Q8_0 = 8
QK = 32
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34}


def f16_to_f64(lo_byte: np.ndarray, hi_byte: np.ndarray) -> np.ndarray:
    """Decode little-endian binary16 from its two bytes into float64, from the
    IEEE 754 field definition (sign 1, exponent 5 with bias 15, fraction 10;
    exponent 0 = subnormal, 31 = inf / NaN)."""
    bits = lo_byte.astype(np.int64) | (hi_byte.astype(np.int64) << 8)
    sign = np.where(bits >> 15, -1.0, 1.0)
    exp = (bits >> 10) & 0x1F
    frac = (bits & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + frac / 1024.0, (exp - 15).astype(np.int32))
    sub = np.ldexp(frac, -24)
    special = np.where(frac == 0, np.inf, np.nan)
    mag = np.where(exp == 0, sub, np.where(exp == 31, special, normal))
    return sign * mag


def decode_blocks(qtype: int, raw: np.ndarray):
    """raw: uint8 [..., block_bytes].  Returns (w int64 [..., 32], d float64 [...]),
    w being the signed weight integers of each block."""
    raw = np.asarray(raw, dtype=np.uint8)
    if raw.shape[-1] != BLOCK_BYTES[qtype]:
        raise ValueError("wrong block size")
    d = f16_to_f64(raw[..., 0], raw[..., 1])
    if qtype == Q4_0:
        qs = raw[..., 2:18].astype(np.int64)
        lo = (qs & 0x0F) - 8          # weights 0..15
        hi = (qs >> 4) - 8            # weights 16..31
        w = np.concatenate([lo, hi], axis=-1)
    elif qtype == Q8_0:
        w = raw[..., 2:34].view(np.int8).astype(np.int64)
    else:
        raise ValueError("unsupported qtype")
    return w, d


def dequantize(qtype: int, raw: np.ndarray) -> np.ndarray:
    """raw: uint8 [rows, cols/32, block_bytes] -> float64 [rows, cols], exact."""
    w, d = decode_blocks(qtype, raw)
    rows, nb = w.shape[0], w.shape[1]
    return (w.astype(np.float64) * d[..., None]).reshape(rows, nb * QK)


# --------------------------------------------------------------------------
# Byte image of the library's repacked ("tiled") layout, written out from its
# definition.  The pages only require separate weight and scale streams read
# as contiguous stripes; the tile geometry below is this library's choice
# and is defined in include/qgemm.h.
#
#   tile = 16 rows x 4 blocks (128 columns); NT = ceil(rows/16) row tiles,
#   KT = ceil(cols/128) column tiles, tile (rt, kt) has index t = rt*KT + kt.
#   Positions beyond rows/cols hold zero weights and a zero scale.
#   Q4_0 weights: 1024 B per tile.  16-byte chunk c = 16*s + r (s = 8-column
#     slice 0..3, r = row in tile) holds 4 little-endian u32 words; word j
#     covers block 4*kt + j, row 16*rt + r, columns 8*s + i (i = 0..7) of that
#     block; the unsigned nibble (weight + 8) of column i = 2*u sits at bits
#     4u..4u+3 and that of column i = 2*u + 1 at bits 16+4u..19+4u (u = 0..3).
#   Q8_0 weights: 2048 B per tile = two 1024-B halves h = 0, 1.  In half h,
#     chunk c = 16*s + r holds 8 bytes for block 4*kt + 2h then 8 bytes for
#     block 4*kt + 2h + 1; byte i is (weight of column 8*s + i) + 128.
#   Scales: 128 B per tile; the f16 scale of row 16*rt + r, block 4*kt + j is
#     at byte 8*r + 2*j.
# --------------------------------------------------------------------------
TILE_ROWS = 16
TILE_BLOCKS = 4
TILE_QS_BYTES = {Q4_0: 1024, Q8_0: 2048}
TILE_D_BYTES = 128


def packed_geometry(rows: int, cols: int):
    nt = -(-rows // TILE_ROWS)
    kt = -(-(cols // QK) // TILE_BLOCKS)
    return nt, kt


def packed_bytes(qtype: int, n_mat: int, rows: int, cols: int):
    nt, kt = packed_geometry(rows, cols)
    return n_mat * nt * kt * TILE_QS_BYTES[qtype], n_mat * nt * kt * TILE_D_BYTES


def repack_reference(qtype: int, raw: np.ndarray):
    """Byte image of the tiled layout for one or more matrices.

    raw: uint8 [n_mat, rows, cols/32, block_bytes] (or without the n_mat axis).
    Returns (qs uint8 [...], d uint8 [...]) flattened over all matrices.  Each
    weight is placed one at a time by the definition above (plain loops over
    positions, vectorised over tiles)."""
    raw = np.asarray(raw, dtype=np.uint8)
    if raw.ndim == 3:
        raw = raw[None]
    n_mat, rows, nb, _ = raw.shape
    w, _ = decode_blocks(qtype, raw)               # [m, rows, nb, 32] signed
    nt, kt = packed_geometry(rows, nb * QK)
    # pad to whole tiles with zero weights / zero scale bytes
    wp = np.zeros((n_mat, nt * TILE_ROWS, kt * TILE_BLOCKS, QK), dtype=np.int64)
    wp[:, :rows, :nb, :] = w
    dbytes = np.zeros((n_mat, nt * TILE_ROWS, kt * TILE_BLOCKS, 2), dtype=np.uint8)
    dbytes[:, :rows, :nb, :] = raw[..., 0:2]
    # view as [m, nt, 16 rows, kt, 4 blocks, 32]
    wt = wp.reshape(n_mat, nt, TILE_ROWS, kt, TILE_BLOCKS, QK)
    dt = dbytes.reshape(n_mat, nt, TILE_ROWS, kt, TILE_BLOCKS, 2)

    tq = TILE_QS_BYTES[qtype]
    qs = np.zeros((n_mat, nt, kt, tq), dtype=np.uint8)
    if qtype == Q4_0:
        for s in range(4):
            for r in range(TILE_ROWS):
                chunk = 16 * s + r
                for j in range(TILE_BLOCKS):
                    word = np.zeros((n_mat, nt, kt), dtype=np.int64)
                    for u in range(4):
                        nib_even = wt[:, :, r, :, j, 8 * s + 2 * u] + 8
                        nib_odd = wt[:, :, r, :, j, 8 * s + 2 * u + 1] + 8
                        word |= nib_even << (4 * u)
                        word |= nib_odd << (16 + 4 * u)
                    base = chunk * 16 + 4 * j
                    for byte in range(4):
                        qs[:, :, :, base + byte] = (word >> (8 * byte)) & 0xFF
    else:
        for h in range(2):
            for s in range(4):
                for r in range(TILE_ROWS):
                    chunk = 16 * s + r
                    for jj in range(2):
                        j = 2 * h + jj
                        for i in range(8):
                            off = h * 1024 + chunk * 16 + jj * 8 + i
                            qs[:, :, :, off] = (wt[:, :, r, :, j, 8 * s + i] + 128) & 0xFF
    d = np.zeros((n_mat, nt, kt, TILE_D_BYTES), dtype=np.uint8)
    for r in range(TILE_ROWS):
        for j in range(TILE_BLOCKS):
            d[:, :, :, 8 * r + 2 * j] = dt[:, :, r, :, j, 0]
            d[:, :, :, 8 * r + 2 * j + 1] = dt[:, :, r, :, j, 1]
    return qs.reshape(-1), d.reshape(-1)
