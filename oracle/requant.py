"""Load-time requantisation of other GGUF block types to Q8_0.  Test
infrastructure only (see the package header).

The pages say which tensors need it ("Engine and kernels", What it runs: a
few tensors of the public MoE file are Q4_1, Q5_0 or K-quants and are
requantized to Q8_0 on the way to the GPU; "Architecture", where the weights
live: such tensors are converted once and the result kept) but define
neither the formats nor the rounding; the block layouts here are the
public GGUF ones (K-quants are not covered):

* Q4_1 (20 B): f16 d, f16 m, qs[16]; weight j = qs[j] & 15, weight j+16 =
  qs[j] >> 4 (j < 16); value = weight * d + m.
* Q5_0 (22 B): f16 d, qh (4 bytes, little-endian u32), qs[16]; weight j =
  (qs[j] & 15) | (bit j of qh) << 4, weight j+16 = (qs[j] >> 4) | (bit
  j+16 of qh) << 4; value = (weight - 16) * d.
* Q5_1 (24 B): f16 d, f16 m, qh, qs[16]; weights as Q5_0; value = weight *
  d + m.

Requantisation of one block of values v (float32): amax = max |v|; d =
amax / 127 (float32); id = 1 / d, 0 when d is 0; q_j = v_j * id rounded to
the nearest integer, halves away from zero; the block stores d as binary16
(nearest, ties to even) and the q_j as signed bytes.  Every step is a
float32 operation, each rounded once, in this order (values: weight * d
rounded, then + m rounded), so the bytes are a function of the input
bytes alone.
"""
from __future__ import annotations

import numpy as np

from .quant import Q8_0

Q4_1, Q5_0, Q5_1 = 3, 6, 7
SRC_BLOCK_BYTES = {Q4_1: 20, Q5_0: 22, Q5_1: 24}


def _f16(raw: np.ndarray, off: int) -> np.ndarray:
    return raw[..., off:off + 2].copy().view(np.float16)[..., 0].astype(np.float32)


def decode_values_f32(src_type: int, raw: np.ndarray) -> np.ndarray:
    """raw: uint8 [nb, block_bytes] -> float32 [nb, 32] block values."""
    raw = np.asarray(raw, dtype=np.uint8)
    if raw.shape[-1] != SRC_BLOCK_BYTES[src_type]:
        raise ValueError("wrong block size")
    d = _f16(raw, 0)[:, None]
    if src_type == Q4_1:
        m = _f16(raw, 2)[:, None]
        qs = raw[:, 4:20].astype(np.int64)
        w = np.concatenate([qs & 15, qs >> 4], axis=1)
        return (w.astype(np.float32) * d).astype(np.float32) + m
    qh_off, qs_off = (2, 6) if src_type == Q5_0 else (4, 8)
    qh = raw[:, qh_off:qh_off + 4].copy().view("<u4")[:, 0].astype(np.int64)
    qs = raw[:, qs_off:qs_off + 16].astype(np.int64)
    j = np.arange(16)
    hi_lo = (qh[:, None] >> j) & 1           # bits 0..15 -> weights 0..15
    hi_hi = (qh[:, None] >> (j + 16)) & 1    # bits 16..31 -> weights 16..31
    w = np.concatenate([(qs & 15) | (hi_lo << 4), (qs >> 4) | (hi_hi << 4)], axis=1)
    if src_type == Q5_0:
        return ((w - 16).astype(np.float32) * d).astype(np.float32)
    m = _f16(raw, 2)[:, None]
    return (w.astype(np.float32) * d).astype(np.float32) + m


def round_half_away(x: np.ndarray) -> np.ndarray:
    """Nearest integer, halves away from zero (in float64, where |x| + 0.5
    is exact for every float32 x)."""
    x = np.asarray(x, dtype=np.float64)
    return np.sign(x) * np.floor(np.abs(x) + 0.5)


def quantize_q8_0(v: np.ndarray) -> np.ndarray:
    """float32 values [nb, 32] -> canonical Q8_0 bytes [nb, 34]."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        idv = np.where(d != 0, (np.float32(1.0) / d).astype(np.float32), np.float32(0.0)).astype(np.float32)
    x = (v * idv[:, None]).astype(np.float32)
    q = round_half_away(x).astype(np.int64)
    out = np.zeros((v.shape[0], 34), dtype=np.uint8)
    out[:, 0:2] = d.astype(np.float16).view(np.uint8).reshape(-1, 2)
    out[:, 2:34] = q.astype(np.int8).view(np.uint8)
    return out


def requant_q8_0(src_type: int, raw: np.ndarray) -> np.ndarray:
    """Source blocks [nb, block_bytes] -> Q8_0 blocks [nb, 34]."""
    return quantize_q8_0(decode_values_f32(src_type, raw))


__all__ = ["Q4_1", "Q5_0", "Q5_1", "Q8_0", "SRC_BLOCK_BYTES", "decode_values_f32", "round_half_away",
           "quantize_q8_0", "requant_q8_0"]
