"""Load-time requantisation of other GGUF block types to Q8_0.  Test
infrastructure only (see the package header).

The pages say which tensors need it ("Engine and kernels", What it runs: a
few tensors of the public MoE file are Q4_1, Q5_0 or K-quants and are
requantized to Q8_0 on the way to the GPU; "Architecture", where the weights
live: such tensors are converted once and the result kept) but define
neither the formats nor the rounding; the block layouts here are the
public GGUF ones:

* Q4_1 (20 B): f16 d, f16 m, qs[16]; weight j = qs[j] & 15, weight j+16 =
  qs[j] >> 4 (j < 16); value = weight * d + m.
* Q5_0 (22 B): f16 d, qh (4 bytes, little-endian u32), qs[16]; weight j =
  (qs[j] & 15) | (bit j of qh) << 4, weight j+16 = (qs[j] >> 4) | (bit
  j+16 of qh) << 4; value = (weight - 16) * d.
* Q5_1 (24 B): f16 d, f16 m, qh, qs[16]; weights as Q5_0; value = weight *
  d + m.

K-quants hold a super-block of 256 values in eight sub-blocks of 32 (Q4_K,
Q5_K) or sixteen of 16 (Q6_K); each run of 32 values becomes one Q8_0
block, so one source block yields eight.

* Q4_K (144 B): f16 d, f16 dmin, scales[12], qs[128].  Sub-block j has a
  6-bit scale sc_j and a 6-bit min m_j packed in the 12 bytes: for j < 4,
  sc_j = low 6 bits of byte j and m_j = low 6 bits of byte j + 4; for j >=
  4, sc_j = low nibble of byte j + 4 plus the top 2 bits of byte j - 4 as
  bits 4-5, m_j = high nibble of byte j + 4 plus the top 2 bits of byte j as
  bits 4-5.  Bytes 32 c .. 32 c + 31 of qs hold sub-blocks 2 c (low
  nibbles) and 2 c + 1 (high nibbles), value i of the sub-block in byte i.
  value = (d * sc_j) * w - dmin * m_j.
* Q5_K (176 B): f16 d, f16 dmin, scales[12], qh[32], qs[128]; as Q4_K with
  a fifth bit: bit j of qh[i] is bit 4 of weight i of sub-block j.
* Q6_K (210 B): ql[128], qh[64], int8 scales[16], f16 d.  Value i (0..255)
  lies in half n = i // 128 at position p = i % 128, quarter k = p // 32,
  lane l = p % 32; its low 4 bits are the low (k < 2) or high (k >= 2)
  nibble of ql[64 n + 32 (k % 2) + l], its top 2 bits are bits 2 k, 2 k + 1
  of qh[32 n + l]; weight w in 0..63, value = (d * scales[i // 16]) * (w -
  32).

In float32: the products d * sc, dmin * m (11 by 6 bits) and (d * sc) * w
(17 by 5 bits) are exact, so a K-quant value of Q4_K / Q5_K is one rounding
of the difference, however it is grouped or fused; for Q6_K, d * sc is
exact (11 by 8 bits) and its product with w - 32 is rounded once.

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
Q4_K, Q5_K, Q6_K = 12, 13, 14
SRC_BLOCK_BYTES = {Q4_1: 20, Q5_0: 22, Q5_1: 24, Q4_K: 144, Q5_K: 176, Q6_K: 210}
SRC_BLOCK_VALUES = {Q4_1: 32, Q5_0: 32, Q5_1: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256}


def _f16(raw: np.ndarray, off: int) -> np.ndarray:
    return raw[..., off:off + 2].copy().view(np.float16)[..., 0].astype(np.float32)


def k_scales_mins(s12: np.ndarray):
    """The 12 packed scale bytes of a Q4_K / Q5_K block -> (sc, m), each
    int64 [nb, 8], 6 bits per sub-block."""
    s = np.asarray(s12, dtype=np.int64)
    lo, mid, hi = s[:, 0:4], s[:, 4:8], s[:, 8:12]
    sc = np.concatenate([lo & 63, (hi & 15) | ((lo >> 6) << 4)], axis=1)
    m = np.concatenate([mid & 63, (hi >> 4) | ((mid >> 6) << 4)], axis=1)
    return sc, m


def _k_weights_4bit(qs: np.ndarray) -> np.ndarray:
    """qs [nb, 128] -> weights [nb, 8, 32]: sub-block 2 c + h is nibble h of
    bytes 32 c .. 32 c + 31."""
    q = np.asarray(qs, dtype=np.int64).reshape(-1, 4, 32)
    return np.stack([q & 15, q >> 4], axis=2).reshape(-1, 8, 32)


def _decode_k(src_type: int, raw: np.ndarray) -> np.ndarray:
    d = _f16(raw, 0 if src_type != Q6_K else 208)[:, None]
    if src_type == Q6_K:
        ql = raw[:, 0:128].astype(np.int64).reshape(-1, 2, 2, 32)      # [half, k % 2, lane]
        qh = raw[:, 128:192].astype(np.int64).reshape(-1, 2, 1, 32)    # [half, -, lane]
        sc = raw[:, 192:208].view(np.int8).astype(np.float32)          # [nb, 16]
        low = np.concatenate([ql & 15, ql >> 4], axis=2)               # [half, k, lane]
        top = (qh >> (2 * np.arange(4)[None, None, :, None])) & 3      # [half, k, lane]
        w = (low | (top << 4)).reshape(-1, 256) - 32
        ds = (d * sc).astype(np.float32)                               # exact
        return (np.repeat(ds, 16, axis=1) * w.astype(np.float32)).astype(np.float32)
    dmin = _f16(raw, 2)[:, None]
    sc, m = k_scales_mins(raw[:, 4:16])
    if src_type == Q4_K:
        w = _k_weights_4bit(raw[:, 16:144])
    else:
        qh = raw[:, 16:48].astype(np.int64)                            # [nb, 32]
        hb = (qh[:, None, :] >> np.arange(8)[None, :, None]) & 1       # [nb, 8, 32]
        w = _k_weights_4bit(raw[:, 48:176]) | (hb << 4)
    d1 = (d * sc.astype(np.float32)).astype(np.float32)                # exact
    m1 = (dmin * m.astype(np.float32)).astype(np.float32)              # exact
    v = (d1[:, :, None] * w.astype(np.float32)).astype(np.float32)     # exact
    return (v - m1[:, :, None]).astype(np.float32).reshape(-1, 256)


def decode_values_f32(src_type: int, raw: np.ndarray) -> np.ndarray:
    """raw: uint8 [nb, block_bytes] -> float32 [nb, values per block]."""
    raw = np.asarray(raw, dtype=np.uint8)
    if raw.shape[-1] != SRC_BLOCK_BYTES[src_type]:
        raise ValueError("wrong block size")
    if src_type in (Q4_K, Q5_K, Q6_K):
        return _decode_k(src_type, raw)
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
    """Source blocks [nb, block_bytes] -> Q8_0 blocks [nb * values / 32,
    34], each run of 32 values in order one block."""
    return quantize_q8_0(decode_values_f32(src_type, raw).reshape(-1, 32))


__all__ = ["Q4_1", "Q5_0", "Q5_1", "Q4_K", "Q5_K", "Q6_K", "Q8_0", "SRC_BLOCK_BYTES", "SRC_BLOCK_VALUES",
           "decode_values_f32", "k_scales_mins", "round_half_away", "quantize_q8_0", "requant_q8_0"]
