"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and writes them out in the GGUF Q4_0 / Q8_0
block byte format, and nothing else: it holds no dequantisation, no product,
no reduction.  Both the CPU oracle and the GPU path receive the same bytes and
decode them independently.

Block formats (the pages: "Engine and kernels", the paragraph under "What it
runs": GGUF Q4_0 / Q8_0 blocks of 32 weights plus one f16 scale; the byte
order is the public GGUF one):

* Q4_0, 18 bytes: little-endian f16 scale, then 16 bytes whose low nibbles are
  weights 0..15 and whose high nibbles are weights 16..31, each stored as the
  unsigned value (weight + 8).
* Q8_0, 34 bytes: little-endian f16 scale, then 32 signed int8 weights.

Distributions follow the workloads on the pages' models (hidden 5120 / 2048,
vocabulary 248,320, 256 experts with 8 active): unsigned nibbles uniform in
0..15, int8 uniform in -127..127, scales |N(0, sigma)| rounded to f16 by
round-to-nearest-even (numpy's float16 cast), activations f32 N(0, 1).
Every stream is `numpy.random.default_rng([cfg_id, tensor_id])` (PCG64).
"""
from __future__ import annotations

import numpy as np

Q4_0 = 2
Q8_0 = 8
QK = 32
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34}

# cfg ids used by the tests and the bench
CFG_GEMV = 1
CFG_FFN = 2
CFG_VERIFY = 3
CFG_PREFILL = 4
CFG_MOE = 5


def rng(cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([int(cfg_id), int(tensor_id)])


def _scales(g: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return np.abs(g.normal(0.0, sigma, size=shape)).astype(np.float16)


def pack_q4_0(nibbles: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Write GGUF Q4_0 bytes.  nibbles: uint8 [..., 32] in 0..15 (weight + 8);
    d: float16 [...].  Returns uint8 [..., 18]."""
    nibbles = np.asarray(nibbles, dtype=np.uint8)
    d = np.asarray(d, dtype=np.float16)
    out = np.empty(nibbles.shape[:-1] + (18,), dtype=np.uint8)
    out[..., 0:2] = d[..., None].view(np.uint8).reshape(d.shape + (2,))
    out[..., 2:18] = (nibbles[..., 0:16] & 0xF) | ((nibbles[..., 16:32] & 0xF) << 4)
    return out


def pack_q8_0(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Write GGUF Q8_0 bytes.  q: int8 [..., 32]; d: float16 [...]."""
    q = np.asarray(q, dtype=np.int8)
    d = np.asarray(d, dtype=np.float16)
    out = np.empty(q.shape[:-1] + (34,), dtype=np.uint8)
    out[..., 0:2] = d[..., None].view(np.uint8).reshape(d.shape + (2,))
    out[..., 2:34] = q.view(np.uint8)
    return out


def gen_weights(qtype: int, rows: int, cols: int, sigma: float,
                g: np.random.Generator) -> np.ndarray:
    """GGUF block bytes for a rows x cols matrix, uint8 [rows, cols/32, bytes].

    Draw order: weight integers, then scales, then packing."""
    if cols % QK:
        raise ValueError("cols must be a multiple of 32")
    nb = cols // QK
    if qtype == Q4_0:
        nib = g.integers(0, 16, size=(rows, nb, QK), dtype=np.uint8)
        d = _scales(g, (rows, nb), sigma)
        return pack_q4_0(nib, d)
    if qtype == Q8_0:
        q = g.integers(-127, 128, size=(rows, nb, QK), dtype=np.int8)
        d = _scales(g, (rows, nb), sigma)
        return pack_q8_0(q, d)
    raise ValueError(f"unsupported qtype {qtype}")


def flip_scale_signs(raw: np.ndarray, g: np.random.Generator, p: float = 0.5) -> np.ndarray:
    """A copy of GGUF Q4_0 / Q8_0 blocks (uint8 [..., bytes]) with the sign bit
    of each block's f16 scale (bit 7 of byte 1) set with probability p.  The
    block definition allows any f16 scale; real files carry both signs."""
    out = np.array(raw, dtype=np.uint8, copy=True)
    out[..., 1] |= (g.random(out.shape[:-1]) < p).astype(np.uint8) << 7
    return out


def plant_q8_min(raw: np.ndarray, g: np.random.Generator, p: float) -> np.ndarray:
    """A copy of GGUF Q8_0 blocks (uint8 [..., 34]) with each weight byte set
    to 0x80 (int8 -128, a valid weight the uniform draw never makes) with
    probability p."""
    out = np.array(raw, dtype=np.uint8, copy=True)
    w = out[..., 2:34]
    w[g.random(w.shape) < p] = 0x80
    return out


def gen_x(cols: int, ncols: int, cfg_id: int, col0: int = 0) -> np.ndarray:
    """Activations, f32 [cols, ncols]; column j comes from rng(cfg_id, 100 + col0 + j)."""
    x = np.empty((cols, ncols), dtype=np.float32)
    for j in range(ncols):
        x[:, j] = rng(cfg_id, 100 + col0 + j).standard_normal(cols).astype(np.float32)
    return x


def gen_f32(shape, sigma: float, g: np.random.Generator) -> np.ndarray:
    return (g.standard_normal(size=shape) * sigma).astype(np.float32)


def tensor_ids():
    """Stable tensor ids inside one cfg (weights < 100, activations >= 100)."""
    return {
        "w": 1, "gate": 2, "up": 3, "down": 4, "w_q8": 5, "w_q4": 6,
        "router": 10, "moe_gate": 11, "moe_up": 12, "moe_down": 13,
        "sh_gate": 14, "sh_up": 15, "sh_down": 16, "y_in": 90,
    }
