"""The products the library computes, by definition, in float64.

Test infrastructure only.  Each function names the passage it follows:
"Engine and kernels" (the Pooled engine page) and "Architecture" (the Pooled
architecture page), plus the MoE layout paragraph of "A 235B model in a
browser window".

Float tolerance (the stated parity bar): for an output element that is a sum
of products w_i * x_i,  |gpu - ref| <= 2e-3 * sum_i |w_i x_i| + 1e-5.  Derived
outputs (SiLU-gated h, down projections of h, the MoE output) carry that
bound through their formula; see `tol_*` below.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .quant import dequantize, Q4_0, Q8_0, QK  # noqa: F401

REL_TOL = 2e-3
ABS_TOL = 1e-5
U32 = 2.0 ** -24          # unit roundoff of binary32
U16 = 2.0 ** -11          # unit roundoff of binary16 (activation operand rounding)
SILU_SLOPE_MAX = 1.09984  # max |d/dg g*sigmoid(g)| = 1.099839..., attained near g = 2.3994


def _row_chunks(rows: int, cols: int, budget: int = 1 << 24):
    step = max(1, budget // max(cols, 1))
    for r0 in range(0, rows, step):
        yield r0, min(rows, r0 + step)


# --------------------------------------------------------------------------
# GEMV / GEMM: y = (y_in) + W x.  "Engine and kernels": cooperative GEMV for
# decode, batched GEMV twins for verify, the 16-column prefill GEMM; all read
# packed blocks and accumulate in f32 ("No f16 accumulation").  The
# accumulate form y += W.x is the "Fewer passes" table's residual epilogue.
# --------------------------------------------------------------------------
def gemv(qtype: int, raw: np.ndarray, x: np.ndarray,
         y_in: Optional[np.ndarray] = None, rows: Optional[np.ndarray] = None):
    """raw: uint8 [R, K/32, B]; x: [K] or [K, C] (any float).  Returns
    (y float64 [R', C], a float64 [R', C]) with a = sum |w x| (the tolerance
    scale), y = y_in + W x when y_in is given.  `rows` selects a subset of
    rows (sampled outputs of a large matrix)."""
    x = np.asarray(x, dtype=np.float64)
    vec = x.ndim == 1
    if vec:
        x = x[:, None]
    if rows is not None:
        raw = raw[np.asarray(rows)]
    nrows, nb = raw.shape[0], raw.shape[1]
    if nb * QK != x.shape[0]:
        raise ValueError("shape mismatch")
    y = np.empty((nrows, x.shape[1]))
    a = np.empty_like(y)
    ax = np.abs(x)
    for r0, r1 in _row_chunks(nrows, nb * QK):
        w = dequantize(qtype, raw[r0:r1])
        y[r0:r1] = w @ x
        a[r0:r1] = np.abs(w) @ ax
    if y_in is not None:
        yi = np.asarray(y_in, dtype=np.float64).reshape(y.shape)
        y = yi + y
    if vec:
        return y[:, 0], a[:, 0]
    return y, a


def tol_dot(a: np.ndarray, y: Optional[np.ndarray] = None) -> np.ndarray:
    """Parity bound for a plain product (and its final f32 rounding)."""
    t = REL_TOL * a + ABS_TOL
    if y is not None:
        t = t + 2 * U32 * np.abs(y)
    return t


# --------------------------------------------------------------------------
# Fused gate/up.  "Engine and kernels", kernel families: both FFN projections
# in one sweep, SiLU applied before writing.  The gated MLP passes one
# projection through SiLU and gates the other (the Three.js page, SmolLM2
# section); the gate matrix "drives a switch" on the up output (the 235B
# page).  Reading: h = silu(Wg x) * (Wu x), silu(g) = g / (1 + exp(-g)).
# --------------------------------------------------------------------------
def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    # g / (1 + e^-g), evaluated without overflow for very negative g
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = g[pos] / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = g[~pos] * e / (1.0 + e)
    return out


# --------------------------------------------------------------------------
# RMSNorm.  "Running LLMs in the browser with Three.js", the Llama-style
# differences (RMSNorm: the root mean square, no mean subtracted) and
# "Architecture", one token end to end (the final RMSNorm before the head);
# "Engine and kernels", the norm fused into the router (kept) and into the
# GEMV (measured slower on Metal).  Reading: n(x)[k] = x[k] * gamma[k] /
# sqrt(mean_k x[k]^2 + eps) per column, eps given by the caller.
# --------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x: [K] or [K, C]; gamma: [K].  float64."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    ms = np.mean(x * x, axis=0)
    inv = 1.0 / np.sqrt(ms + float(eps))
    return (x * inv) * (g if x.ndim == 1 else g[:, None])


def gateup_silu(qtype: int, g_raw: np.ndarray, u_raw: np.ndarray, x: np.ndarray):
    """Returns (h, tol_h, g, u) float64, shapes [F] or [F, C]."""
    g, ag = gemv(qtype, g_raw, x)
    u, au = gemv(qtype, u_raw, x)
    h = silu(g) * u
    tg = tol_dot(ag)
    tu = tol_dot(au)
    th = (1.1 * tg * (np.abs(u) + tu) + np.abs(silu(g)) * tu
          + 4 * U32 * np.abs(h) + ABS_TOL)
    return h, th, g, u


def down_tol(qtype: int, d_raw: np.ndarray, h: np.ndarray, tol_h: np.ndarray):
    """Bound for W_d h when h itself carries error <= tol_h (elementwise)."""
    h = np.asarray(h, dtype=np.float64)
    vec = h.ndim == 1
    hh = h[:, None] if vec else h
    th = tol_h[:, None] if vec else tol_h
    out = np.empty((d_raw.shape[0], hh.shape[1]))
    for r0, r1 in _row_chunks(d_raw.shape[0], hh.shape[0]):
        aw = np.abs(dequantize(qtype, d_raw[r0:r1]))
        out[r0:r1] = REL_TOL * (aw @ np.abs(hh)) + aw @ th + ABS_TOL
    return out[:, 0] if vec else out


# --------------------------------------------------------------------------
# LM head + greedy argmax.  "Architecture", one token end to end (the head
# runs over all 248,320 rows; greedy sampling on the GPU) and "Engine and
# kernels", Fewer passes (lowest-index tie-breaking matches the CPU loop);
# Speculation table (drafts use a prefix of the vocabulary rows).
# --------------------------------------------------------------------------
def argmax_first(v: np.ndarray) -> int:
    """The CPU loop: keep the first strictly greater value."""
    v = np.asarray(v)
    # vectorised form of the loop (pinned against the loop in the tests)
    return int(np.flatnonzero(v == np.max(v))[0])


def argmax_certified(logits: np.ndarray, a: np.ndarray, k_terms: int,
                     eps_op: float) -> bool:
    """True when every computation of the logits whose per-row error stays
    within (gamma_K + eps_op) * a_r must give the same argmax.  gamma_K is the
    classical bound K u / (1 - K u) for f32 summation of K products in any
    order; eps_op covers rounding the activation operand (0 or 2^-11)."""
    gam = k_terms * U32 / (1 - k_terms * U32)
    bound = (gam + eps_op * (1 + gam)) * a
    i = argmax_first(logits)
    others = np.ones(len(logits), dtype=bool)
    others[i] = False
    if not others.any():
        return True
    margin = logits[i] - bound[i] - (logits[others] + bound[others])
    return bool(np.all(margin > 0))


# --------------------------------------------------------------------------
# Router top-k.  "Engine and kernels", kernel families: router, top-k,
# expert gate/up and down and the weighted combine all on the GPU; the same
# lowest-index rule for ties as the argmax.  Readings: order by (value
# descending, index ascending); weights = softmax over the k selected logits
# (normalize=True) or the full softmax evaluated at the selected experts.
# --------------------------------------------------------------------------
def topk_lowest_index(logits: np.ndarray, k: int) -> np.ndarray:
    logits = np.asarray(logits)
    idx = np.arange(len(logits))
    order = np.lexsort((idx, -logits))      # primary: -value, secondary: index
    return order[:k]


def softmax(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    e = np.exp(v - np.max(v))
    return e / np.sum(e)


def topk_certified(logits: np.ndarray, a: np.ndarray, k: int, k_terms: int,
                   eps_op: float = 0.0, order: bool = False) -> bool:
    """Set of the top k is forced by the error bound (and, with order=True,
    also the order inside it)."""
    gam = k_terms * U32 / (1 - k_terms * U32)
    bound = (gam + eps_op * (1 + gam)) * a
    sel = topk_lowest_index(logits, len(logits))
    lo = logits[sel] - bound[sel]
    hi = logits[sel] + bound[sel]
    if k < len(logits) and not (np.min(lo[:k]) > np.max(hi[k:])):
        return False
    if order:
        for i in range(k - 1):
            if not lo[i] > hi[i + 1]:
                return False
    return True


# --------------------------------------------------------------------------
# LM head + top-k candidates.  "Architecture", one token end to end (greedy
# and top-k sampling on the GPU, a few bytes read back instead of the 1 MB
# logits); "Engine and kernels", Sampling and Fewer passes (GPU top-k, the
# CPU loop's lowest-index ties); "Running LLMs in the browser with Three.js",
# Reduce sampling on the GPU (a small top-k reduction on the GPU, the host
# finishes the draw from the candidates).  Reading: the candidates are the k
# largest logits over rows < n_rows, ordered by (value descending, index
# ascending); k is small (the Three.js example asks for 10).
# --------------------------------------------------------------------------
def lmhead_topk(qtype: int, raw: np.ndarray, x: np.ndarray, n_rows: int, k: int):
    """raw: uint8 [R, K/32, B]; x: [K].  Returns (idx int64 [k], val float64
    [k], logits float64 [n_rows], a [n_rows]) with a = |W| |x| the scale of the
    logits' rounding error."""
    logits, a = gemv(qtype, raw[:n_rows], x)
    idx = topk_lowest_index(logits, k)
    return idx, logits[idx], logits, a


# --------------------------------------------------------------------------
# MoE FFN.  "Engine and kernels": the MoE model's FFN is 256 experts (8 active
# per token) plus a shared expert; router, top-k, expert gate/up and down and
# the weighted combine on the GPU.  "A 235B model in a browser window": each
# expert is a gated FFN of three matrices, stored stacked by role (all gate
# matrices in one tensor, all up in a second, all down in a third).
# Readings: shared expert ungated (weight 1); the result accumulates into
# the residual y like the FFN down projection.
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, router: np.ndarray):
    """Router scores l = R x (f32 router weights, [E, H]) for x [H] or [H, T],
    and a = |R| |x|, the scale of their rounding error."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[:, None]
    R = np.asarray(router, dtype=np.float64)
    return R @ x, np.abs(R) @ np.abs(x)


def routing_certified(logits: np.ndarray, la: np.ndarray, top_k: int, hidden: int,
                      order: bool = False) -> np.ndarray:
    """Per token: is the selected set (and, with order=True, its order) forced
    by the error bound of an f32 router product of `hidden` terms?"""
    return np.array([topk_certified(logits[:, t], la[:, t], top_k, hidden + 2, order=order)
                     for t in range(logits.shape[1])])


def moe_router(x: np.ndarray, router: np.ndarray, norm_w: Optional[np.ndarray] = None,
               norm_eps: float = 0.0):
    """The input the router and the experts read (x [H, T], or RMSNorm(x)
    with weights norm_w), the router's logits [E, T] and their rounding-error
    scale, as moe_ffn takes them."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[:, None]
    H = x.shape[0]
    if norm_w is not None:
        x = rmsnorm(x, norm_w, norm_eps)
    logits, la = router_logits(x, router)       # [E, T]
    if norm_w is not None:
        # the norm's 1 / rms in f32 (sum of H squares, square root, division)
        # scales every logit of a token: relative error (H + 8) u32 more
        gam = (H + 2) * U32 / (1 - (H + 2) * U32)
        la = la + (H + 8) * U32 / gam * np.abs(logits)
    return x, logits, la


def moe_ffn(x: np.ndarray, router: np.ndarray, qtype: int,
            gate_raw: np.ndarray, up_raw: np.ndarray, down_raw: np.ndarray,
            top_k: int, normalize: bool = True,
            sh_gate: Optional[np.ndarray] = None, sh_up: Optional[np.ndarray] = None,
            sh_down: Optional[np.ndarray] = None,
            y_in: Optional[np.ndarray] = None,
            norm_w: Optional[np.ndarray] = None, norm_eps: float = 0.0):
    """x: [H, T]; router: [E, H] f32; gate/up raw: [E, F, H/32, B];
    down raw: [E, H, F/32, B]; y_in: [H, T] or None.  norm_w: with it, the
    router and every expert read RMSNorm(x) (weights norm_w, eps norm_eps)
    instead of x ("Engine and kernels": the norm fused ahead of the router);
    the residual y is not normalised.

    Returns dict with y [H, T], tol [H, T], idx [T, k], p [T, k],
    logits [E, T], logit_a [E, T]."""
    x, logits, la = moe_router(x, router, norm_w, norm_eps)
    H, T = x.shape
    gam = (H + 2) * U32 / (1 - (H + 2) * U32)
    y = np.zeros((H, T)) if y_in is None else np.asarray(y_in, dtype=np.float64).reshape(H, T).copy()
    tol = np.full((H, T), ABS_TOL)
    idx = np.zeros((T, top_k), dtype=np.int64)
    pw = np.zeros((T, top_k))
    for t in range(T):
        sel = topk_lowest_index(logits[:, t], top_k)
        idx[t] = sel
        if normalize:
            p = softmax(logits[sel, t])
        else:
            p = softmax(logits[:, t])[sel]
        pw[t] = p
        # softmax moves by at most 2 p_k max|dl| for logit errors dl (any
        # order of f32 summation of the router GEMV), plus its own rounding
        dl = gam * np.max(la[sel if normalize else slice(None), t])
        dp = p * (np.expm1(2 * dl)) + 8 * U32
        xt = x[:, t]
        for k, e in enumerate(sel):
            h, th, _, _ = gateup_silu(qtype, gate_raw[e], up_raw[e], xt)
            z, az = gemv(qtype, down_raw[e], h)
            tz = down_tol(qtype, down_raw[e], h, th)
            y[:, t] += p[k] * z
            tol[:, t] += dp[k] * np.abs(z) + (p[k] + dp[k]) * tz
        if sh_gate is not None:
            h, th, _, _ = gateup_silu(qtype, sh_gate, sh_up, xt)
            z, _ = gemv(qtype, sh_down, h)
            y[:, t] += z
            tol[:, t] += down_tol(qtype, sh_down, h, th)
    tol += 4 * U32 * np.abs(y)
    return {"y": y, "tol": tol, "idx": idx, "p": pw, "logits": logits, "logit_a": la}


def moe_routing_certified(res: dict, top_k: int, hidden: int) -> bool:
    return bool(np.all(routing_certified(res["logits"], res["logit_a"], top_k, hidden)))


def silu_slope_bound_holds() -> bool:
    g = np.linspace(-20, 20, 400001)
    s = 1.0 / (1.0 + np.exp(-g))
    slope = s * (1 + g * (1 - s))
    return float(np.max(np.abs(slope))) <= SILU_SLOPE_MAX


def gamma(k: int) -> float:
    return k * U32 / (1 - k * U32)


__all__ = [
    "gemv", "tol_dot", "silu", "gateup_silu", "down_tol", "argmax_first",
    "argmax_certified", "topk_lowest_index", "softmax", "topk_certified",
    "router_logits", "routing_certified", "moe_router", "moe_ffn", "moe_routing_certified", "gamma",
]
