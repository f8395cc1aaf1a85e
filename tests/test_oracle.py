"""Pins for the CPU oracle: hand-worked blocks, exact rational brute force,
closed forms, library special cases and invariants.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import synth
from oracle import ops, quant
from tests.conftest import golden

Q4, Q8 = quant.Q4_0, quant.Q8_0


def _block(name):
    g = golden(name)
    raw = np.array([int(b, 16) for b in g["bytes"].split()], dtype=np.uint8)
    return raw, g


# ---------------------------------------------------------------- f16 decode
def test_f16_decode_matches_worked_values():
    g = golden("f16_values.txt")
    for bits, val in g.items():
        b = int(bits, 16)
        got = quant.f16_to_f64(np.array([b & 0xFF], np.uint8), np.array([b >> 8], np.uint8))[0]
        assert got == float(val), bits
        if bits == "8000":
            assert np.signbit(got)


def test_f16_decode_agrees_with_numpy_for_all_finite_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = quant.f16_to_f64((bits & 0xFF).astype(np.uint8), (bits >> 8).astype(np.uint8))
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


# ---------------------------------------------------------- hand-worked blocks
@pytest.mark.parametrize("name,qtype", [("q4_0_block.txt", Q4), ("q8_0_block.txt", Q8),
                                        ("q4_0_block_neg_scale.txt", Q4), ("q8_0_block_min.txt", Q8)])
def test_hand_worked_block(name, qtype):
    raw, g = _block(name)
    raw = raw.reshape(1, 1, -1)
    for key, val in g.items():
        if key == "bytes":
            continue
        x = np.zeros(32)
        if key == "ones":
            x[:] = 1.0
        else:
            x[int(key[1:])] = 1.0
        y, _ = ops.gemv(qtype, raw, x)
        assert y[0] == float(val), key


def test_special_cases():
    # all nibbles 8 -> exactly 0 for any scale
    nib = np.full((3, 2, 32), 8, np.uint8)
    d = np.array([[1.5, 2.0 ** -24], [65504.0, 0.0], [0.02, 3.0]], np.float16)
    raw = synth.pack_q4_0(nib, d)
    x = np.random.default_rng(0).standard_normal((64, 3))
    y, _ = ops.gemv(Q4, raw, x)
    assert np.all(y == 0)
    # zero scale -> 0
    nib = np.random.default_rng(1).integers(0, 16, (2, 2, 32)).astype(np.uint8)
    raw = synth.pack_q4_0(nib, np.zeros((2, 2), np.float16))
    y, a = ops.gemv(Q4, raw, x[:, :1])
    assert np.all(y == 0) and np.all(a == 0)
    # smallest subnormal scale, q = 15 (weight 7), x = 1 -> 7 * 2^-24
    nib = np.full((1, 1, 32), 8, np.uint8)
    nib[0, 0, 5] = 15
    raw = synth.pack_q4_0(nib, np.array([[2.0 ** -24]], np.float16))
    y, _ = ops.gemv(Q4, raw, np.ones(32))
    assert y[0] == 7 * 2.0 ** -24


# ---------------------------------------------------- exact rational brute force
def _exact(ints, scales, x):
    """ints [R, nb, 32] python ints, scales float16 [R, nb], x float32 [K, C]."""
    R, nb, _ = ints.shape
    C = x.shape[1]
    out = [[Fraction(0)] * C for _ in range(R)]
    for r in range(R):
        for b in range(nb):
            d = Fraction(float(scales[r, b]))
            for j in range(32):
                w = int(ints[r, b, j]) * d
                for c in range(C):
                    out[r][c] += w * Fraction(float(x[b * 32 + j, c]))
    return out


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("R,K", [(1, 32), (3, 64), (5, 96)])
def test_exact_brute_force(qtype, R, K):
    g = np.random.default_rng([qtype, R, K])
    nb = K // 32
    scales = np.abs(g.normal(0, 0.05, (R, nb))).astype(np.float16)
    scales[0, 0] = np.float16(2.0 ** -20)       # a subnormal scale
    x = g.standard_normal((K, 2)).astype(np.float32)
    if qtype == Q4:
        nib = g.integers(0, 16, (R, nb, 32)).astype(np.uint8)
        raw = synth.pack_q4_0(nib, scales)
        ints = nib.astype(np.int64) - 8
    else:
        q = g.integers(-127, 128, (R, nb, 32)).astype(np.int8)
        raw = synth.pack_q8_0(q, scales)
        ints = q.astype(np.int64)
    ex = _exact(ints, scales, x)
    y, a = ops.gemv(qtype, raw, x)
    for r in range(R):
        for c in range(2):
            err = abs(Fraction(float(y[r, c])) - ex[r][c])
            assert err <= Fraction(K * 2.0 ** -53) * Fraction(float(a[r, c])) + Fraction(1, 10 ** 300)
    # accumulate form: y_in + W x
    y_in = g.standard_normal((R, 2)).astype(np.float32)
    y2, _ = ops.gemv(qtype, raw, x, y_in=y_in)
    for r in range(R):
        for c in range(2):
            want = ex[r][c] + Fraction(float(y_in[r, c]))
            assert abs(Fraction(float(y2[r, c])) - want) <= Fraction(4 * K * 2.0 ** -53) * (
                Fraction(float(a[r, c])) + abs(Fraction(float(y_in[r, c])))) + Fraction(1, 10 ** 300)


# ------------------------------------------------------------------ invariants
def test_linearity_exact():
    g = np.random.default_rng(7)
    raw = synth.gen_weights(Q4, 6, 128, 0.02, g)
    x1 = g.integers(-3, 4, 128).astype(np.float64)
    x2 = g.integers(-3, 4, 128).astype(np.float64)
    y1, _ = ops.gemv(Q4, raw, x1)
    y2, _ = ops.gemv(Q4, raw, x2)
    y12, _ = ops.gemv(Q4, raw, 0.5 * x1 + 4.0 * x2)
    assert np.array_equal(y12, 0.5 * y1 + 4.0 * y2)


def test_row_permutation_commutes():
    g = np.random.default_rng(8)
    raw = synth.gen_weights(Q8, 9, 64, 0.005, g)
    x = g.standard_normal(64)
    perm = g.permutation(9)
    y, a = ops.gemv(Q8, raw, x)
    yp, _ = ops.gemv(Q8, raw[perm], x)
    # BLAS may block rows differently; equal up to f64 summation error
    assert np.all(np.abs(yp - y[perm]) <= 64 * 2.0 ** -52 * a[perm])


def test_q4_q8_reencoding_identical():
    g = np.random.default_rng(9)
    nib = g.integers(0, 16, (7, 3, 32)).astype(np.uint8)
    d = np.abs(g.normal(0, 0.02, (7, 3))).astype(np.float16)
    r4 = synth.pack_q4_0(nib, d)
    r8 = synth.pack_q8_0(nib.astype(np.int16) - 8, d)
    x = g.standard_normal((96, 4))
    assert np.array_equal(ops.gemv(Q4, r4, x)[0], ops.gemv(Q8, r8, x)[0])


def test_columns_equal_single_column():
    g = np.random.default_rng(10)
    raw = synth.gen_weights(Q4, 5, 64, 0.02, g)
    X = g.standard_normal((64, 16))
    Y, _ = ops.gemv(Q4, raw, X)
    for j in range(16):
        assert np.allclose(Y[:, j], ops.gemv(Q4, raw, X[:, j])[0], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------- SiLU
def test_silu_closed_forms():
    g = np.linspace(-30, 30, 1201)
    s = ops.silu(g)
    assert ops.silu(np.array([0.0]))[0] == 0.0
    assert np.max(np.abs((s - ops.silu(-g)) - g)) < 1e-13       # silu(g) - silu(-g) = g
    assert np.allclose(s, g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    assert abs(ops.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert -1e-12 < ops.silu(np.array([-40.0]))[0] < 0
    assert ops.silu_slope_bound_holds()


def test_gateup_tolerance_covers_perturbations():
    g = np.random.default_rng(11)
    gr = synth.gen_weights(Q4, 64, 256, 0.02, g)
    ur = synth.gen_weights(Q4, 64, 256, 0.02, g)
    x = g.standard_normal(256)
    h, th, gg, uu = ops.gateup_silu(Q4, gr, ur, x)
    tg = ops.tol_dot(ops.gemv(Q4, gr, x)[1])
    tu = ops.tol_dot(ops.gemv(Q4, ur, x)[1])
    for _ in range(20):
        pg = gg + tg * g.uniform(-1, 1, 64)
        pu = uu + tu * g.uniform(-1, 1, 64)
        assert np.all(np.abs(ops.silu(pg) * pu - h) <= th)


# ---------------------------------------------------------------- argmax / topk
def _loop_argmax(v):
    best, bv = 0, v[0]
    for i in range(1, len(v)):
        if v[i] > bv:
            best, bv = i, v[i]
    return best


def test_argmax_first_matches_cpu_loop_and_ties():
    g = np.random.default_rng(12)
    for _ in range(50):
        v = g.integers(-5, 6, 40).astype(np.float64)   # many exact ties
        assert ops.argmax_first(v) == _loop_argmax(v) == int(np.argmax(v))
    assert ops.argmax_first(np.zeros(17)) == 0
    v = np.zeros(10)
    v[3] = v[9] = 1.0
    assert ops.argmax_first(v) == 3
    v = np.array([-0.0, 0.0])
    assert ops.argmax_first(v) == 0


def test_argmax_certification():
    v = np.array([1.0, 5.0, 2.0])
    a = np.ones(3)
    assert ops.argmax_certified(v, a, 1000, 0.0)
    v2 = np.array([1.0, 5.0, 5.0])
    assert not ops.argmax_certified(v2, a, 1000, 0.0)
    v3 = np.array([5.0 - 1e-9, 5.0])
    assert not ops.argmax_certified(v3, np.full(2, 100.0), 1000, 2.0 ** -11)


def test_topk_matches_sorted_and_ties():
    g = np.random.default_rng(13)
    for _ in range(50):
        v = g.integers(-4, 5, 30).astype(np.float64)
        want = sorted(range(30), key=lambda i: (-v[i], i))[:8]
        assert list(ops.topk_lowest_index(v, 8)) == want
    assert list(ops.topk_lowest_index(np.zeros(12), 8)) == list(range(8))


def test_lmhead_topk_by_brute_force():
    """The LM-head candidates: each one's logit is its row's exact product
    (rational brute force over the decoded block), the list is what a full
    sort of all rows by (value desc, index asc) starts with, k = 1 is the
    greedy argmax, and rows at or past n_rows never appear."""
    from fractions import Fraction
    g = np.random.default_rng(15)
    for qtype in (Q4, Q8):
        rows, cols, n_rows = 23, 64, 19
        raw = synth.gen_weights(qtype, rows, cols, 0.02, g)
        x = (g.integers(-8, 9, cols) / 8.0).astype(np.float64)
        w = quant.dequantize(qtype, raw)
        exact = [sum(Fraction(float(w[r, j])) * Fraction(float(x[j])) for j in range(cols)) for r in range(n_rows)]
        for k in (1, 4, n_rows):
            idx, val, logits, _ = ops.lmhead_topk(qtype, raw, x, n_rows, k)
            want = sorted(range(n_rows), key=lambda r: (-exact[r], r))[:k]
            assert list(idx) == want
            assert all(float(exact[r]) == v for r, v in zip(idx, val))
            assert max(idx) < n_rows
        idx1, _, logits, _ = ops.lmhead_topk(qtype, raw, x, n_rows, 1)
        assert idx1[0] == ops.argmax_first(logits)
    # planted ties: duplicated rows give equal logits, the lower row first
    raw = synth.gen_weights(Q8, 6, 32, 0.02, g)
    raw[4] = raw[1]
    raw[5] = raw[1]
    x = np.ones(32)
    idx, val, logits, _ = ops.lmhead_topk(Q8, raw, x, 6, 6)
    pos = {int(r): i for i, r in enumerate(idx)}
    assert pos[1] < pos[4] < pos[5] and pos[5] == pos[1] + 2


def test_rmsnorm_by_definition_and_closed_forms():
    """n(x) = x * gamma / sqrt(mean(x^2) + eps): an explicit loop with exact
    rational arithmetic before the one square root; a constant column c gives
    gamma * c / sqrt(c^2 + eps); with eps = 0 the result does not change when
    x is scaled by any a > 0 and has root mean square 1 for gamma = 1; columns
    are independent."""
    from fractions import Fraction
    import math
    g = np.random.default_rng(16)
    K = 48
    x = (g.integers(-64, 65, K) / 16.0).astype(np.float64)
    gam = (g.integers(1, 9, K) / 4.0).astype(np.float64)
    eps = 2.0 ** -10
    ms = sum(Fraction(float(v)) ** 2 for v in x) / K + Fraction(eps)
    inv = 1.0 / math.sqrt(float(ms))
    want = [float(Fraction(float(v)) * Fraction(float(gg))) * inv for v, gg in zip(x, gam)]
    assert np.allclose(ops.rmsnorm(x, gam, eps), want, rtol=4e-16, atol=0)
    c = 3.0
    assert np.allclose(ops.rmsnorm(np.full(K, c), gam, eps), gam * c / np.sqrt(c * c + eps), rtol=1e-15)
    assert np.allclose(ops.rmsnorm(-np.full(K, c), gam, eps), -gam * c / np.sqrt(c * c + eps), rtol=1e-15)
    one = np.ones(K)
    n0 = ops.rmsnorm(x, one, 0.0)
    assert np.allclose(ops.rmsnorm(7.5 * x, one, 0.0), n0, rtol=1e-14)
    assert abs(np.sqrt(np.mean(n0 * n0)) - 1.0) < 1e-14
    X = np.stack([x, 2 * x[::-1], np.full(K, -0.5)], axis=1)
    N = ops.rmsnorm(X, gam, eps)
    for j in range(3):
        assert np.array_equal(N[:, j], ops.rmsnorm(X[:, j], gam, eps))


def test_moe_with_norm_invariants():
    """The norm ahead of the MoE: with unit weights and eps = 0, scaling x by
    any a > 0 changes nothing (router and experts both read the normalised
    x); with unit weights the experts chosen are those of the plain layer
    (1 / rms is one positive factor per token); and the result is the plain
    layer applied to the normalised x, whose RMS is 1."""
    g = np.random.default_rng(17)
    E, H, F, k = 6, 64, 32, 2
    router = (g.standard_normal((E, H)) * 0.1).astype(np.float32)
    gate = np.stack([synth.gen_weights(Q4, F, H, 0.05, g) for _ in range(E)])
    upw = np.stack([synth.gen_weights(Q4, F, H, 0.05, g) for _ in range(E)])
    down = np.stack([synth.gen_weights(Q4, H, F, 0.05, g) for _ in range(E)])
    x = g.standard_normal((H, 3)) * 4.0
    one = np.ones(H)
    r1 = ops.moe_ffn(x, router, Q4, gate, upw, down, top_k=k, norm_w=one, norm_eps=0.0)
    r2 = ops.moe_ffn(2.5 * x, router, Q4, gate, upw, down, top_k=k, norm_w=one, norm_eps=0.0)
    assert np.array_equal(r1["idx"], r2["idx"])
    assert np.allclose(r1["y"], r2["y"], rtol=1e-12, atol=1e-14)
    plain = ops.moe_ffn(x, router, Q4, gate, upw, down, top_k=k)
    assert np.array_equal(r1["idx"], plain["idx"])
    xn = x / np.sqrt(np.mean(x * x, axis=0))
    assert np.allclose(np.sqrt(np.mean(xn * xn, axis=0)), 1.0, rtol=1e-14)
    r3 = ops.moe_ffn(xn, router, Q4, gate, upw, down, top_k=k)
    assert np.allclose(r1["y"], r3["y"], rtol=1e-12, atol=1e-14)
    assert np.all(r1["logit_a"] >= ops.router_logits(xn, router)[1])


def test_requant_decoding_by_hand():
    """Hand-built source blocks with known values: Q4_1 weight j at nibble
    j (low) or j - 16 (high), value w * d + m; Q5_0 / Q5_1 with single qh
    bits set (bit j adds 16 to weight j, bit j + 16 to weight j + 16)."""
    from oracle import requant as rq
    d_one, m_neg2 = np.array([1.0], np.float16).view(np.uint8), np.array([-2.0], np.float16).view(np.uint8)
    b = np.zeros((1, 20), np.uint8)
    b[0, 0:2], b[0, 2:4] = d_one, m_neg2
    b[0, 4:20] = np.arange(16, dtype=np.uint8) | ((15 - np.arange(16, dtype=np.uint8)) << 4)
    v = rq.decode_values_f32(rq.Q4_1, b)[0]
    assert list(v[:16]) == [j - 2.0 for j in range(16)] and list(v[16:]) == [13.0 - j for j in range(16)]
    half = np.array([0.5], np.float16).view(np.uint8)
    for t, qh_off, qs_off in ((rq.Q5_0, 2, 6), (rq.Q5_1, 4, 8)):
        b = np.zeros((1, rq.SRC_BLOCK_BYTES[t]), np.uint8)
        b[0, 0:2] = half
        if t == rq.Q5_1:
            b[0, 2:4] = m_neg2
        b[0, qs_off:qs_off + 16] = 0x31            # low nibble 1, high nibble 3
        b[0, qh_off:qh_off + 4] = np.array([(1 << 5) | (1 << 20)], "<u4").view(np.uint8)
        v = rq.decode_values_f32(t, b)[0]
        w = np.array([1] * 16 + [3] * 16)
        w[5] += 16
        w[20] += 16
        want = (w - 16) * 0.5 if t == rq.Q5_0 else w * 0.5 - 2.0
        assert np.array_equal(v, want.astype(np.float32)), t


def test_requant_rounding_rules():
    """Q8_0 requantisation: all-zero blocks stay zero with scale 0; the
    largest magnitude maps to +-127; halves round away from zero (checked
    against the definition on exact float32 halves); the reconstruction
    error stays within half a step plus the f16 rounding of the scale; and
    negating the values negates the weights."""
    from oracle import requant as rq
    assert list(rq.round_half_away(np.array([0.5, -0.5, 1.5, -2.5, 0.49999997, 2.4999998]))) == \
        [1.0, -1.0, 2.0, -3.0, 0.0, 2.0]
    z = rq.quantize_q8_0(np.zeros((1, 32), np.float32))
    assert not z.any()
    g = np.random.default_rng(18)
    v = (g.standard_normal((200, 32)) * g.uniform(1e-3, 50.0, (200, 1))).astype(np.float32)
    out = rq.quantize_q8_0(v)
    w, d = quant.decode_blocks(quant.Q8_0, out)
    top = np.argmax(np.abs(v), axis=1)
    assert np.all(np.abs(w[np.arange(200), top]) == 127)
    amax = np.max(np.abs(v), axis=1).astype(np.float64)
    step = amax / 127.0
    err = np.abs(w * d[:, None] - v.astype(np.float64))
    assert np.all(err <= 0.5 * step[:, None] * (1 + 1e-6) + 127 * np.abs(d - step)[:, None] + 1e-12)
    neg = rq.quantize_q8_0(-v)
    wn, dn = quant.decode_blocks(quant.Q8_0, neg)
    assert np.array_equal(wn, -w) and np.array_equal(dn, d)


@pytest.mark.parametrize("name,src", [("q4_k_block.txt", 12), ("q5_k_block.txt", 13), ("q6_k_block.txt", 14)])
def test_kquant_decoding_golden(name, src):
    """Hand-worked K-quant super-blocks (values worked out in the fixture
    comments from the public GGUF layouts)."""
    from oracle import requant as rq
    raw, g = _block(name)
    assert raw.size == rq.SRC_BLOCK_BYTES[src]
    v = rq.decode_values_f32(src, raw[None, :])[0]
    assert v.shape == (256,) and v.dtype == np.float32
    keys = [k for k in g if k.startswith("v")]
    assert len(keys) >= 10
    for k in keys:
        assert v[int(k[1:])] == float(g[k]), (name, k, v[int(k[1:])], g[k])
    out = rq.requant_q8_0(src, np.stack([raw, raw]))
    assert out.shape == (16, 34)


def _pack_k_scales(sc, m):
    """12 scale bytes from 6-bit scales and mins, the packing direction:
    sub-blocks 0..3 fill the low 6 bits of bytes 0..3 (scales) and 4..7
    (mins); sub-blocks 4..7 put scale | min << 4 (low nibbles) in bytes
    8..11 and their top two bits in the top bits of bytes 0..3 (scales) and
    4..7 (mins)."""
    b = np.zeros(sc.shape[:-1] + (12,), np.int64)
    for j in range(4):
        b[..., j] = sc[..., j] | ((sc[..., j + 4] >> 4) << 6)
        b[..., j + 4] = m[..., j] | ((m[..., j + 4] >> 4) << 6)
        b[..., j + 8] = (sc[..., j + 4] & 15) | ((m[..., j + 4] & 15) << 4)
    return b.astype(np.uint8)


def test_kquant_scale_packing_round_trip():
    from oracle import requant as rq
    g = np.random.default_rng(41)
    sc, m = g.integers(0, 64, (2000, 8)), g.integers(0, 64, (2000, 8))
    got_sc, got_m = rq.k_scales_mins(_pack_k_scales(sc, m))
    assert np.array_equal(got_sc, sc) and np.array_equal(got_m, m)
    # every byte value is a legal packing: decoding covers 0..63 and re-packs
    s12 = g.integers(0, 256, (2000, 12)).astype(np.uint8)
    a, b = rq.k_scales_mins(s12)
    assert a.min() >= 0 and a.max() <= 63 and b.min() >= 0 and b.max() <= 63
    assert np.array_equal(_pack_k_scales(a, b), s12)


def _f16b(x):
    return np.asarray(x, np.float16).view(np.uint8).reshape(-1, 2)


def test_kquant_sub_blocks_are_legacy_blocks():
    """Special cases that reduce to the (separately pinned) 32-value
    formats.  A Q4_K / Q5_K sub-block whose d * sc and dmin * m are exact in
    f16 is the Q4_1 / Q5_1 block with scale d * sc, offset -dmin * m and the
    same weights (both formats round the one difference of exact terms); a
    Q6_K run of 32 whose two 16-value scales agree is the Q8_0 block with
    scale d * sc and weights w - 32."""
    from oracle import requant as rq
    g = np.random.default_rng(43)
    nb = 96
    for src, legacy, wbits in ((rq.Q4_K, rq.Q4_1, 4), (rq.Q5_K, rq.Q5_1, 5)):
        sc, m = g.integers(0, 64, (nb, 8)), g.integers(0, 64, (nb, 8))
        d, dmin = 2.0 ** g.integers(-10, 2, nb), 2.0 ** g.integers(-10, 2, nb)
        w = g.integers(0, 1 << wbits, (nb, 8, 32))
        raw = np.zeros((nb, rq.SRC_BLOCK_BYTES[src]), np.uint8)
        raw[:, 0:2], raw[:, 2:4], raw[:, 4:16] = _f16b(d), _f16b(dmin), _pack_k_scales(sc, m)
        lo = w & 15
        qs = (lo[:, 0::2, :] | (lo[:, 1::2, :] << 4)).reshape(nb, 128)   # byte 32 c + i
        if src == rq.Q4_K:
            raw[:, 16:144] = qs
        else:
            raw[:, 16:48] = sum(((w[:, j, :] >> 4) & 1) << j for j in range(8))
            raw[:, 48:176] = qs
        leg = np.zeros((nb, 8, rq.SRC_BLOCK_BYTES[legacy]), np.uint8)
        leg[..., 0:2] = _f16b((d[:, None] * sc).reshape(-1)).reshape(nb, 8, 2)
        leg[..., 2:4] = _f16b((-dmin[:, None] * m).reshape(-1)).reshape(nb, 8, 2)
        nib = (w[..., :16] & 15) | ((w[..., 16:] & 15) << 4)
        if legacy == rq.Q4_1:
            leg[..., 4:20] = nib
        else:
            hb = sum(((w[..., i] >> 4) & 1) << i for i in range(32)).astype("<u4")
            leg[..., 4:8] = hb[..., None].view(np.uint8)
            leg[..., 8:24] = nib
        want = rq.decode_values_f32(legacy, leg.reshape(nb * 8, -1))
        got = rq.decode_values_f32(src, raw).reshape(nb * 8, 32)
        assert np.array_equal(got, want), src
    # Q6_K: scales equal in pairs
    sc = np.repeat(g.integers(-128, 128, (nb, 8)), 2, axis=1)
    d = 2.0 ** g.integers(-12, -2, nb)
    w = g.integers(0, 64, (nb, 256))
    raw = np.zeros((nb, 210), np.uint8)
    h = w.reshape(nb, 2, 4, 32)                       # [half, quarter, lane]
    raw[:, 0:128] = ((h[:, :, 0:2, :] & 15) | ((h[:, :, 2:4, :] & 15) << 4)).reshape(nb, 128)
    raw[:, 128:192] = sum(((h[:, :, k, :] >> 4) & 3) << (2 * k) for k in range(4)).reshape(nb, 64)
    raw[:, 192:208] = sc.astype(np.int8).view(np.uint8)
    raw[:, 208:210] = _f16b(d)
    q8 = np.zeros((nb, 8, 34), np.uint8)
    q8[..., 0:2] = _f16b((d[:, None] * sc[:, 0::2]).reshape(-1)).reshape(nb, 8, 2)
    q8[..., 2:34] = (w - 32).astype(np.int8).view(np.uint8).reshape(nb, 8, 32)
    wq, dq = quant.decode_blocks(Q8, q8.reshape(-1, 34))
    got = rq.decode_values_f32(rq.Q6_K, raw).reshape(nb * 8, 32).astype(np.float64)
    assert np.array_equal(got, wq * dq[:, None])


def test_softmax_properties():
    g = np.random.default_rng(14)
    v = g.standard_normal(8)
    p = ops.softmax(v)
    assert abs(p.sum() - 1) < 1e-15
    assert np.allclose(p, ops.softmax(v + 123.0), rtol=1e-13)
    assert np.allclose(p, scipy.special.softmax(v), rtol=1e-14)


# ----------------------------------------------------------------------- MoE
def _moe_inputs(E, H, F, seed, shared=True, identical=False):
    g = np.random.default_rng(seed)
    gate = np.stack([synth.gen_weights(Q4, F, H, 0.02, g) for _ in range(E)])
    up = np.stack([synth.gen_weights(Q4, F, H, 0.02, g) for _ in range(E)])
    down = np.stack([synth.gen_weights(Q4, H, F, 0.02, g) for _ in range(E)])
    if identical:
        gate[:] = gate[0]
        up[:] = up[0]
        down[:] = down[0]
    router = synth.gen_f32((E, H), 0.02, g)
    sh = None
    if shared:
        sh = (synth.gen_weights(Q4, F, H, 0.02, g), synth.gen_weights(Q4, F, H, 0.02, g),
              synth.gen_weights(Q4, H, F, 0.02, g))
    x = g.standard_normal((H, 3)).astype(np.float32)
    return gate, up, down, router, sh, x


def _dense_ffn(gr, ur, dr, x):
    G, U, D = (quant.dequantize(Q4, r) for r in (gr, ur, dr))
    xx = np.asarray(x, np.float64)
    gg = G @ xx
    return D @ (gg * scipy.special.expit(gg) * (U @ xx))


def test_moe_single_expert_is_dense_ffn():
    gate, up, down, router, sh, x = _moe_inputs(1, 64, 32, 20)
    res = ops.moe_ffn(x, router, Q4, gate, up, down, top_k=1,
                      sh_gate=sh[0], sh_up=sh[1], sh_down=sh[2])
    want = _dense_ffn(gate[0], up[0], down[0], x) + _dense_ffn(*sh, x)
    assert np.allclose(res["y"], want, rtol=1e-12, atol=1e-12)
    assert np.all(res["p"] == 1.0)


def test_moe_identical_experts_equal_one_ffn():
    gate, up, down, router, _, x = _moe_inputs(6, 64, 32, 21, shared=False, identical=True)
    res = ops.moe_ffn(x, router, Q4, gate, up, down, top_k=3)
    want = _dense_ffn(gate[0], up[0], down[0], x)
    assert np.allclose(res["y"], want, rtol=1e-12, atol=1e-12)
    assert np.allclose(res["p"].sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_moe_expert_relabeling_invariant_and_accumulates():
    gate, up, down, router, sh, x = _moe_inputs(6, 64, 32, 22)
    y_in = np.random.default_rng(5).standard_normal((64, 3)).astype(np.float32)
    res = ops.moe_ffn(x, router, Q4, gate, up, down, top_k=2, y_in=y_in,
                      sh_gate=sh[0], sh_up=sh[1], sh_down=sh[2])
    perm = np.random.default_rng(6).permutation(6)
    res2 = ops.moe_ffn(x, router[perm], Q4, gate[perm], up[perm], down[perm], top_k=2,
                       y_in=y_in, sh_gate=sh[0], sh_up=sh[1], sh_down=sh[2])
    assert np.allclose(res["y"], res2["y"], rtol=1e-13, atol=1e-13)
    # the same experts are chosen (no ties among continuous logits)
    assert np.array_equal(np.sort(perm[res2["idx"]], axis=1), np.sort(res["idx"], axis=1))
    res0 = ops.moe_ffn(x, router, Q4, gate, up, down, top_k=2,
                       sh_gate=sh[0], sh_up=sh[1], sh_down=sh[2])
    assert np.allclose(res["y"] - y_in, res0["y"], rtol=1e-12, atol=1e-12)


def test_moe_unnormalized_weights_are_full_softmax():
    gate, up, down, router, _, x = _moe_inputs(5, 64, 32, 23, shared=False)
    res = ops.moe_ffn(x, router, Q4, gate, up, down, top_k=5, normalize=False)
    assert np.allclose(res["p"].sum(axis=1), 1.0, atol=1e-14)
    res2 = ops.moe_ffn(x, router, Q4, gate, up, down, top_k=2, normalize=False)
    assert np.all(res2["p"].sum(axis=1) < 1.0)


# ---------------------------------------------------------------- repacked layout
def _unpack_tiled(qtype, qs, d, rows, cols):
    """Independent reader of the tiled layout: walks every weight position and
    extracts it with explicit bit arithmetic."""
    nt, kt = -(-rows // 16), -(-(cols // 32) // 4)
    W = np.zeros((nt * 16, kt * 128), np.int64)
    S = np.zeros((nt * 16, kt * 4), np.float64)
    for rt in range(nt):
        for k in range(kt):
            t = rt * kt + k
            for r in range(16):
                for j in range(4):
                    off = t * 128 + 8 * r + 2 * j
                    S[rt * 16 + r, k * 4 + j] = quant.f16_to_f64(d[off:off + 1], d[off + 1:off + 2])[0]
                for col in range(128):
                    j, within = divmod(col, 32)
                    s, i = divmod(within, 8)
                    if qtype == Q4:
                        base = t * 1024 + (16 * s + r) * 16 + 4 * j
                        word = int.from_bytes(bytes(qs[base:base + 4]), "little")
                        shift = 4 * (i // 2) + (16 if i % 2 else 0)
                        W[rt * 16 + r, k * 128 + col] = ((word >> shift) & 0xF) - 8
                    else:
                        h, jj = divmod(j, 2)
                        off = t * 2048 + h * 1024 + (16 * s + r) * 16 + jj * 8 + i
                        W[rt * 16 + r, k * 128 + col] = int(qs[off]) - 128
    return W, S


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_repack_reference_round_trip(qtype):
    g = np.random.default_rng(30)
    rows, cols = 20, 160                      # ragged in both directions
    raw = synth.gen_weights(qtype, rows, cols, 0.02, g)
    qs, d = quant.repack_reference(qtype, raw)
    assert (qs.size, d.size) == quant.packed_bytes(qtype, 1, rows, cols)
    W, S = _unpack_tiled(qtype, qs, d, rows, cols)
    w, sc = quant.decode_blocks(qtype, raw)
    assert np.array_equal(W[:rows, :cols], w.reshape(rows, cols))
    assert np.array_equal(S[:rows, :cols // 32], sc)
    assert np.all(W[rows:] == 0) and np.all(W[:, cols:] == 0)
    assert np.all(S[rows:] == 0) and np.all(S[:, cols // 32:] == 0)


def test_repack_reference_stacked_matrices_are_independent():
    g = np.random.default_rng(31)
    raw = np.stack([synth.gen_weights(Q4, 18, 64, 0.02, g) for _ in range(3)])
    qs, d = quant.repack_reference(Q4, raw)
    qb, db = quant.packed_bytes(Q4, 1, 18, 64)
    for m in range(3):
        q1, d1 = quant.repack_reference(Q4, raw[m])
        assert np.array_equal(qs[m * qb:(m + 1) * qb], q1)
        assert np.array_equal(d[m * db:(m + 1) * db], d1)
