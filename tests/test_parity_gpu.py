"""GPU parity: the HIP path (through the C-ABI) against the f64 oracle.

Float outputs must satisfy |gpu - ref| <= 2e-3 * sum|w x| + 1e-5 (derived
bounds for SiLU-gated and MoE outputs, see oracle.ops); indices bit-exact
whenever the oracle certifies them; byte outputs (the repack) bit-exact.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import EPS_OP, assert_tol, check_routing, check_topk_order, host, say, up
from oracle import ops, quant

pytestmark = pytest.mark.gpu

Q4, Q8 = synth.Q4_0, synth.Q8_0
SIG = {Q4: 0.02, Q8: 0.005}


def make(env, qtype, rows, cols, seed, sigma=None, n_mat=1):
    torch, qg, dev = env
    g = np.random.default_rng(seed)
    if n_mat == 1:
        raw = synth.gen_weights(qtype, rows, cols, SIG[qtype] if sigma is None else sigma, g)
    else:
        raw = np.stack([synth.gen_weights(qtype, rows, cols, SIG[qtype] if sigma is None else sigma, g)
                        for _ in range(n_mat)])
    W = qg.qg_repack(qtype, up(env, raw.reshape(-1)), rows, cols, n_mat)
    return raw, W


# ------------------------------------------------------------------ repack
@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("n_mat,rows,cols", [(1, 40, 416), (3, 20, 160), (1, 64, 2048)])
def test_repack_bit_exact(env, qtype, n_mat, rows, cols):
    torch, qg, dev = env
    say(f"repack qtype={qtype} n_mat={n_mat} {rows}x{cols}")
    raw, W = make(env, qtype, rows, cols, seed=1, n_mat=n_mat)
    torch.cuda.synchronize()
    qs_ref, d_ref = quant.repack_reference(qtype, raw)
    assert np.array_equal(W.qs.cpu().numpy(), qs_ref)
    assert np.array_equal(W.d.cpu().numpy(), d_ref)


# -------------------------------------------------------------------- GEMV
SMALL = [(40, 416), (16, 128), (64, 4096), (200, 2080), (2048, 2048)]


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", SMALL)
@pytest.mark.parametrize("ncols", [1, 3, 8])
@pytest.mark.parametrize("acc", [0, 1])
def test_gemv_parity(env, qtype, rows, cols, ncols, acc):
    torch, qg, dev = env
    say(f"gemv qtype={qtype} {rows}x{cols} ncols={ncols} acc={acc}")
    raw, W = make(env, qtype, rows, cols, seed=rows * 7 + cols)
    X = synth.gen_x(cols, ncols, cfg_id=rows + cols)
    y_in = synth.rng(9, rows).standard_normal((rows, ncols)).astype(np.float32)
    Xd = up(env, X.T)
    Yd = up(env, y_in.T) if acc else None
    Yd = qg.qgemv(W, Xd, Yd, accumulate=bool(acc))
    torch.cuda.synchronize()
    ref, a = ops.gemv(qtype, raw, X, y_in=y_in if acc else None)
    assert_tol(host(Yd).T, ref, ops.tol_dot(a, ref), "gemv")


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(40, 416), (64, 4096), (5120, 5120)])
def test_batched_columns_bitwise_equal_single(env, qtype, rows, cols):
    torch, qg, dev = env
    say(f"bit-identity qtype={qtype} {rows}x{cols}")
    _, W = make(env, qtype, rows, cols, seed=3)
    X = up(env, synth.gen_x(cols, 8, cfg_id=33).T)
    for n in range(1, 9):
        Yn = qg.qgemv(W, X[:n].contiguous())
        for j in range(n):
            Y1 = qg.qgemv(W, X[j:j + 1].contiguous())
            assert torch.equal(Yn[j], Y1[0]), (n, j)


# ------------------------------------------ signed scales, int8 -128, range
def make_signed(env, qtype, rows, cols, seed):
    """Weights with seeded sign flips on the block scales and (Q8_0) planted
    -128 bytes, repacked on the GPU."""
    torch, qg, dev = env
    g = np.random.default_rng(seed)
    raw = synth.flip_scale_signs(synth.gen_weights(qtype, rows, cols, SIG[qtype], g), g)
    if qtype == Q8:
        raw = synth.plant_q8_min(raw, g, 0.05)
    return raw, qg.qg_repack(qtype, up(env, raw.reshape(-1)), rows, cols)


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(40, 416), (200, 2080), (64, 8192)])
@pytest.mark.parametrize("ncols", [1, 3, 8, 16])
def test_signed_scales_and_int8_min(env, qtype, rows, cols, ncols):
    """Negative block scales (about half of them) and Q8_0 weights of -128:
    GEMV (accumulating), 16-column GEMM and gate/up against the oracle."""
    torch, qg, dev = env
    say(f"signed scales qtype={qtype} {rows}x{cols} ncols={ncols}")
    raw, W = make_signed(env, qtype, rows, cols, seed=rows + cols + ncols)
    assert np.any(raw[..., 1] & 0x80) and np.any(~raw[..., 1] & 0x80)
    if qtype == Q8:
        assert np.any(raw[..., 2:] == 0x80)
    X = synth.gen_x(cols, ncols, cfg_id=500 + ncols)
    y_in = synth.rng(501, rows).standard_normal((rows, ncols)).astype(np.float32)
    if ncols == 16:
        Y = qg.qgemm16(W, up(env, X.T), up(env, y_in.T), accumulate=True)
    else:
        Y = qg.qgemv(W, up(env, X.T), up(env, y_in.T), accumulate=True)
    torch.cuda.synchronize()
    ref, a = ops.gemv(qtype, raw, X, y_in=y_in)
    assert_tol(host(Y).T, ref, ops.tol_dot(a, ref), "signed gemv")
    if ncols <= 8:
        uraw, U = make_signed(env, qtype, rows, cols, seed=rows + cols + 77)
        H = qg.gateup_silu(W, U, up(env, X.T))
        hr, th, _, _ = ops.gateup_silu(qtype, raw, uraw, X)
        assert_tol(host(H).T, hr, th, "signed gate/up")


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_signed_scales_lmhead(env, qtype):
    """The LM head's argmax and top-k on weights with signed scales."""
    torch, qg, dev = env
    rows, cols = 3000, 1024
    raw, W = make_signed(env, qtype, rows, cols, seed=503)
    seen = 0
    for s in range(30):
        x = synth.gen_x(cols, 1, cfg_id=504 + s)[:, 0]
        ref, a = ops.gemv(qtype, raw, x)
        if not ops.topk_certified(ref, a, 8, cols + 64, EPS_OP, order=True):
            continue
        idx, val = qg.lmhead_argmax(W, up(env, x))
        ti, tv = qg.lmhead_topk(W, up(env, x), 8)
        assert int(idx.item()) == ops.argmax_first(ref)
        assert list(ti.cpu().numpy()) == list(ops.topk_lowest_index(ref, 8))
        seen += 1
        if seen == 3:
            break
    assert seen == 3


def _x_scaled(kind, cols, ncols, cfg):
    """Activations far outside the f16 range: 'huge' (|x| up to ~1e8), 'tiny'
    (|x| ~ 1e-18, below the f16 subnormals), 'mixed' (each block of 32 of each
    column scaled by its own power of two in 2^-60 .. 2^40)."""
    X = synth.gen_x(cols, ncols, cfg_id=cfg).astype(np.float64)
    if kind == "huge":
        X *= 2.0 ** 24
    elif kind == "tiny":
        X *= 2.0 ** -60
    else:
        e = synth.rng(cfg, 95).integers(-60, 41, size=(cols // 32, ncols))
        X *= np.repeat(2.0 ** e, 32, axis=0)
    return X.astype(np.float32)


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(200, 2080), (64, 8192)])
@pytest.mark.parametrize("ncols", [1, 3, 8])
@pytest.mark.parametrize("kind", ["huge", "tiny", "mixed"])
def test_activation_range(env, qtype, rows, cols, ncols, kind):
    """Products of 1..8 columns keep the f32 range of the activations: the
    relative bound 2e-3 * sum|w x| holds with no absolute floor, at
    magnitudes where f16 operands overflow or flush to zero.  Also the LM
    head (1 column) on huge inputs."""
    torch, qg, dev = env
    say(f"activation range qtype={qtype} {rows}x{cols} ncols={ncols} {kind}")
    raw, W = make_signed(env, qtype, rows, cols, seed=7 * rows + cols)
    X = _x_scaled(kind, cols, ncols, cfg=510 + ncols)
    Y = qg.qgemv(W, up(env, X.T))
    torch.cuda.synchronize()
    ref, a = ops.gemv(qtype, raw, X)
    got = host(Y).T
    assert np.all(np.isfinite(got))
    assert_tol(got, ref, ops.REL_TOL * a + 2 * ops.U32 * np.abs(ref), f"range {kind}")
    if ncols == 1 and kind != "tiny":
        idx, val = qg.lmhead_argmax(W, up(env, X[:, 0]))
        if ops.argmax_certified(ref[:, 0], a[:, 0], cols + 64, EPS_OP):
            assert int(idx.item()) == ops.argmax_first(ref[:, 0])


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("ncols", [1, 5])
def test_activation_precision_systematic(env, qtype, ncols):
    """Activations 2^e * (1 + 2^-12), which f16 cannot hold (it would round
    every one down by 2^-12 relative), against weights of one sign: the
    error must stay within the f32 summation bound plus 2^-22 per operand,
    far below the 2^-12 * sum|w x| an f16 operand would leave."""
    torch, qg, dev = env
    rows, cols = 48, 1024
    g = np.random.default_rng(520 + ncols)
    if qtype == Q4:
        nib = g.integers(9, 16, size=(rows, cols // 32, 32), dtype=np.uint8)   # weights 1..7
        raw = synth.pack_q4_0(nib, np.full((rows, cols // 32), 0.03125, np.float16))
    else:
        q = g.integers(1, 128, size=(rows, cols // 32, 32)).astype(np.int8)
        raw = synth.pack_q8_0(q, np.full((rows, cols // 32), 0.0078125, np.float16))
    W = qg.qg_repack(qtype, up(env, raw.reshape(-1)), rows, cols)
    e = g.integers(-8, 9, size=(cols, ncols))
    X = ((1.0 + 2.0 ** -12) * 2.0 ** e).astype(np.float32)
    assert np.all(X.astype(np.float16).astype(np.float32) != X)
    Y = host(qg.qgemv(W, up(env, X.T))).T
    ref, a = ops.gemv(qtype, raw, X)
    k = cols + 64
    gam = k * ops.U32 / (1 - k * ops.U32)
    bound = (gam + EPS_OP * (1 + gam)) * a
    assert np.all(bound < 2.0 ** -12 * a / 2)
    assert_tol(Y, ref, bound, "systematic precision")


def test_workspace_shared_across_shapes_and_calls(env):
    """One workspace serves interleaved calls of different shapes and entry
    points: a call's scratch (partials, argmax candidates) never lands on
    another call's counters."""
    torch, qg, dev = env
    ws = torch.zeros(max(qg.lib.qg_gemv_ws_bytes(r, c) for r, c in ((64, 4096), (5120, 5120), (40, 416)))
                     + (1 << 22), dtype=torch.uint8, device=dev)
    cases = []
    for qtype, rows, cols, nc in ((Q4, 64, 4096, 8), (Q4, 5120, 5120, 2), (Q8, 40, 416, 3),
                                  (Q4, 5120, 5120, 5), (Q8, 64, 4096, 2)):
        raw, W = make(env, qtype, rows, cols, seed=rows + cols + nc)
        X = synth.gen_x(cols, nc, cfg_id=300 + nc)
        ref, a = ops.gemv(qtype, raw, X)
        cases.append((W, up(env, X.T), ref, a))
    for rep in range(3):
        for i, (W, Xd, ref, a) in enumerate(cases):
            Y = torch.full((Xd.shape[0], W.rows), float("nan"), device=dev)
            st = (qg.lib.qgemv_q4_0 if W.qtype == Q4 else qg.lib.qgemv_q8_0)(
                W.qs.data_ptr(), W.d.data_ptr(), W.rows, W.cols, Xd.data_ptr(), Xd.shape[1], Xd.shape[0],
                Y.data_ptr(), W.rows, 0, ws.data_ptr(), ws.numel(), qg._stream(dev))
            assert st == 0, qg.lib.qg_strerror(st)
            torch.cuda.synchronize()
            assert_tol(host(Y).T, ref, ops.tol_dot(a), f"shared ws rep {rep} case {i}")


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_repeat_runs_bitwise_identical(env, qtype):
    torch, qg, dev = env
    _, W = make(env, qtype, 5120, 17408, seed=4)
    X = up(env, synth.gen_x(17408, 4, cfg_id=44).T)
    Y0 = qg.qgemv(W, X).clone()
    for _ in range(3):
        assert torch.equal(qg.qgemv(W, X), Y0)
    Z0 = qg.qgemm16(W, up(env, synth.gen_x(17408, 16, cfg_id=45).T)).clone()
    assert torch.equal(qg.qgemm16(W, up(env, synth.gen_x(17408, 16, cfg_id=45).T)), Z0)


def test_degenerate_weights(env):
    torch, qg, dev = env
    say("degenerate weights")
    rows, cols = 48, 256
    nib = np.full((rows, cols // 32, 32), 8, np.uint8)
    d = np.abs(np.random.default_rng(0).normal(0, 1, (rows, cols // 32))).astype(np.float16)
    raw = synth.pack_q4_0(nib, d)
    W = qg.qg_repack(Q4, up(env, raw.reshape(-1)), rows, cols)
    X = up(env, synth.gen_x(cols, 2, cfg_id=5).T)
    assert torch.count_nonzero(qg.qgemv(W, X)) == 0
    nib = np.random.default_rng(1).integers(0, 16, (rows, cols // 32, 32)).astype(np.uint8)
    raw = synth.pack_q4_0(nib, np.zeros((rows, cols // 32), np.float16))
    W = qg.qg_repack(Q4, up(env, raw.reshape(-1)), rows, cols)
    assert torch.count_nonzero(qg.qgemv(W, X)) == 0
    assert torch.count_nonzero(qg.qgemm16(W, up(env, synth.gen_x(cols, 16, cfg_id=6).T))) == 0


# ------------------------------------------------------------------ gemm16
# (4352, 2048), (8200, 1664), (12300, 1152): several row tiles per CU with
# 4, 3 and 2 K segments and ragged last row tiles.
@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(40, 416), (64, 4096), (200, 2080), (16, 128),
                                       (4352, 2048), (8200, 1664), (12300, 1152)])
@pytest.mark.parametrize("acc", [0, 1])
def test_gemm16_parity(env, qtype, rows, cols, acc):
    torch, qg, dev = env
    say(f"gemm16 qtype={qtype} {rows}x{cols} acc={acc}")
    raw, W = make(env, qtype, rows, cols, seed=rows + 11 * cols)
    X = synth.gen_x(cols, 16, cfg_id=7)
    y_in = synth.rng(8, rows).standard_normal((rows, 16)).astype(np.float32)
    Yd = up(env, y_in.T) if acc else None
    Yd = qg.qgemm16(W, up(env, X.T), Yd, accumulate=bool(acc))
    torch.cuda.synchronize()
    ref, a = ops.gemv(qtype, raw, X, y_in=y_in if acc else None)
    assert_tol(host(Yd).T, ref, ops.tol_dot(a, ref), "gemm16")


# --------------------------------------------- 16 columns, several problems
BATCH = [(Q4, 40, 416, 0), (Q8, 200, 2080, 1), (Q4, 600, 11264, 1), (Q8, 64, 4096, 0),
         (Q4, 16, 128, 1), (Q8, 2100, 2048, 0), (Q4, 5120, 512, 0), (Q8, 40, 416, 1)]


@pytest.mark.parametrize("n", [1, 3, 8])
def test_gemm16_batch(env, n):
    """Several 16-column problems (Q4_0 and Q8_0 mixed, storing and
    accumulating, one to eight of them) in one launch: each output against
    the oracle, bitwise equal to qgemm16 on that problem with the launch's
    K split pinned, and bitwise equal again on a repeat launch."""
    torch, qg, dev = env
    say(f"gemm16 batch n={n}")
    probs, refs = [], []
    for i, (qt, rows, cols, acc) in enumerate(BATCH[:n]):
        raw, W = make(env, qt, rows, cols, seed=700 + i)
        X = synth.gen_x(cols, 16, cfg_id=701 + i)
        y0 = synth.rng(702, i).standard_normal((rows, 16)).astype(np.float32)
        probs.append((W, up(env, X.T), up(env, y0.T) if acc else None, acc))
        refs.append((raw, X, y0))
    splits = qg.gemm16_batch_splits(probs)
    say(f"  splits {splits}")
    try:
        for (qt, rows, cols, _), sp in zip(BATCH[:n], splits):
            qg.plan_set(qg.OP_GEMV, qt, rows, cols, 16, qg.PLAN_SPLIT(sp) | qg.PLAN_STRICT)
        single = [qg.qgemm16(W, X, None if Y is None else Y.clone(), accumulate=bool(acc)) for W, X, Y, acc in probs]
    finally:
        qg.plan_reset()
    outs = qg.qgemm16_batch([(W, X, None if Y is None else Y.clone(), acc) for W, X, Y, acc in probs])
    again = qg.qgemm16_batch([(W, X, None if Y is None else Y.clone(), acc) for W, X, Y, acc in probs])
    torch.cuda.synchronize()
    for i, ((qt, rows, cols, acc), (raw, X, y0)) in enumerate(zip(BATCH[:n], refs)):
        ref, a = ops.gemv(qt, raw, X, y_in=y0 if acc else None)
        assert_tol(host(outs[i]).T, ref, ops.tol_dot(a, ref), f"batch problem {i}")
        assert torch.equal(outs[i], single[i]), i
        assert torch.equal(again[i], outs[i]), i


# ----------------------------------------------------------------- gate/up
@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(40, 416), (64, 4096), (512, 2048)])
@pytest.mark.parametrize("ncols", [1, 4, 8])
def test_gateup_parity(env, qtype, rows, cols, ncols):
    torch, qg, dev = env
    say(f"gateup qtype={qtype} {rows}x{cols} ncols={ncols}")
    graw, G = make(env, qtype, rows, cols, seed=21)
    uraw, U = make(env, qtype, rows, cols, seed=22)
    X = synth.gen_x(cols, ncols, cfg_id=23)
    H = qg.gateup_silu(G, U, up(env, X.T))
    torch.cuda.synchronize()
    h, th, _, _ = ops.gateup_silu(qtype, graw, uraw, X)
    assert_tol(host(H).T, h, th, "gateup")


# --------------------------------------------------- requantisation to Q8_0
def _src_blocks(src_type, nb, seed):
    """Random source blocks with finite scales of moderate size (the f16
    exponent kept in 2^-14 .. 2^1) and random offsets (Q4_1, Q5_1) or
    sub-block mins (Q4_K, Q5_K) for the types that have one; the rest of
    the bytes (weights, K-quant scale bytes) uniformly random."""
    from oracle import requant as rq
    g = np.random.default_rng(seed)
    raw = g.integers(0, 256, (nb, rq.SRC_BLOCK_BYTES[src_type]), dtype=np.uint8)
    d = (g.uniform(-1.0, 1.0, nb) * 2.0 ** g.integers(-14, 2, nb)).astype(np.float16)
    d_off = 208 if src_type == rq.Q6_K else 0
    raw[:, d_off:d_off + 2] = d.view(np.uint8).reshape(-1, 2)
    if src_type not in (rq.Q5_0, rq.Q6_K):
        m = (g.standard_normal(nb) * 2.0 ** g.integers(-12, 3, nb)).astype(np.float16)
        raw[:, 2:4] = m.view(np.uint8).reshape(-1, 2)
    return raw


def _ktie_block(src_type):
    """A K-quant super-block whose first run has largest magnitude 127 and
    values on exact halves (Q8_0 scale 1, reciprocal exact): Q4_K / Q5_K
    with d = dmin = 0.5, sc_0 = 17, m_0 = 1 (8.5 w - 0.5, w = 0..15 twice);
    Q6_K with d = 1/32, scales 0 and 1 = 127 ((127 / 32)(w - 32), w = 2 l
    mod 64: w = 0 gives -127, w = 16 and 48 give -63.5 and 63.5).  The
    other runs random."""
    from oracle import requant as rq
    b = np.random.default_rng(5).integers(0, 256, rq.SRC_BLOCK_BYTES[src_type]).astype(np.uint8)
    if src_type == rq.Q6_K:
        w = (2 * np.arange(32)) % 64
        b[0:32] = (b[0:32] & 0xF0) | (w & 15)
        b[128:160] = (b[128:160] & 0xFC) | (w >> 4)
        b[192:194] = 127
        b[208:210] = np.array([1.0 / 32], np.float16).view(np.uint8)
        return b
    b[0:4] = np.array([0.5, 0.5], np.float16).view(np.uint8)
    b[4] = (b[4] & 0xC0) | 17
    b[8] = (b[8] & 0xC0) | 1
    q0 = 16 if src_type == rq.Q4_K else 48
    b[q0:q0 + 32] = (b[q0:q0 + 32] & 0xF0) | (np.arange(32) % 16)
    if src_type == rq.Q5_K:
        b[16:48] &= 0xFE
    return b


def _tie_block(src_type):
    """A block whose largest magnitude is 127, so the Q8_0 scale is 1 and
    its reciprocal exact, with values on exact halves: Q4_1 / Q5_1 with
    d = 8.5, m = -0.5 (8.5 n - 0.5, halves at every even n); Q5_0 with
    d = 7.9375 ((w - 16) d, +-63.5 at w = 8 and 24)."""
    from oracle import requant as rq
    b = np.zeros(rq.SRC_BLOCK_BYTES[src_type], np.uint8)
    if src_type == rq.Q5_0:
        b[0:2] = np.array([7.9375], np.float16).view(np.uint8)
        w = np.arange(32)
        qh = 0
        for j in range(32):
            qh |= int(w[j] >> 4) << j
        b[2:6] = np.array([qh], "<u4").view(np.uint8)
        b[6:22] = (w[:16] & 15) | ((w[16:] & 15) << 4)
    else:
        b[0:2] = np.array([8.5], np.float16).view(np.uint8)
        b[2:4] = np.array([-0.5], np.float16).view(np.uint8)
        j = np.arange(16)
        q0 = 4 if src_type == rq.Q4_1 else 8
        b[q0:q0 + 16] = j | ((15 - j) << 4)
    return b


def test_tie_block_has_halves():
    """The planted blocks do put quotients on exact halves (oracle)."""
    from oracle import requant as rq
    for t in (3, 6, 7):
        v = rq.decode_values_f32(t, _tie_block(t)[None, :])[0]
        assert np.max(np.abs(v)) == 127.0
        assert np.any(np.abs(v - np.trunc(v)) == 0.5)
    for t in (12, 13, 14):
        v = rq.decode_values_f32(t, _ktie_block(t)[None, :])[0, :32]
        assert np.max(np.abs(v)) == 127.0
        assert np.any(np.abs(v - np.trunc(v)) == 0.5)


_RQ_SIZES = {3: [1, 255, 256, 257, 1024, 40000], 6: [1, 255, 256, 257, 1024, 40000],
             7: [1, 255, 256, 257, 1024, 40000], 12: [1, 31, 32, 33, 1000, 5000],
             13: [1, 31, 32, 33, 1000, 5000], 14: [1, 31, 32, 33, 1000, 5000]}


@pytest.mark.parametrize("src_type,nb", [(t, n) for t, ns in _RQ_SIZES.items() for n in ns])
def test_requant_bytes_exact(env, src_type, nb):
    """Every output byte equal to the oracle's, including all-zero blocks,
    blocks of one value (Q4_1 / Q5_0 / Q5_1 scale only) or all-zero runs
    (K-quants with zero scales), a block with ties and a tail past a
    workgroup's run (256 blocks; 32 K-quant super-blocks)."""
    torch, qg, dev = env
    from oracle import requant as rq
    raw = _src_blocks(src_type, nb, seed=nb + src_type)
    kq = src_type in (rq.Q4_K, rq.Q5_K, rq.Q6_K)
    if nb > 3:
        raw[1, :] = 0                                  # all zero
        if src_type == rq.Q6_K:
            raw[2, 192:200] = 0                        # runs 0..3 zero
        elif kq:
            raw[2, 4:16] = 0                           # every scale and min zero
        else:
            raw[2, 4:] = 0                             # scale only: every value the offset (or -16 d)
        raw[3] = _ktie_block(src_type) if kq else _tie_block(src_type)
    want = rq.requant_q8_0(src_type, raw)
    nout = want.shape[0]
    got = host(qg.requant_q8_0(src_type, up(env, raw.reshape(-1)), nb)).reshape(nout, 34)
    bad = np.flatnonzero(np.any(got != want, axis=1))
    assert bad.size == 0, (bad[:5], got[bad[:1]], want[bad[:1]])


@pytest.mark.parametrize("src_type", [3, 6, 7, 12, 13, 14])
def test_requant_unaligned(env, src_type):
    """Source and destination 2 bytes past a 16-byte boundary (the 16-bit
    word path) give the same bytes, and nothing outside the output is
    written."""
    torch, qg, dev = env
    from oracle import requant as rq
    nb = 1000 if src_type < 12 else 130
    raw = _src_blocks(src_type, nb, seed=77 + src_type)
    bs = rq.SRC_BLOCK_BYTES[src_type]
    want = rq.requant_q8_0(src_type, raw)
    no = want.size
    sbuf = torch.zeros(nb * bs + 16, dtype=torch.uint8, device=dev)
    sbuf[2:2 + nb * bs] = up(env, raw.reshape(-1))
    dbuf = torch.full((no + 16,), 0xA5, dtype=torch.uint8, device=dev)
    qg.requant_q8_0(src_type, sbuf[2:2 + nb * bs], nb, dbuf[2:2 + no])
    got = dbuf.cpu().numpy()
    assert np.all(got[:2] == 0xA5) and np.all(got[2 + no:] == 0xA5)
    assert np.array_equal(got[2:2 + no].reshape(-1, 34), want)


@pytest.mark.parametrize("src_type", [3, 12, 13, 14])
def test_requant_then_product(env, src_type):
    """The requantised blocks through repack and the GEMV: against the
    oracle's product of the oracle's Q8_0 bytes (the source blocks in row
    order, so each row of 1024 values is 32 Q8_0 blocks)."""
    torch, qg, dev = env
    from oracle import requant as rq
    rows, cols = 300, 1024
    nb = rows * cols // (256 if src_type >= 12 else 32)
    raw = _src_blocks(src_type, nb, seed=9)
    q8d = qg.requant_q8_0(src_type, up(env, raw.reshape(-1)), nb)
    want = rq.requant_q8_0(src_type, raw)
    assert np.array_equal(q8d.cpu().numpy().reshape(-1, 34), want)
    W = qg.qg_repack(Q8, q8d, rows, cols)
    x = synth.gen_x(cols, 2, cfg_id=11)
    Y = qg.qgemv(W, up(env, x.T))
    ref, a = ops.gemv(Q8, want.reshape(rows, cols // 32, 34), x)
    assert_tol(host(Y).T, ref, ops.tol_dot(a), "requant gemv")


# ------------------------------------------------------- RMSNorm prologue
@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(40, 416), (64, 4096), (512, 2048), (300, 5120)])
@pytest.mark.parametrize("ncols", [1, 3, 8])
@pytest.mark.parametrize("xscale", [3.0, 3.0e5])
def test_gateup_rmsnorm_parity(env, qtype, rows, cols, ncols, xscale):
    """gate/up of RMSNorm(X): against the oracle (norm in f64, then the
    products), each column bitwise equal to a 1-column call, and the
    stand-alone norm followed by gateup_silu within the same bound.  At
    xscale 3e5 the un-normalised x * gamma the unit stages reaches ~2e6,
    beyond the f16 range."""
    torch, qg, dev = env
    say(f"gateup rmsnorm qtype={qtype} {rows}x{cols} ncols={ncols} xscale={xscale}")
    graw, G = make(env, qtype, rows, cols, seed=31 + cols)
    uraw, U = make(env, qtype, rows, cols, seed=32 + cols)
    X = (synth.gen_x(cols, ncols, cfg_id=60 + ncols) * xscale).astype(np.float32)
    gam = synth.rng(61, cols).uniform(-2.0, 2.0, cols).astype(np.float32)
    eps = 1e-5
    if xscale > 1e4:
        assert np.max(np.abs(X * gam[:, None])) > 65504
    n = ops.rmsnorm(X.astype(np.float64), gam.astype(np.float64), eps)
    hr, th, _, _ = ops.gateup_silu(qtype, graw, uraw, n)
    gd = up(env, gam)
    H = qg.gateup_silu_rmsnorm(G, U, up(env, X.T), gd, eps)
    torch.cuda.synchronize()
    assert_tol(host(H).T, hr, th, "h")
    for j in range(ncols):
        h1 = qg.gateup_silu_rmsnorm(G, U, up(env, X[:, j:j + 1].T), gd, eps)
        assert torch.equal(h1[0], H[j]), j
    Xn = qg.rmsnorm(up(env, X.T), gd, eps)
    H2 = qg.gateup_silu(G, U, Xn)
    assert_tol(host(H2).T, hr, th, "h via rmsnorm")


@pytest.mark.parametrize("cols,ncols", [(128, 1), (416, 3), (5120, 8), (100, 2)])
def test_rmsnorm_parity(env, cols, ncols):
    """The stand-alone norm against the oracle (f32 bound: the squares' sum,
    the square root and two products), in place as well."""
    torch, qg, dev = env
    X = synth.gen_x(cols, ncols, cfg_id=70 + cols) * 5.0
    gam = synth.rng(71, cols).uniform(-2.0, 2.0, cols).astype(np.float32)
    eps = 1e-6
    ref = ops.rmsnorm(X.astype(np.float64), gam.astype(np.float64), eps)
    Y = host(qg.rmsnorm(up(env, X.T), up(env, gam), eps)).T.astype(np.float64)
    tol = (cols + 16) * 2.0 ** -24 * np.abs(ref) + 1e-30
    assert np.all(np.abs(Y - ref) <= tol)
    Xd = up(env, X.T)
    qg.rmsnorm(Xd, up(env, gam), eps, Y=Xd)
    assert np.array_equal(host(Xd).T.astype(np.float64), Y)


def test_gateup_rmsnorm_unsupported_split(env):
    """cols > 5120 with K split into contiguous segments across workgroups
    (600 x 11264: 22 segments, too many for one workgroup): no unit stages
    all of K, so the fused form refuses (QG_EUNSUPPORTED)."""
    torch, qg, dev = env
    _, G = make(env, Q4, 600, 11264, seed=5)
    _, U = make(env, Q4, 600, 11264, seed=6)
    with pytest.raises(qg.QGError) as e:
        qg.gateup_silu_rmsnorm(G, U, up(env, synth.gen_x(11264, 1, cfg_id=3).T),
                               up(env, np.ones(11264, np.float32)), 1e-6)
    assert e.value.status == -4


# ----------------------------------------------------------------- LM head
def _lm_case(env, qtype, rows, cols, seed, plant=None):
    torch, qg, dev = env
    g = np.random.default_rng(seed)
    raw = synth.gen_weights(qtype, rows, cols, SIG[qtype], g)
    if plant:
        for dst, src in plant:
            raw[dst] = raw[src]
    W = qg.qg_repack(qtype, up(env, raw.reshape(-1)), rows, cols)
    return raw, W


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(40, 416), (1000, 512), (70000, 1024)])
def test_lmhead_argmax_certified(env, qtype, rows, cols):
    torch, qg, dev = env
    say(f"lmhead qtype={qtype} {rows}x{cols}")
    raw, W = _lm_case(env, qtype, rows, cols, seed=rows)
    for s in range(20):
        x = synth.gen_x(cols, 1, cfg_id=1000 + s)[:, 0]
        ref, a = ops.gemv(qtype, raw, x)
        if ops.argmax_certified(ref, a, cols + 64, EPS_OP):
            break
    else:
        pytest.fail("no certified seed")
    idx, val = qg.lmhead_argmax(W, up(env, x))
    torch.cuda.synchronize()
    i = int(idx.item())
    assert i == ops.argmax_first(ref)
    assert abs(val.item() - ref[i]) <= ops.tol_dot(a[i])


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols,k", [(40, 416, 1), (40, 416, 16), (16, 128, 16), (1000, 512, 10),
                                         (70000, 1024, 16)])
def test_lmhead_topk_certified(env, qtype, rows, cols, k):
    """The k candidates, in order, against the oracle on inputs whose order
    the error bound forces (k = 1 is the argmax; k = rows sorts them all)."""
    torch, qg, dev = env
    say(f"lmhead topk qtype={qtype} {rows}x{cols} k={k}")
    raw, W = _lm_case(env, qtype, rows, cols, seed=rows + k)
    for s in range(40):
        x = synth.gen_x(cols, 1, cfg_id=2000 + s)[:, 0]
        want, _, ref, a = ops.lmhead_topk(qtype, raw, x, rows, k)
        if ops.topk_certified(ref, a, k, cols + 64, EPS_OP):
            break
    else:
        pytest.fail("no certified seed")
    idx, val = qg.lmhead_topk(W, up(env, x), k)
    torch.cuda.synchronize()
    check_topk_order(host(idx), host(val), want, ref, a, cols + 64)
    if k == 1:
        i, _ = qg.lmhead_argmax(W, up(env, x))
        assert int(i.item()) == int(host(idx)[0])


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_lmhead_topk_ties_and_prefix(env, qtype):
    """Copies of a top row in other tiles and row groups tie exactly: they
    follow in row order.  Row prefixes (rows < n_rows only) and k = n_rows."""
    torch, qg, dev = env
    rows, cols, k = 5000, 512, 6
    raw = synth.gen_weights(qtype, rows, cols, SIG[qtype], np.random.default_rng(6))
    plant = (17, 4099, rows - 1)
    for s in range(40):
        x = synth.gen_x(cols, 1, cfg_id=75 + s)[:, 0]
        ref, a = ops.gemv(qtype, raw, x)
        top = int(ops.topk_lowest_index(ref, 2)[1])   # the second best row gets the copies
        if top not in plant and ops.topk_certified(ref, a, k, cols + 64, EPS_OP, order=True):
            break
    else:
        pytest.fail("no certified seed")
    for where in plant:
        raw[where] = raw[top]
        ref[where], a[where] = ref[top], a[top]
    W = qg.qg_repack(qtype, up(env, raw.reshape(-1)), rows, cols)
    xd = up(env, x)
    copies = np.array(sorted(set(plant + (top,))))

    def check(n_rows, kk):
        want = ops.topk_lowest_index(ref[:n_rows], kk)
        # certify with each group of bitwise-identical rows counted once
        keep = np.ones(n_rows, bool)
        c = copies[copies < n_rows]
        if len(c):
            keep[c] = False
            keep[c[0]] = True
        sub = np.flatnonzero(keep)
        kk_sub = len(set(want) - set(c[1:]))
        if not ops.topk_certified(ref[sub], a[sub], min(kk_sub, len(sub)), cols + 64, EPS_OP, order=True):
            return False
        idx, _ = qg.lmhead_topk(W, xd, kk, n_rows=n_rows)
        assert list(host(idx).astype(np.int64)) == list(want), (n_rows, kk)
        return True

    assert check(rows, k)
    got = list(host(qg.lmhead_topk(W, xd, k)[0]))
    pos = [got.index(r) for r in copies if r in got]
    assert pos == sorted(pos) and len(pos) == len(copies)
    checked = sum(check(n, k) for n in (k, 17, 18, 4099, 4100, rows - 1)) + check(12, 12)
    assert checked >= 3


def test_lmhead_topk_rejects(env):
    torch, qg, dev = env
    raw, W = _lm_case(env, Q8, 40, 416, seed=3)
    xd = up(env, synth.gen_x(416, 1, cfg_id=9)[:, 0])
    for k, n_rows in ((0, 40), (17, 40), (8, 7)):
        with pytest.raises(qg.QGError) as e:
            qg.lmhead_topk(W, xd, k, n_rows=n_rows)
        assert e.value.status == -2


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_lmhead_planted_ties_and_prefix(env, qtype):
    torch, qg, dev = env
    rows, cols = 5000, 512
    raw = synth.gen_weights(qtype, rows, cols, SIG[qtype], np.random.default_rng(5))
    for s in range(20):
        x = synth.gen_x(cols, 1, cfg_id=55 + s)[:, 0]
        ref, a = ops.gemv(qtype, raw, x)
        top = ops.argmax_first(ref)
        if top not in (17, 4099, rows - 1) and ops.argmax_certified(ref, a, cols + 64, EPS_OP):
            break
    else:
        pytest.fail("no certified seed")
    # identical rows give bitwise-identical logits: copies of the best row in
    # other tiles and row groups, before and after it, and at the last row
    plant = (17, 4099, rows - 1)
    for where in plant:
        raw[where] = raw[top]
        ref[where], a[where] = ref[top], a[top]
    W = qg.qg_repack(qtype, up(env, raw.reshape(-1)), rows, cols)
    xd = up(env, x)
    idx, val = qg.lmhead_argmax(W, xd)
    assert int(idx.item()) == min(17, top)
    # row prefixes (a draft head reads only rows < n_rows)
    copies = np.array(sorted(set(plant + (top,))))
    for n_rows in (1, 17, 18, 4099, 4100, rows - 1, rows):
        want = ops.argmax_first(ref[:n_rows])
        # bitwise-identical rows tie exactly on the GPU too; certify the rest
        keep = np.ones(n_rows, bool)
        if want in copies:
            keep[copies[copies < n_rows]] = False
            keep[want] = True
        sub = np.flatnonzero(keep)
        if not ops.argmax_certified(ref[sub], a[sub], cols + 64, EPS_OP):
            continue
        idx, _ = qg.lmhead_argmax(W, xd, n_rows=n_rows)
        assert int(idx.item()) == want, n_rows
    # all rows identical -> index 0
    raw[:] = raw[3]
    W = qg.qg_repack(qtype, up(env, raw.reshape(-1)), rows, cols)
    idx, _ = qg.lmhead_argmax(W, xd)
    assert int(idx.item()) == 0


# -------------------------------------------------------------------- MoE
def _moe_build(env, E, H, F, k, seed, shared=True, normalize=True, qtype=Q4):
    torch, qg, dev = env
    g = np.random.default_rng(seed)
    sig = SIG[qtype]
    gate = np.stack([synth.gen_weights(qtype, F, H, sig, g) for _ in range(E)])
    upw = np.stack([synth.gen_weights(qtype, F, H, sig, g) for _ in range(E)])
    down = np.stack([synth.gen_weights(qtype, H, F, sig, g) for _ in range(E)])
    router = synth.gen_f32((E, H), 0.02, g)
    sh = None
    if shared:
        sh = tuple(synth.gen_weights(qtype, r, c, sig, g) for r, c in ((F, H), (F, H), (H, F)))
    rep = lambda raw, r, c, n=1: qg.qg_repack(qtype, up(env, raw.reshape(-1)), r, c, n)
    m = qg.MoE(hidden=H, ffn=F, n_expert=E, top_k=k, router=up(env, router),
               gate=rep(gate, F, H, E), up=rep(upw, F, H, E), down=rep(down, H, F, E),
               normalize_topk=normalize)
    if shared:
        m.sh_gate, m.sh_up, m.sh_down = rep(sh[0], F, H), rep(sh[1], F, H), rep(sh[2], H, F)
    return m, (gate, upw, down, router, sh)


def _moe_check(env, m, host_w, T, k, cfg, normalize=True, tries=40, norm=None, xscale=1.0):
    torch, qg, dev = env
    gate, upw, down, router, sh = host_w
    H = m.hidden
    for s in range(tries):
        X = (synth.gen_x(H, T, cfg_id=cfg + 1000 * s) * xscale).astype(np.float32)
        res = ops.moe_ffn(X, router, m.qtype, gate, upw, down, top_k=k, normalize=normalize,
                          sh_gate=None if sh is None else sh[0], sh_up=None if sh is None else sh[1],
                          sh_down=None if sh is None else sh[2],
                          y_in=synth.rng(cfg, 90).standard_normal((H, T)).astype(np.float32),
                          norm_w=None if norm is None else norm[0].astype(np.float64),
                          norm_eps=0.0 if norm is None else norm[1])
        if ops.moe_routing_certified(res, k, H):
            break
    else:
        pytest.fail("no certified routing seed")
    y_in = synth.rng(cfg, 90).standard_normal((H, T)).astype(np.float32)
    Y = up(env, y_in.T)
    tidx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    qg.moe_ffn(m, up(env, X.T), Y, tidx, tw)
    torch.cuda.synchronize()
    check_routing(tidx.cpu().numpy(), tw.cpu().numpy(), res, k, H)
    assert_tol(host(Y).T, res["y"], res["tol"], f"moe T={T}")


@pytest.mark.parametrize("T", [1, 3, 16])
@pytest.mark.parametrize("shared", [True, False])
def test_moe_small(env, T, shared):
    say(f"moe small T={T} shared={shared}")
    m, hw = _moe_build(env, E=16, H=256, F=128, k=4, seed=60 + T, shared=shared)
    _moe_check(env, m, hw, T, 4, cfg=70 + T)


def test_moe_wide_experts(env):
    # experts too wide for the token-major down projection's on-chip h
    # columns: the entry-grouped down path and its cross-workgroup combine
    say("moe wide experts (ffn 11008)")
    m, hw = _moe_build(env, E=6, H=128, F=11008, k=5, seed=85)
    _moe_check(env, m, hw, 3, 5, cfg=86)


@pytest.mark.parametrize("T", [1, 3, 16])
def test_moe_rmsnorm(env, T):
    """The RMSNorm ahead of router and experts (the residual not normalised):
    routing and output against the oracle, on inputs far from unit RMS."""
    torch, qg, dev = env
    say(f"moe rmsnorm T={T}")
    m, hw = _moe_build(env, E=16, H=256, F=128, k=4, seed=95 + T)
    gam = synth.rng(96, 256).uniform(0.5, 1.5, 256).astype(np.float32)
    m.norm_weight, m.norm_eps = up(env, gam), 1e-5
    _moe_check(env, m, hw, T, 4, cfg=97 + T, norm=(gam, 1e-5), xscale=7.0)


@pytest.mark.parametrize("T", [1, 3, 16])
def test_moe_q8_0(env, T):
    """Q8_0 experts (and shared expert): the Q8_0 expert units and the Q8_0
    token-major down projection."""
    say(f"moe q8_0 T={T}")
    m, hw = _moe_build(env, E=16, H=256, F=128, k=4, seed=110 + T, qtype=Q8)
    _moe_check(env, m, hw, T, 4, cfg=111 + T)


@pytest.mark.parametrize("T", [1, 4])
def test_moe_many_experts(env, T):
    """300 experts (more than 256: every lane of the selecting wave holds 5
    logits) with top-8 and a shared expert."""
    say(f"moe 300 experts T={T}")
    m, hw = _moe_build(env, E=300, H=256, F=128, k=8, seed=120 + T)
    _moe_check(env, m, hw, T, 8, cfg=121 + T)


@pytest.mark.parametrize("T", [7, 16])
def test_moe_few_experts(env, T):
    """6 experts, top-2: each router workgroup (16 logits) holds logits of
    up to three tokens and may complete, and select, several of them."""
    say(f"moe 6 experts T={T}")
    m, hw = _moe_build(env, E=6, H=256, F=128, k=2, seed=140 + T)
    _moe_check(env, m, hw, T, 2, cfg=141 + T)


def test_moe_rmsnorm_large_input(env):
    """The MoE norm path with |x * gamma| beyond the f16 range (the expert
    units stage the un-normalised product)."""
    torch, qg, dev = env
    m, hw = _moe_build(env, E=16, H=256, F=128, k=4, seed=130)
    gam = synth.rng(131, 256).uniform(0.5, 1.5, 256).astype(np.float32)
    m.norm_weight, m.norm_eps = up(env, gam), 1e-5
    _moe_check(env, m, hw, 3, 4, cfg=132, norm=(gam, 1e-5), xscale=3.0e5)


def test_moe_unnormalized(env):
    m, hw = _moe_build(env, E=12, H=256, F=128, k=3, seed=80, normalize=False)
    _moe_check(env, m, hw, 5, 3, cfg=81, normalize=False)


def test_moe_repeat_bitwise(env):
    torch, qg, dev = env
    m, hw = _moe_build(env, E=16, H=256, F=128, k=4, seed=90)
    X = up(env, synth.gen_x(256, 16, cfg_id=91).T)
    Y0 = torch.zeros((16, 256), device=dev)
    qg.moe_ffn(m, X, Y0)
    for _ in range(3):
        Y = torch.zeros((16, 256), device=dev)
        qg.moe_ffn(m, X, Y)
        assert torch.equal(Y, Y0)


# ------------------------------------------------------------ launch plans
def _under_plans(env, op, qtype, rows, cols, nc, call, plans):
    """call() (host arrays) with the built-in plan, then under each plan
    pinned strict (None where the call refuses it)."""
    torch, qg, dev = env
    qg.plan_reset()
    base = call()
    out = {}
    try:
        for p in plans:
            qg.plan_set(op, qtype, rows, cols, nc, p | qg.PLAN_STRICT)
            try:
                out[p] = call()
            except qg.QGError as e:
                assert e.status == -4, e            # QG_EUNSUPPORTED, refused before launching
                out[p] = None
    finally:
        qg.plan_reset()
    return base, out


def _same_bits(base, out, may_refuse):
    applied = [p for p, o in out.items() if o is not None]
    say(f"  plans applied {applied}, refused {[p for p in out if p not in applied]}")
    assert len(applied) >= len(out) - len(may_refuse)
    for p, o in out.items():
        if o is None:
            assert p in may_refuse, p
            continue
        for a, b in zip(base, o):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b), p


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(300, 1024), (64, 8192), (2100, 2048), (600, 11264)])
@pytest.mark.parametrize("ncols", [1, 5])
def test_plans_gemv_same_bits(env, qtype, rows, cols, ncols):
    """Every launch plan (4 / 8 / 12 / 16 waves, in-workgroup segments) gives
    the built-in plan's bits, storing and accumulating; only in-workgroup
    segments may be refused, and the result matches the oracle."""
    torch, qg, dev = env
    say(f"plans gemv qtype={qtype} {rows}x{cols} ncols={ncols}")
    raw, W = make(env, qtype, rows, cols, seed=rows + cols + ncols)
    X = synth.gen_x(cols, ncols, cfg_id=rows * 3 + cols)
    Xd = up(env, X.T)
    y0 = synth.rng(5, rows).standard_normal((ncols, rows)).astype(np.float32)

    def call():
        Y = qg.qgemv(W, Xd)
        Ya = qg.qgemv(W, Xd, up(env, y0), accumulate=True)
        return Y.cpu().numpy(), Ya.cpu().numpy()

    plans = [4, 8, 12, 16, qg.PLAN_SW]
    base, out = _under_plans(env, qg.OP_GEMV, qtype, rows, cols, ncols, call, plans)
    _same_bits(base, out, {qg.PLAN_SW})
    ref, a = ops.gemv(qtype, raw, X)
    assert_tol(base[0].astype(np.float64).T, ref, ops.tol_dot(a), "gemv")


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(300, 1024), (2100, 2048)])
def test_plans_gemm16_same_bits(env, qtype, rows, cols):
    torch, qg, dev = env
    say(f"plans gemm16 qtype={qtype} {rows}x{cols}")
    raw, W = make(env, qtype, rows, cols, seed=rows + cols + 16)
    X = synth.gen_x(cols, 16, cfg_id=rows + 5 * cols)
    Xd = up(env, X.T)
    base, out = _under_plans(env, qg.OP_GEMV, qtype, rows, cols, 16,
                             lambda: (qg.qgemm16(W, Xd).cpu().numpy(),), [8, 12, 16])
    _same_bits(base, out, set())


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols,ncols", [(300, 1024, 1), (1000, 5120, 3), (700, 8192, 1)])
def test_plans_gateup_same_bits(env, qtype, rows, cols, ncols):
    torch, qg, dev = env
    say(f"plans gateup qtype={qtype} {rows}x{cols} ncols={ncols}")
    _, G = make(env, qtype, rows, cols, seed=rows + cols + 2)
    _, U = make(env, qtype, rows, cols, seed=rows + cols + 3)
    X = synth.gen_x(cols, ncols, cfg_id=rows + 7 * cols)
    Xd = up(env, X.T)
    base, out = _under_plans(env, qg.OP_GATEUP, qtype, rows, cols, ncols,
                             lambda: (qg.gateup_silu(G, U, Xd).cpu().numpy(),), [4, 8, 12, 16, qg.PLAN_SW])
    _same_bits(base, out, {qg.PLAN_SW})


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols", [(5000, 1024), (300, 2048)])
def test_plans_lmhead_same_bits(env, qtype, rows, cols):
    """Argmax and top-k under every plan: the same rows and value bits."""
    torch, qg, dev = env
    say(f"plans lmhead qtype={qtype} {rows}x{cols}")
    raw, W = _lm_case(env, qtype, rows, cols, seed=rows + cols)
    x = up(env, synth.gen_x(cols, 1, cfg_id=rows)[:, 0])

    def call():
        i, v = qg.lmhead_argmax(W, x)
        ti, tv = qg.lmhead_topk(W, x, 5)
        return i.cpu().numpy(), v.cpu().numpy(), ti.cpu().numpy(), tv.cpu().numpy()

    base, out = _under_plans(env, qg.OP_LMHEAD, qtype, rows, cols, 1, call, [4, 8, 12, 16, qg.PLAN_SW])
    _same_bits(base, out, {qg.PLAN_SW})


def test_tune_keeps_bits_and_fills_the_table(env):
    """The tuners return a candidate plan, store it for the shape, leave the
    built-in plan's outputs, and later calls keep those bits."""
    torch, qg, dev = env
    qg.plan_reset()
    try:
        rows, cols = 2100, 2048
        raw, W = make(env, Q4, rows, cols, seed=31)
        X = up(env, synth.gen_x(cols, 2, cfg_id=3).T)
        base = qg.qgemv(W, X).cpu().numpy()
        p = qg.tune_gemv(W, X)
        say(f"  tuned gemv plan {p}")
        assert p in (0, 4, 8, 12, 16, qg.PLAN_SW)
        assert qg.plan_get(qg.OP_GEMV, Q4, rows, cols, 2) == p
        Y = torch.full((2, rows), 7.0, device=dev)
        qg.tune_gemv(W, X, Y)                         # stores, never accumulates
        assert np.array_equal(Y.cpu().numpy().view(np.uint32), base.view(np.uint32))
        assert np.array_equal(qg.qgemv(W, X).cpu().numpy().view(np.uint32), base.view(np.uint32))

        X16 = up(env, synth.gen_x(cols, 16, cfg_id=4).T)
        b16 = qg.qgemm16(W, X16).cpu().numpy()
        p16 = qg.tune_gemv(W, X16)
        assert p16 in (0, 8, 12, 16)
        assert np.array_equal(qg.qgemm16(W, X16).cpu().numpy().view(np.uint32), b16.view(np.uint32))

        _, G = make(env, Q8, 1000, 5120, seed=32)
        _, U = make(env, Q8, 1000, 5120, seed=34)
        x1 = up(env, synth.gen_x(5120, 1, cfg_id=5).T)
        hb = qg.gateup_silu(G, U, x1).cpu().numpy()
        pg = qg.tune_gateup(G, U, x1)
        assert qg.plan_get(qg.OP_GATEUP, Q8, 1000, 5120, 1) == pg
        assert np.array_equal(qg.gateup_silu(G, U, x1).cpu().numpy().view(np.uint32), hb.view(np.uint32))

        raw3, W3 = _lm_case(env, Q8, 5000, 1024, seed=33)
        x3 = up(env, synth.gen_x(1024, 1, cfg_id=6)[:, 0])
        i0, v0 = (t.cpu().numpy() for t in qg.lmhead_argmax(W3, x3))
        pl = qg.tune_lmhead(W3, x3)
        assert qg.plan_get(qg.OP_LMHEAD, Q8, 5000, 1024, 1) == pl
        i1, v1 = (t.cpu().numpy() for t in qg.lmhead_argmax(W3, x3))
        assert i0[0] == i1[0] and v0.view(np.uint32)[0] == v1.view(np.uint32)[0]
        say(f"  tuned plans: gemv {p}, gemm16 {p16}, gateup {pg}, lmhead {pl}")
    finally:
        qg.plan_reset()


def _split_runs(env, op, qtype, rows, cols, nc, call, splits, layouts=(0,)):
    """call() twice under each pinned strict split: (split, layout, out) for
    those applied; refusals must be for room (workspace) or layout."""
    torch, qg, dev = env
    done = []
    qg.plan_reset()
    try:
        for sp in splits:
            for lay in layouts:
                qg.plan_set(op, qtype, rows, cols, nc, qg.PLAN_SPLIT(sp) | lay | qg.PLAN_STRICT)
                try:
                    a, b = call(), call()
                except qg.QGError as e:
                    assert e.status in (-4, -5), e
                    continue
                for u, v in zip(a, b):
                    assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), (sp, lay)
                done.append((sp, lay, a))
    finally:
        qg.plan_reset()
    say(f"  splits applied {[(s, l) for s, l, _ in done]}")
    return done


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("rows,cols,ncols", [(2100, 2048, 1), (64, 8192, 3), (600, 11264, 1)])
def test_split_plans_gemv(env, qtype, rows, cols, ncols):
    """K splits pinned per shape: within the oracle's tolerance, the same bits
    on repeat calls, storing and accumulating."""
    torch, qg, dev = env
    say(f"split gemv qtype={qtype} {rows}x{cols} ncols={ncols}")
    raw, W = make(env, qtype, rows, cols, seed=rows + 3 * cols)
    X = synth.gen_x(cols, ncols, cfg_id=rows + 11)
    Xd = up(env, X.T)
    y0 = synth.rng(6, rows).standard_normal((ncols, rows)).astype(np.float32)
    done = _split_runs(env, qg.OP_GEMV, qtype, rows, cols, ncols,
                       lambda: (qg.qgemv(W, Xd).cpu().numpy(),
                                qg.qgemv(W, Xd, up(env, y0), accumulate=True).cpu().numpy()),
                       [1, 2, 3, 4, 6, 8], (0, 8))
    assert len(done) >= 4
    ref, a = ops.gemv(qtype, raw, X)
    for sp, lay, (Y, Ya) in done:
        assert_tol(Y.astype(np.float64).T, ref, ops.tol_dot(a), f"split {sp} lay {lay}")
        ya = ref + y0.T.astype(np.float64)
        assert_tol(Ya.astype(np.float64).T, ya, ops.tol_dot(a, ya), f"split {sp} lay {lay} acc")


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_split_plans_gemm16_and_gateup(env, qtype):
    torch, qg, dev = env
    rows, cols = 2100, 2048
    raw, W = make(env, qtype, rows, cols, seed=71)
    X = synth.gen_x(cols, 16, cfg_id=72)
    Xd = up(env, X.T)
    done = _split_runs(env, qg.OP_GEMV, qtype, rows, cols, 16, lambda: (qg.qgemm16(W, Xd).cpu().numpy(),),
                       [1, 2, 4], (0, 12))
    assert len(done) >= 3
    ref, a = ops.gemv(qtype, raw, X)
    for sp, lay, (Y,) in done:
        assert_tol(Y.astype(np.float64).T, ref, ops.tol_dot(a), f"gemm16 split {sp}")
    graw, G = make(env, qtype, 1000, 5120, seed=73)
    uraw, U = make(env, qtype, 1000, 5120, seed=74)
    x = synth.gen_x(5120, 1, cfg_id=75)
    xd = up(env, x.T)
    done = _split_runs(env, qg.OP_GATEUP, qtype, 1000, 5120, 1, lambda: (qg.gateup_silu(G, U, xd).cpu().numpy(),),
                       [1, 2, 3, 6], (0, qg.PLAN_SW))
    assert len(done) >= 3
    h, th, _, _ = ops.gateup_silu(qtype, graw, uraw, x)
    for sp, lay, (H,) in done:
        assert_tol(H.astype(np.float64).T, h, th, f"gateup split {sp}")


def test_tune_with_splits(env):
    """Tuning over K splits too: the kept plan's results stay within the
    oracle's tolerance and repeat bitwise."""
    torch, qg, dev = env
    qg.plan_reset()
    try:
        rows, cols = 1200, 8192
        raw, W = make(env, Q4, rows, cols, seed=81)
        X = synth.gen_x(cols, 1, cfg_id=82)
        Xd = up(env, X.T)
        p = qg.tune_gemv(W, Xd, split=True)
        say(f"  tuned with splits: plan {p:#x}")
        lay, sp = p & ~(0xFF << 12), (p >> 12) & 0xFF
        assert lay in (0, 4, 8, 12, 16, qg.PLAN_SW) and sp >= 0
        assert qg.plan_get(qg.OP_GEMV, Q4, rows, cols, 1) == p
        Y1, Y2 = qg.qgemv(W, Xd).cpu().numpy(), qg.qgemv(W, Xd).cpu().numpy()
        assert np.array_equal(Y1.view(np.uint32), Y2.view(np.uint32))
        ref, a = ops.gemv(Q4, raw, X)
        assert_tol(Y1.astype(np.float64).T, ref, ops.tol_dot(a), "tuned split gemv")
    finally:
        qg.plan_reset()


def test_graph_replay_decode_step(env):
    """The decode step (residual reset by a copy, gate/up, down accumulating)
    captured in a HIP graph: every replay, with eager calls on the same
    workspace between replays, gives the eager result bitwise; also with a
    plan pinned for the down projection (read when the graph is captured).
    Between capture and the replays an eager call of a larger shape on the
    capture stream grows that stream's workspace: the graph keeps the one
    it captured, which stays allocated."""
    torch, qg, dev = env
    F, Hd = 1024, 2048
    _, G = make(env, Q4, F, Hd, seed=91)
    _, U = make(env, Q4, F, Hd, seed=92)
    _, D = make(env, Q4, Hd, F, seed=93)
    _, Big = make(env, Q4, 8192, 16384, seed=98)
    xb = up(env, synth.gen_x(16384, 8, cfg_id=99).T)
    x = up(env, synth.gen_x(Hd, 1, cfg_id=9).T)
    y0 = up(env, synth.rng(94, Hd).standard_normal((1, Hd)).astype(np.float32))
    h = torch.empty((1, F), device=dev)
    y = torch.empty((1, Hd), device=dev)
    spare = torch.empty((1, Hd), device=dev)

    def step():
        y.copy_(y0)
        qg.gateup_silu(G, U, x, h)
        qg.qgemv(D, h, y, accumulate=True)

    try:
        for pin in (None, 8):
            qg.plan_reset()
            if pin:
                qg.plan_set(qg.OP_GEMV, Q4, Hd, F, 1, pin | qg.PLAN_STRICT)
            step()
            torch.cuda.synchronize()
            want_h, want_y = h.cpu().numpy().copy(), y.cpu().numpy().copy()
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                step()                         # the capture stream's workspace, made eagerly
                with torch.cuda.graph(g, stream=s):
                    step()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                before = qg.workspace(0, dev).data_ptr()
                qg.qgemv(Big, xb)              # needs a larger workspace than the graph's
                assert qg.workspace(0, dev).data_ptr() != before
            torch.cuda.synchronize()
            for r in range(3):
                h.zero_()
                y.zero_()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                assert np.array_equal(h.cpu().numpy().view(np.uint32), want_h.view(np.uint32)), (pin, r)
                assert np.array_equal(y.cpu().numpy().view(np.uint32), want_y.view(np.uint32)), (pin, r)
                with torch.cuda.stream(s):
                    qg.qgemv(D, h, spare)      # eager work on the capture stream's workspace between replays
                    qg.qgemv(Big, xb)
                torch.cuda.synchronize()
            say(f"  graph replays equal eager (plan {pin})")
            del g
    finally:
        qg.plan_reset()


@pytest.mark.parametrize("T", [1, 3])
def test_graph_replay_moe(env, T):
    """The MoE layer (router counters, work list, expert units) captured in a
    HIP graph: every replay, with an eager layer call on the same workspace
    between replays, gives the eager result bitwise."""
    torch, qg, dev = env
    m, _ = _moe_build(env, 16, 256, 128, 4, seed=95)
    X = up(env, synth.gen_x(256, T, cfg_id=96).T)
    y0 = up(env, synth.rng(97, 256).standard_normal((T, 256)).astype(np.float32))
    Y = torch.empty((T, 256), device=dev)
    Ys = torch.empty((T, 256), device=dev)
    ti = torch.empty((T, 4), dtype=torch.int32, device=dev)

    def layer():
        Y.copy_(y0)
        qg.moe_ffn(m, X, Y, ti)

    layer()
    torch.cuda.synchronize()
    want_y, want_i = Y.cpu().numpy().copy(), ti.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()                             # the capture stream's workspace, made eagerly
        with torch.cuda.graph(g, stream=s):
            layer()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        Y.zero_()
        ti.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().view(np.uint32), want_y.view(np.uint32)), r
        assert np.array_equal(ti.cpu().numpy(), want_i), r
        with torch.cuda.stream(s):
            Ys.copy_(y0)
            qg.moe_ffn(m, X, Ys)            # eager layer on the capture stream's workspace between replays
        torch.cuda.synchronize()
    say(f"  moe graph replays equal eager (T={T})")
