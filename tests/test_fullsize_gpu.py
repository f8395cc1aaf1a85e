"""GPU parity at the benchmarked sizes, in the launch configurations the bench
times (the launch plan depends on the shape and the column count only).

* decode FFN layer, batch 1: gate/up Q4_0 5120 -> 2 x 17408 with SiLU, then
  down Q4_0 17408 -> 5120 accumulated into the residual, end to end; the
  gate/up with the RMSNorm of x folded in, and after the stand-alone norm;
* speculative-verify GEMVs, 4 and 8 columns: Q8_0 5120 x 5120, Q4_0
  5120 -> 17408;
* 16-column prefill GEMMs, Q4_0 and Q8_0, 5120 -> 17408 and 17408 -> 5120;
* LM head Q8_0 5120 -> 248,320 with argmax (and a 65,536-row draft prefix);
* MoE FFN, 256 experts of 2048 -> 512 -> 2048 (top-8) + shared expert,
  1 and 16 tokens, plain and with the RMSNorm of x folded in.
* load-time requantisation to Q8_0 of a 17408 x 5120 matrix held as Q4_1
  blocks and as Q4_K and Q6_K super-blocks (every output byte).

Every output element is checked against the f64 oracle (these sizes run in
seconds on the host); indices bit-exact where the oracle certifies them.
Weights and activations are drawn exactly as the bench draws them.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import EPS_OP, assert_tol, check_routing, check_topk_order, host, say, up
from oracle import ops

pytestmark = pytest.mark.gpu

Q4, Q8 = synth.Q4_0, synth.Q8_0
SIG = {Q4: 0.02, Q8: 0.005}


def matrix(env, qtype, rows, cols, seed):
    _, qg, _ = env
    raw = synth.gen_weights(qtype, rows, cols, SIG[qtype], np.random.default_rng(seed))
    return raw, qg.qg_repack(qtype, up(env, raw.reshape(-1)), rows, cols)


def test_decode_ffn_layer(env):
    torch, qg, dev = env
    N, K = 17408, 5120
    say(f"decode FFN gate/up {K}->2x{N}, down {N}->{K}, batch 1")
    graw, G = matrix(env, Q4, N, K, 21)
    uraw, U = matrix(env, Q4, N, K, 22)
    draw, D = matrix(env, Q4, K, N, 23)
    x = synth.gen_x(K, 1, cfg_id=synth.CFG_FFN)
    y_in = synth.rng(synth.CFG_FFN, 90).standard_normal((K, 1)).astype(np.float32)
    H = qg.gateup_silu(G, U, up(env, x.T))
    Y = up(env, y_in.T)
    qg.qgemv(D, H, Y, accumulate=True)
    torch.cuda.synchronize()
    h, th, _, _ = ops.gateup_silu(Q4, graw, uraw, x)
    assert_tol(host(H).T, h, th, "h = silu(Wg x) * (Wu x)")
    y, _ = ops.gemv(Q4, draw, h, y_in=y_in)
    ty = ops.down_tol(Q4, draw, h, th) + 2 * ops.U32 * np.abs(y)
    assert_tol(host(Y).T, y, ty, "y += Wd h")


def test_decode_gateup_rmsnorm(env):
    """gate/up Q4_0 5120 -> 2 x 17408 of RMSNorm(x) at batch 1, as the bench
    times it (gamma uniform in [0.5, 1.5], eps 1e-6): the folded call and the
    stand-alone norm followed by gate/up, both against the oracle (the norm
    in f64, then the products)."""
    torch, qg, dev = env
    N, K = 17408, 5120
    say(f"decode gate/up with RMSNorm {K}->2x{N}, batch 1")
    graw, G = matrix(env, Q4, N, K, 21)
    uraw, U = matrix(env, Q4, N, K, 22)
    x = synth.gen_x(K, 1, cfg_id=synth.CFG_FFN)
    gam = synth.rng(3, K).uniform(0.5, 1.5, K).astype(np.float32)
    n = ops.rmsnorm(x.astype(np.float64), gam.astype(np.float64), 1e-6)
    h, th, _, _ = ops.gateup_silu(Q4, graw, uraw, n)
    gd = up(env, gam)
    H = qg.gateup_silu_rmsnorm(G, U, up(env, x.T), gd, 1e-6)
    H2 = qg.gateup_silu(G, U, qg.rmsnorm(up(env, x.T), gd, 1e-6))
    torch.cuda.synchronize()
    assert_tol(host(H).T, h, th, "h = silu(Wg n) * (Wu n), norm folded")
    assert_tol(host(H2).T, h, th, "h after the stand-alone norm")


@pytest.mark.parametrize("qtype,N,K", [(Q8, 5120, 5120), (Q4, 17408, 5120)])
@pytest.mark.parametrize("ncols", [4, 8])
def test_verify_gemv(env, qtype, N, K, ncols):
    torch, qg, dev = env
    say(f"verify qtype={qtype} {K}->{N} ncols={ncols}")
    raw, W = matrix(env, qtype, N, K, 31)
    X = synth.gen_x(K, ncols, cfg_id=synth.CFG_VERIFY)
    Xd = up(env, X.T)
    Y = qg.qgemv(W, Xd)
    torch.cuda.synchronize()
    ref, a = ops.gemv(qtype, raw, X)
    assert_tol(host(Y).T, ref, ops.tol_dot(a), "verify")
    # column j of the batched product equals the 1-column product, bitwise
    for j in range(ncols):
        assert torch.equal(Y[j], qg.qgemv(W, Xd[j:j + 1].contiguous())[0]), j


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408)])
def test_prefill_gemm16(env, qtype, N, K):
    torch, qg, dev = env
    say(f"gemm16 qtype={qtype} {K}->{N}")
    raw, W = matrix(env, qtype, N, K, 41)
    X = synth.gen_x(K, 16, cfg_id=synth.CFG_PREFILL)
    Y = qg.qgemm16(W, up(env, X.T))
    torch.cuda.synchronize()
    ref, a = ops.gemv(qtype, raw, X)
    assert_tol(host(Y).T, ref, ops.tol_dot(a), "gemm16")


def test_prefill_pass_batch(env):
    """One prefill pass of the 16-column workload as one launch: Q4_0 and
    Q8_0 at 5120 -> 17408 and 17408 -> 5120, each output bitwise equal to its
    qgemm16 call with the launch's K split pinned, and rows sampled across
    every row tile group checked against the oracle."""
    torch, qg, dev = env
    probs, raws = [], []
    for i, (qt, N, K) in enumerate([(Q4, 17408, 5120), (Q4, 5120, 17408), (Q8, 17408, 5120), (Q8, 5120, 17408)]):
        raw, W = matrix(env, qt, N, K, 45 + i)
        X = synth.gen_x(K, 16, cfg_id=synth.CFG_PREFILL, col0=16 * i)
        probs.append((W, up(env, X.T), None, 0))
        raws.append((qt, raw, X))
    splits = qg.gemm16_batch_splits(probs)
    say(f"prefill pass: 4 matrices in one launch, K splits {splits}")
    assert splits == [1, 3, 1, 3]   # segments as long as the shortest K; 512 units (2 per CU)
    outs = qg.qgemm16_batch(probs)
    try:
        for (W, _, _, _), sp in zip(probs, splits):
            qg.plan_set(qg.OP_GEMV, W.qtype, W.rows, W.cols, 16, qg.PLAN_SPLIT(sp) | qg.PLAN_STRICT)
        single = [qg.qgemm16(W, X) for W, X, _, _ in probs]
    finally:
        qg.plan_reset()
    torch.cuda.synchronize()
    g = np.random.default_rng(46)
    for i, (W, X, _, _) in enumerate(probs):
        assert torch.equal(outs[i], single[i]), i
        qt, raw, Xh = raws[i]
        rows = np.unique(np.concatenate([g.integers(0, W.rows, 600), [0, W.rows - 1]]))
        ref, a = ops.gemv(qt, raw, Xh, rows=rows)
        assert_tol(host(outs[i])[:, rows].T, ref, ops.tol_dot(a), f"pass problem {i}")


def test_lmhead_argmax_full_vocabulary(env):
    torch, qg, dev = env
    N, K = 248320, 5120
    say(f"LM head Q8_0 {K}->{N}")
    raw, W = matrix(env, Q8, N, K, 51)
    X = synth.gen_x(K, 8, cfg_id=synth.CFG_PREFILL)   # column 0 is the bench's x
    ref, a = ops.gemv(Q8, raw, X)
    cols = [j for j in range(8) if ops.argmax_certified(ref[:, j], a[:, j], K + 64, EPS_OP)]
    say(f"  certified columns: {cols}")
    assert cols, "no certified column"
    checked_prefix = 0
    for j in cols[:3]:
        xd = up(env, X[:, j])
        idx, val = qg.lmhead_argmax(W, xd)
        torch.cuda.synchronize()
        i = int(idx.item())
        assert i == ops.argmax_first(ref[:, j]), (j, i)
        assert abs(val.item() - ref[i, j]) <= ops.tol_dot(a[i, j])
        n = 65536
        if ops.argmax_certified(ref[:n, j], a[:n, j], K + 64, EPS_OP):
            idx, _ = qg.lmhead_argmax(W, xd, n_rows=n)
            assert int(idx.item()) == ops.argmax_first(ref[:n, j]), (j, "prefix")
            checked_prefix += 1
    assert checked_prefix, "no certified draft prefix"


def test_lmhead_topk_full_vocabulary(env):
    """The full LM head.  Natural inputs: the largest k of 10 (the size the
    Three.js page's example asks for), 8, 4 whose set the error bound forces
    on one of 24 input columns.  Planted: the best row copied to 20 rows
    spread over the vocabulary, each copy's block scales multiplied by 3,
    3.25, 3.5, ..., so that k = 10 and k = 16 candidates come from many row
    groups in a forced order."""
    torch, qg, dev = env
    N, K = 248320, 5120
    say(f"LM head top-k Q8_0 {K}->{N}")
    raw, W = matrix(env, Q8, N, K, 51)
    X = np.concatenate([synth.gen_x(K, 8, cfg_id=synth.CFG_PREFILL), synth.gen_x(K, 16, cfg_id=61)], axis=1)
    ref, a = ops.gemv(Q8, raw, X)
    found = None
    for k in (10, 8, 4):
        for j in range(X.shape[1]):
            if ops.topk_certified(ref[:, j], a[:, j], k, K + 64, EPS_OP):
                found = (k, j)
                break
        if found:
            break
    assert found, "no certified column"
    k, j = found
    say(f"  natural inputs: k = {k}, column {j}")
    idx, val = qg.lmhead_topk(W, up(env, X[:, j]), k)
    torch.cuda.synchronize()
    check_topk_order(host(idx), host(val), ops.topk_lowest_index(ref[:, j], k), ref[:, j], a[:, j], K + 64)
    del W
    x = X[:, 0]
    best = ops.argmax_first(ref[:, 0])
    rows = np.linspace(3, N - 1, 20).astype(np.int64)
    src = raw[best].copy()
    for i, r in enumerate(rows):
        blk = src.copy()
        d = blk[:, 0:2].copy().view(np.float16)
        blk[:, 0:2] = (d.astype(np.float32) * np.float32(3.0 + 0.25 * i)).astype(np.float16).view(np.uint8)
        raw[r] = blk
    W = qg.qg_repack(Q8, up(env, raw.reshape(-1)), N, K)
    ref, a = ops.gemv(Q8, raw, x)
    for k in (10, 16):
        assert ops.topk_certified(ref, a, k, K + 64, EPS_OP, order=True)
        idx, val = qg.lmhead_topk(W, up(env, x), k)
        torch.cuda.synchronize()
        want = ops.topk_lowest_index(ref, k)
        assert set(int(r) for r in want) <= set(int(r) for r in rows)
        check_topk_order(host(idx), host(val), want, ref, a, K + 64)
        assert list(host(idx).astype(np.int64)) == list(want)


@pytest.fixture(scope="module")
def moe_full(env):
    """The MoE layer exactly as the bench draws it."""
    torch, qg, dev = env
    E, H, F = 256, 2048, 512
    g = np.random.default_rng(61)
    stack = lambda r, c: np.stack([synth.gen_weights(Q4, r, c, 0.02, g) for _ in range(E)])
    gate, upw, down = stack(F, H), stack(F, H), stack(H, F)
    sh = [synth.gen_weights(Q4, r, c, 0.02, np.random.default_rng(62 + i))
          for i, (r, c) in enumerate(((F, H), (F, H), (H, F)))]
    router = synth.gen_f32((E, H), 0.02, g)
    rep = lambda raw, r, c, n=1: qg.qg_repack(Q4, up(env, raw.reshape(-1)), r, c, n)
    m = qg.MoE(hidden=H, ffn=F, n_expert=E, top_k=8, router=up(env, router),
               gate=rep(gate, F, H, E), up=rep(upw, F, H, E), down=rep(down, H, F, E),
               sh_gate=rep(sh[0], F, H), sh_up=rep(sh[1], F, H), sh_down=rep(sh[2], H, F))
    return m, (gate, upw, down, router, sh)


@pytest.mark.parametrize("T", [1, 16])
def test_moe_full_layer(env, moe_full, T):
    torch, qg, dev = env
    m, (gate, upw, down, router, sh) = moe_full
    H, k = m.hidden, m.top_k
    say(f"MoE 256 experts top-8 + shared, hidden 2048, ffn 512, T={T}")
    # the bench's tokens first, then later seeds until the oracle certifies
    # every token's selected set
    for c in range(0, 64 * T, T):
        X = synth.gen_x(H, T, cfg_id=synth.CFG_MOE, col0=c)
        lg, la = ops.router_logits(X, router)
        if np.all(ops.routing_certified(lg, la, k, H)):
            break
    else:
        pytest.fail("no certified routing")
    say(f"  tokens from column {c}")
    y_in = synth.rng(synth.CFG_MOE, 90).standard_normal((H, T)).astype(np.float32)
    Y = up(env, y_in.T)
    tidx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    qg.moe_ffn(m, up(env, X.T), Y, tidx, tw)
    torch.cuda.synchronize()
    res = ops.moe_ffn(X, router, Q4, gate, upw, down, top_k=k,
                      sh_gate=sh[0], sh_up=sh[1], sh_down=sh[2], y_in=y_in)
    n_ord = check_routing(tidx.cpu().numpy(), tw.cpu().numpy(), res, k, H)
    say(f"  routing: {T} tokens, order certified for {n_ord}")
    assert_tol(host(Y).T, res["y"], res["tol"], f"moe T={T}")


@pytest.mark.parametrize("T", [1, 16])
def test_moe_full_layer_rmsnorm(env, moe_full, T):
    """The layer with the RMSNorm of x folded in ahead of router and experts,
    as the bench times it (gamma uniform in [0.5, 1.5], eps 1e-6; the
    residual not normalised), and the stand-alone norm followed by the plain
    layer: routing and output against the oracle, whose norm is in f64."""
    torch, qg, dev = env
    m, (gate, upw, down, router, sh) = moe_full
    H, k = m.hidden, m.top_k
    say(f"MoE with RMSNorm, 256 experts top-8 + shared, T={T}")
    gam = synth.rng(63, H).uniform(0.5, 1.5, H).astype(np.float32)
    y_in = synth.rng(synth.CFG_MOE, 90).standard_normal((H, T)).astype(np.float32)
    # the bench's tokens first, then later seeds until the oracle certifies
    # every token's selected set
    for c in range(0, 64 * T, T):
        X = synth.gen_x(H, T, cfg_id=synth.CFG_MOE, col0=c)
        _, lg, la = ops.moe_router(X, router, gam.astype(np.float64), 1e-6)
        if np.all(ops.routing_certified(lg, la, k, H)):
            break
    else:
        pytest.fail("no certified routing")
    say(f"  tokens from column {c}")
    res = ops.moe_ffn(X, router, Q4, gate, upw, down, top_k=k, sh_gate=sh[0], sh_up=sh[1],
                      sh_down=sh[2], y_in=y_in, norm_w=gam.astype(np.float64), norm_eps=1e-6)
    Y = up(env, y_in.T)
    tidx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    m.norm_weight, m.norm_eps = up(env, gam), 1e-6
    try:
        qg.moe_ffn(m, up(env, X.T), Y, tidx, tw)
        torch.cuda.synchronize()
    finally:
        m.norm_weight = None
    n_ord = check_routing(tidx.cpu().numpy(), tw.cpu().numpy(), res, k, H)
    say(f"  routing: {T} tokens, order certified for {n_ord}")
    assert_tol(host(Y).T, res["y"], res["tol"], f"moe with norm T={T}")
    # the stand-alone norm, then the plain layer
    Y2 = up(env, y_in.T)
    qg.moe_ffn(m, qg.rmsnorm(up(env, X.T), up(env, gam), 1e-6), Y2, tidx, tw)
    torch.cuda.synchronize()
    check_routing(tidx.cpu().numpy(), tw.cpu().numpy(), res, k, H)
    assert_tol(host(Y2).T, res["y"], res["tol"], f"rmsnorm then moe T={T}")


@pytest.mark.parametrize("src_type", [3, 12, 14])
def test_requant_full_matrix(env, src_type):
    """A 17408 x 5120 matrix (89,128,960 values) of Q4_1 blocks or Q4_K / Q6_K
    super-blocks requantised to Q8_0 as the bench times it (one call over all
    blocks), drawn by the bench's recipe: uniformly random bytes with each f16
    scale's high byte set to 0x3C (scales near 1; Q4_1 offsets near -1, Q4_K
    mins near 1).  Every one of the 2,785,280 output blocks equal, byte for
    byte, to the oracle's."""
    torch, qg, dev = env
    from oracle import requant as rq
    bs, nv = rq.SRC_BLOCK_BYTES[src_type], rq.SRC_BLOCK_VALUES[src_type]
    nb = 17408 * 5120 // nv
    raw = np.random.default_rng(90 + src_type).integers(0, 256, (nb, bs), dtype=np.uint8)
    d_off = 208 if src_type == rq.Q6_K else 0
    raw[:, d_off + 1] = 0x3C
    if src_type == rq.Q4_1:
        raw[:, 3] = 0xBC
    elif src_type == rq.Q4_K:
        raw[:, 3] = 0x3C
    say(f"requant full matrix: type {src_type}, {nb} source blocks")
    got = qg.requant_q8_0(src_type, up(env, raw.reshape(-1)), nb).cpu().numpy().reshape(-1, 34)
    want = rq.requant_q8_0(src_type, raw)
    assert got.shape == want.shape
    bad = np.flatnonzero(np.any(got != want, axis=1))
    assert bad.size == 0, (bad.size, bad[:5], got[bad[:1]], want[bad[:1]])
