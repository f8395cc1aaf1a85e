"""C-ABI checks that need no GPU: every declared symbol is exported, the
size queries, and every argument check (each returns before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import gemm_q4_q8_amd as qg
from oracle import quant
from tests.conftest import ROOT

L = qg.lib
OK, EINVAL, ESHAPE, EALIGN, EUNSUP, EWS = 0, -1, -2, -3, -4, -5
FAKE = 1 << 40          # an aligned, never-dereferenced "device" address


def _declared():
    src = open(os.path.join(ROOT, "include", "qgemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char|void)\s*\*?\s*(\w+)\s*\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"qgemv_q4_0", "qgemv_q8_0", "qgemm16", "gateup_silu", "moe_ffn",
            "lmhead_argmax", "lmhead_topk", "gateup_silu_rmsnorm", "qg_rmsnorm", "qg_requant_q8_0",
            "qg_repack", "qg_packed_bytes"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_strerror():
    for s in (0, -1, -2, -3, -4, -5, -6, 7):
        assert isinstance(L.qg_strerror(s), bytes) and L.qg_strerror(s)


@pytest.mark.parametrize("qtype", [qg.Q4_0, qg.Q8_0])
@pytest.mark.parametrize("n_mat,rows,cols", [(1, 2048, 2048), (1, 20, 160), (3, 512, 2048), (1, 248320, 5120)])
def test_packed_bytes_match_layout_definition(qtype, n_mat, rows, cols):
    assert qg.packed_bytes(qtype, rows, cols, n_mat) == quant.packed_bytes(qtype, n_mat, rows, cols)


def test_packed_bytes_exact_sizes_for_whole_tiles():
    # 17408 x 5120 Q4_0: 44,564,480 weight bytes + 5,570,560 scale bytes (18 B per 32 weights)
    assert qg.packed_bytes(qg.Q4_0, 17408, 5120) == (44564480, 5570560)
    assert sum(qg.packed_bytes(qg.Q8_0, 248320, 5120)) == 248320 * 5120 // 32 * 34


def test_packed_bytes_rejects():
    qb, db = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.qg_packed_bytes(3, 1, 16, 32, ctypes.byref(qb), ctypes.byref(db)) == EINVAL
    assert L.qg_packed_bytes(2, 1, 16, 33, ctypes.byref(qb), ctypes.byref(db)) == ESHAPE
    assert L.qg_packed_bytes(2, 0, 16, 32, ctypes.byref(qb), ctypes.byref(db)) == ESHAPE
    assert L.qg_packed_bytes(2, 1, 16, 32, None, ctypes.byref(db)) == EINVAL


def test_ws_queries():
    assert L.qg_gemv_ws_bytes(5120, 17408) > 0
    assert L.qg_gemv_ws_bytes(5120, 17) == 0
    # 16 columns hold at least the partials of 8 (4 values per lane either way)
    assert L.qg_gemm16_ws_bytes(2, 5120, 17408) >= L.qg_gemv_ws_bytes(5120, 17408)
    assert L.qg_gateup_ws_bytes(17408, 5120) >= L.qg_gemv_ws_bytes(17408, 5120)
    assert L.qg_lmhead_ws_bytes(248320, 5120) > 0


def test_ws_queries_cover_the_counter_prefix():
    # every workspace starts with the shared counters the header declares
    hdr = open(os.path.join(ROOT, "include", "qgemm.h")).read()
    sync = int(re.search(r"#define QG_WS_SYNC_BYTES (\d+)u", hdr).group(1))
    assert sync % 256 == 0
    for q in (L.qg_gemv_ws_bytes(2048, 2048), L.qg_gemv_ws_bytes(16, 128),
              L.qg_gemm16_ws_bytes(8, 5120, 17408), L.qg_gateup_ws_bytes(512, 2048),
              L.qg_lmhead_ws_bytes(248320, 5120), L.qg_moe_ws_bytes(ctypes.byref(_moe()), 1)):
        assert q >= sync


def _gemv(**kw):
    a = dict(qs=FAKE, d=FAKE, rows=64, cols=128, X=FAKE + (1 << 20), ldx=128, ncols=1,
             Y=FAKE + (2 << 20), ldy=64, acc=0, ws=FAKE + (3 << 20), wsb=1 << 20, stream=None)
    a.update(kw)
    return L.qgemv_q4_0(a["qs"], a["d"], a["rows"], a["cols"], a["X"], a["ldx"], a["ncols"],
                        a["Y"], a["ldy"], a["acc"], a["ws"], a["wsb"], a["stream"])


def test_gemv_argument_checks():
    assert _gemv(qs=None) == EINVAL
    assert _gemv(d=None) == EINVAL
    assert _gemv(X=None) == EINVAL
    assert _gemv(Y=None) == EINVAL
    assert _gemv(cols=100) == ESHAPE
    assert _gemv(rows=0) == ESHAPE
    assert _gemv(ncols=0) == ESHAPE
    assert _gemv(ncols=9) == ESHAPE
    assert _gemv(ldx=64) == ESHAPE
    assert _gemv(ldy=10) == ESHAPE
    assert _gemv(qs=FAKE + 8) == EALIGN
    assert _gemv(d=FAKE + 4) == EALIGN
    assert _gemv(X=FAKE + (1 << 20) + 4) == EALIGN
    assert _gemv(ldx=130) == EALIGN
    assert _gemv(Y=FAKE + (2 << 20) + 2) == EALIGN
    assert _gemv(ws=None) == EWS
    assert _gemv(wsb=16) == EWS
    assert _gemv(ws=FAKE + (3 << 20) + 16) == EALIGN
    # output overlapping the input
    assert _gemv(Y=FAKE + (1 << 20) + 64) == EINVAL


def test_gemm16_batch_checks():
    P = qg.qg_gemm16_problem
    X0, Y0, X1, Y1 = (FAKE + (k << 24) for k in (1, 2, 3, 4))

    def arr(*probs):
        a = (P * max(len(probs), 1))()
        for i, p in enumerate(probs):
            a[i] = p
        return a

    good = [P(2, 0, FAKE, FAKE, 64, 128, X0, 128, Y0, 64), P(8, 1, FAKE, FAKE, 100, 256, X1, 256, Y1, 100)]
    a = arr(*good)
    wsb = L.qg_gemm16_batch_ws_bytes(a, 2)
    assert wsb >= 262144
    ws = FAKE + (7 << 24)
    # sizes grow with the problems, and one problem of the pair needs less
    assert L.qg_gemm16_batch_ws_bytes(a, 1) <= wsb
    assert L.qgemm16_batch(None, 2, ws, wsb, None) == EINVAL
    assert L.qgemm16_batch(a, 0, ws, wsb, None) == ESHAPE
    assert L.qgemm16_batch(arr(*(good * 5)), 9, ws, 1 << 30, None) == ESHAPE
    assert L.qg_gemm16_batch_ws_bytes(a, 0) == 0
    bad = list(good); bad[1] = P(5, 0, FAKE, FAKE, 100, 256, X1, 256, Y1, 100)
    assert L.qgemm16_batch(arr(*bad), 2, ws, wsb, None) == EINVAL      # type id
    bad[1] = P(8, 0, FAKE, FAKE, 100, 250, X1, 256, Y1, 100)
    assert L.qgemm16_batch(arr(*bad), 2, ws, wsb, None) == ESHAPE      # cols % 32
    bad[1] = P(8, 0, FAKE, FAKE, 100, 256, X1 + 4, 256, Y1, 100)
    assert L.qgemm16_batch(arr(*bad), 2, ws, wsb, None) == EALIGN      # X not 16-byte aligned
    bad[1] = P(8, 0, FAKE, FAKE, 100, 256, X1, 256, X0 + 64, 100)
    assert L.qgemm16_batch(arr(*bad), 2, ws, wsb, None) == EINVAL      # Y_1 overlaps X_0
    bad[1] = P(8, 0, FAKE, FAKE, 100, 256, X1, 256, Y0 + 400, 100)
    assert L.qgemm16_batch(arr(*bad), 2, ws, wsb, None) == EINVAL      # Y_1 overlaps Y_0
    bad[1] = P(8, 0, FAKE, FAKE, 100, 256, X1, 256, X1 + 64, 100)
    assert L.qgemm16_batch(arr(*bad), 2, ws, wsb, None) == EINVAL      # Y_1 overlaps its own X
    assert L.qgemm16_batch(a, 2, ws, wsb - 1, None) == EWS
    assert L.qgemm16_batch(a, 2, None, wsb, None) == EWS
    assert L.qgemm16_batch(a, 2, ws + 16, wsb, None) == EALIGN


def test_gemm16_batch_splits():
    """The grouped launch's K splits (device without a GPU: 256 CUs): the
    prefill pass's segments as long as its shortest K; a lone problem split
    until it has two units per CU; short K never split."""
    P = qg.qg_gemm16_problem
    Xs = [FAKE + (k << 26) for k in range(1, 5)]
    Ys = [FAKE + (k << 26) for k in range(5, 9)]

    def splits(shapes):
        a = (P * len(shapes))()
        for i, (qt, r, c) in enumerate(shapes):
            a[i] = P(qt, 0, FAKE, FAKE, r, c, Xs[i], c, Ys[i], r)
        out = (ctypes.c_int32 * len(shapes))()
        assert L.qg_gemm16_batch_splits(a, len(shapes), out) == 0
        return list(out)

    assert splits([(2, 17408, 5120), (2, 5120, 17408), (8, 17408, 5120), (8, 5120, 17408)]) == [1, 3, 1, 3]
    assert splits([(2, 17408, 5120)]) == [4]          # 136 row groups x 4 >= 512 units
    assert splits([(8, 5120, 17408)]) == [13]         # 40 row groups x 13
    assert splits([(2, 64, 128), (8, 100, 256)]) == [1, 1]
    a = (P * 1)(P(2, 0, FAKE, FAKE, 64, 128, Xs[0], 128, Ys[0], 64))
    assert L.qg_gemm16_batch_splits(a, 1, None) == EINVAL
    assert L.qg_gemm16_batch_splits(a, 0, (ctypes.c_int32 * 1)()) == ESHAPE


def test_lmhead_noalloc_checks():
    x, oi = FAKE + (1 << 20), FAKE + (2 << 20)
    f = L.lmhead_argmax_noalloc
    assert f(5, FAKE, FAKE, 64, 128, 64, x, oi, None, None) == EINVAL
    assert f(2, FAKE, FAKE, 64, 100, 64, x, oi, None, None) == ESHAPE
    assert f(2, FAKE, FAKE, 64, 128, 65, x, oi, None, None) == ESHAPE
    assert f(2, FAKE, FAKE, 64, 128, 64, x + 4, oi, None, None) == EALIGN
    assert f(2, FAKE, FAKE, 64, 128, 64, x, None, None, None) == EINVAL
    # a head whose launch needs more than the 2 MiB scratch is refused before
    # anything runs (50,000,000 rows: 12.5 MB of row-group candidates)
    assert f(2, FAKE, FAKE, 50_000_000, 128, 50_000_000, x, oi, None, None) == EUNSUP


def test_gemm16_and_gateup_checks():
    ws = FAKE + (3 << 20)
    X, Y = FAKE + (1 << 20), FAKE + (2 << 20)
    assert L.qgemm16(5, FAKE, FAKE, 64, 128, X, 128, Y, 64, 0, ws, 1 << 24, None) == EINVAL
    assert L.qgemm16(2, FAKE, FAKE, 64, 100, X, 128, Y, 64, 0, ws, 1 << 24, None) == ESHAPE
    assert L.qgemm16(2, FAKE, FAKE, 64, 128, X, 128, Y, 64, 0, ws, 8, None) == EWS
    assert L.gateup_silu(2, FAKE, FAKE, None, FAKE, 64, 128, X, 128, 1, Y, 64, ws, 1 << 20, None) == EINVAL
    assert L.gateup_silu(2, FAKE, FAKE, FAKE, FAKE, 64, 128, X, 128, 9, Y, 64, ws, 1 << 20, None) == ESHAPE
    assert L.gateup_silu(2, FAKE, FAKE, FAKE, FAKE, 64, 128, X, 128, 1, X, 64, ws, 1 << 20, None) == EINVAL


def test_lmhead_checks():
    ws = FAKE + (3 << 20)
    x, o = FAKE + (1 << 20), FAKE + (2 << 20)
    assert L.lmhead_argmax(2, FAKE, FAKE, 64, 128, 0, x, o, None, ws, 1 << 20, None) == ESHAPE
    assert L.lmhead_argmax(2, FAKE, FAKE, 64, 128, 65, x, o, None, ws, 1 << 20, None) == ESHAPE
    assert L.lmhead_argmax(2, FAKE, FAKE, 64, 128, 64, x, None, None, ws, 1 << 20, None) == EINVAL
    assert L.lmhead_argmax(2, FAKE, FAKE, 64, 128, 64, x, o + 2, None, ws, 1 << 20, None) == EALIGN
    assert L.lmhead_argmax(2, FAKE, FAKE, 64, 128, 64, x, o, None, ws, 4, None) == EWS


def test_lmhead_topk_checks():
    assert L.qg_lmhead_topk_ws_bytes(248320, 5120, 10) > 0
    assert L.qg_lmhead_topk_ws_bytes(248320, 5120, 16) > L.qg_lmhead_topk_ws_bytes(248320, 5120, 10)
    assert L.qg_lmhead_topk_ws_bytes(248320, 5120, 0) == 0
    assert L.qg_lmhead_topk_ws_bytes(248320, 5120, 17) == 0
    ws = FAKE + (3 << 20)
    x, o = FAKE + (1 << 20), FAKE + (2 << 20)
    big = 1 << 20
    assert L.lmhead_topk(2, FAKE, FAKE, 64, 128, 64, x, 0, o, None, ws, big, None) == ESHAPE
    assert L.lmhead_topk(2, FAKE, FAKE, 64, 128, 64, x, 17, o, None, ws, big, None) == ESHAPE
    assert L.lmhead_topk(2, FAKE, FAKE, 64, 128, 8, x, 9, o, None, ws, big, None) == ESHAPE
    assert L.lmhead_topk(2, FAKE, FAKE, 64, 128, 65, x, 4, o, None, ws, big, None) == ESHAPE
    assert L.lmhead_topk(2, FAKE, FAKE, 64, 128, 64, x, 4, None, None, ws, big, None) == EINVAL
    assert L.lmhead_topk(2, FAKE, FAKE, 64, 128, 64, x, 4, o + 2, None, ws, big, None) == EALIGN
    assert L.lmhead_topk(2, FAKE, FAKE, 64, 128, 64, x, 4, o, o + 6, ws, big, None) == EALIGN
    assert L.lmhead_topk(2, FAKE, FAKE, 64, 128, 64, x, 4, o, None, ws, 4, None) == EWS
    assert L.lmhead_topk(5, FAKE, FAKE, 64, 128, 64, x, 4, o, None, ws, big, None) == EINVAL


def test_requant_checks():
    src, dst = FAKE, FAKE + (1 << 30)
    rq = L.qg_requant_q8_0
    assert rq(2, 10, src, dst, None) == EINVAL          # Q4_0 is not a source type
    assert rq(8, 10, src, dst, None) == EINVAL
    assert rq(3, 0, src, dst, None) == ESHAPE
    assert rq(3, 10, None, dst, None) == EINVAL
    assert rq(6, 10, src + 1, dst, None) == EALIGN
    assert rq(7, 10, src, dst + 1, None) == EALIGN
    assert rq(3, 10, src, src + 100, None) == EINVAL   # 200 source bytes overlap the output
    assert rq(15, 10, src, dst, None) == EINVAL         # Q8_K is not a source type
    assert rq(12, (1 << 33) + 1, src, dst, None) == ESHAPE   # more than 2^36 output blocks
    assert rq(3, (1 << 36) + 1, src, dst, None) == ESHAPE
    assert rq(14, 10, src + 1, dst, None) == EALIGN
    assert rq(13, 10, src, src + 1000, None) == EINVAL  # 1760 source bytes overlap the output
    assert rq(12, 10, src, src - 2000, None) == EINVAL  # 2720 output bytes overlap the source


def test_rmsnorm_checks():
    X, Y, G = FAKE, FAKE + (1 << 20), FAKE + (2 << 20)
    ws = FAKE + (3 << 20)
    big = 1 << 22
    gu = lambda gamma, eps, qt=2: L.gateup_silu_rmsnorm(qt, FAKE, FAKE, FAKE, FAKE, 64, 128, X, 128, 1, gamma, eps,
                                                       Y, 64, ws, big, None)
    assert gu(None, 1e-6) == EINVAL
    assert gu(G + 4, 1e-6) == EALIGN
    assert gu(G, -1.0) == EINVAL
    assert gu(G, float("nan")) == EINVAL
    assert gu(G, float("inf")) == EINVAL
    assert gu(G, 1e-6, qt=5) == EINVAL
    assert L.gateup_silu_rmsnorm(2, FAKE, FAKE, FAKE, FAKE, 64, 128, X, 128, 9, G, 1e-6, Y, 64, ws, big,
                                 None) == ESHAPE
    assert L.gateup_silu_rmsnorm(2, FAKE, FAKE, FAKE, FAKE, 64, 128, X, 128, 1, G, 1e-6, Y, 64, ws, 8,
                                 None) == EWS
    rn = L.qg_rmsnorm
    assert rn(None, 128, 128, 1, G, 1e-6, Y, 128, None) == EINVAL
    assert rn(X, 128, 128, 1, None, 1e-6, Y, 128, None) == EINVAL
    assert rn(X, 128, 0, 1, G, 1e-6, Y, 128, None) == ESHAPE
    assert rn(X, 100, 128, 1, G, 1e-6, Y, 128, None) == ESHAPE
    assert rn(X, 128, 128, 0, G, 1e-6, Y, 128, None) == ESHAPE
    assert rn(X + 2, 128, 128, 1, G, 1e-6, Y, 128, None) == EALIGN
    assert rn(X, 128, 128, 1, G, -1e-6, Y, 128, None) == EINVAL
    assert rn(X, 128, 128, 2, G, 1e-6, X + 64, 128, None) == EINVAL      # shifted overlap
    assert rn(X, 128, 128, 2, G, 1e-6, X, 256, None) == EINVAL           # in place with another ld


def test_repack_checks():
    src, qs, d = FAKE, FAKE + (1 << 30), FAKE + (2 << 30)
    assert L.qg_repack(2, 1, 16, 128, None, qs, d, None) == EINVAL
    assert L.qg_repack(2, 1, 16, 128, src + 1, qs, d, None) == EALIGN
    assert L.qg_repack(2, 1, 16, 128, src, qs + 4, d, None) == EALIGN
    assert L.qg_repack(2, 1, 16, 100, src, qs, d, None) == ESHAPE
    assert L.qg_repack(2, 1, 16, 128, src, src + 64, d, None) == EINVAL   # overlaps input


def _moe(**kw):
    m = qg.qg_moe()
    m.hidden, m.ffn, m.n_expert, m.top_k, m.normalize_topk, m.qtype = 256, 128, 16, 4, 1, 2
    m.router = FAKE
    for f in ("gate_qs", "up_qs", "down_qs", "gate_d", "up_d", "down_d"):
        setattr(m, f, FAKE + (1 << 24))
    m.sh_ffn = 0
    for k, v in kw.items():
        setattr(m, k, v)
    return m


def test_moe_checks():
    X, Y, ws = FAKE + (1 << 28), FAKE + (2 << 28), FAKE + (3 << 28)

    def call(m, ntok=1, wsb=1 << 26):
        return L.moe_ffn(ctypes.byref(m), X, 256, ntok, Y, 256, None, None, ws, wsb, None)

    assert L.qg_moe_ws_bytes(ctypes.byref(_moe()), 16) > 0
    assert call(_moe(), ntok=0) == ESHAPE
    assert call(_moe(), ntok=17) == ESHAPE
    assert call(_moe(top_k=9)) == ESHAPE
    assert call(_moe(top_k=17, n_expert=16)) == ESHAPE
    assert call(_moe(n_expert=4, top_k=5)) == ESHAPE
    assert call(_moe(hidden=200)) == ESHAPE
    assert call(_moe(ffn=96)) == ESHAPE
    assert call(_moe(qtype=3)) == EINVAL
    assert call(_moe(router=None)) == EINVAL
    assert call(_moe(router=FAKE + 4)) == EALIGN
    assert call(_moe(sh_ffn=128)) == EINVAL          # shared expert pointers missing
    assert call(_moe(), wsb=8) == EWS
    # the RMSNorm ahead of router and experts
    G = FAKE + (5 << 28)
    assert call(_moe(norm_weight=G + 4, norm_eps=1e-6)) == EALIGN
    assert call(_moe(norm_weight=G, norm_eps=-1.0)) == EINVAL
    assert call(_moe(norm_weight=G, norm_eps=float("nan"))) == EINVAL
    X2 = FAKE + (6 << 28)
    wide = _moe(norm_weight=G, norm_eps=1e-6, hidden=8192)
    assert L.moe_ffn(ctypes.byref(wide), X2, 8192, 1, X2 + (1 << 20), 8192, None, None, ws, 1 << 26,
                     None) == EUNSUP


def test_read_probe_checks():
    sink = ctypes.c_void_p(256)
    assert L.qg_read_probe(None, 1024, sink, None) == EINVAL
    assert L.qg_read_probe(ctypes.c_void_p(4096), 1024, None, None) == EINVAL
    assert L.qg_read_probe(ctypes.c_void_p(4096), 0, sink, None) == ESHAPE
    assert L.qg_read_probe(ctypes.c_void_p(4096), 1000, sink, None) == ESHAPE
    assert L.qg_read_probe(ctypes.c_void_p(4104), 1024, sink, None) == EALIGN


def test_plan_table():
    """Plan entries: valid ops, shapes and plans only; set, get, reset."""
    get = lambda *a: qg.plan_get(*a)
    L.qg_plan_reset()
    assert get(qg.OP_GEMV, 2, 64, 128, 1) == 0
    for op, nc, plan in [(qg.OP_GEMV, 1, 4), (qg.OP_GEMV, 8, qg.PLAN_SW), (qg.OP_GEMV, 16, 12),
                         (qg.OP_GATEUP, 3, 16), (qg.OP_LMHEAD, 1, 8 | qg.PLAN_STRICT),
                         (qg.OP_GEMV, 2, qg.PLAN_SPLIT(3)), (qg.OP_GEMV, 16, qg.PLAN_SPLIT(5) | 8),
                         (qg.OP_GATEUP, 1, qg.PLAN_SPLIT(255) | qg.PLAN_SW | qg.PLAN_STRICT)]:
        assert L.qg_plan_set(op, 2, 64, 128, nc, plan) == OK
        assert get(op, 2, 64, 128, nc) == plan
    assert get(qg.OP_GEMV, 8, 64, 128, 1) == 0           # other qtype: no entry
    bad = [(3, 2, 64, 128, 1, 0),                          # op
           (qg.OP_GEMV, 3, 64, 128, 1, 0),                 # qtype
           (qg.OP_GEMV, 2, 64, 100, 1, 0),                 # cols % 32
           (qg.OP_GEMV, 2, 0, 128, 1, 0),                  # rows
           (qg.OP_GEMV, 2, 64, 128, 9, 0),                 # ncols
           (qg.OP_GATEUP, 2, 64, 128, 16, 0),
           (qg.OP_LMHEAD, 2, 64, 128, 2, 0),
           (qg.OP_GEMV, 2, 64, 128, 1, 17),                # plans
           (qg.OP_GEMV, 2, 64, 128, 1, -1),
           (qg.OP_GEMV, 2, 64, 128, 1, 0x400),
           (qg.OP_GEMV, 2, 64, 128, 1, qg.PLAN_SW | 4),
           (qg.OP_GEMV, 2, 64, 128, 1, qg.PLAN_STRICT),
           (qg.OP_GEMV, 2, 64, 128, 16, 4),                # 16 columns: 8..16 waves
           (qg.OP_GEMV, 2, 64, 128, 16, qg.PLAN_SW),
           (qg.OP_GEMV, 2, 64, 128, 16, qg.PLAN_SPLIT(2) | 4),
           (qg.OP_GEMV, 2, 64, 128, 1, qg.PLAN_SPLIT(256)),  # 1..255 segments
           (qg.OP_GEMV, 2, 64, 128, 1, qg.PLAN_SPLIT(3) | 17)]
    for a in bad:
        assert L.qg_plan_set(*a) == EINVAL, a
    assert L.qg_plan_get(qg.OP_GEMV, 2, 64, 128, 1, None) == EINVAL
    L.qg_plan_reset()
    assert get(qg.OP_GEMV, 2, 64, 128, 1) == 0
    assert get(qg.OP_GATEUP, 2, 64, 128, 3) == 0


def test_tune_argument_checks():
    """The tuning calls check their arguments as the calls they tune (before
    any HIP call)."""
    ws, X, Y = FAKE + (3 << 20), FAKE + (1 << 20), FAKE + (2 << 20)
    tg = lambda **k: L.qg_tune_gemv(k.get("qt", 2), k.get("qs", FAKE), FAKE, 64, 128, X, 128, k.get("nc", 1),
                                    k.get("Y", Y), 64, ws, 1 << 20, None, 0, None)
    assert tg(qs=None) == EINVAL
    assert tg(qt=3) == EINVAL
    assert tg(nc=9) == ESHAPE
    assert tg(Y=X + 64) == EINVAL
    assert L.qg_tune_gateup(2, FAKE, FAKE, None, FAKE, 64, 128, X, 128, 1, Y, 64, ws, 1 << 20, None,
                            0, None) == EINVAL
    assert L.qg_tune_gateup(2, FAKE, FAKE, FAKE, FAKE, 64, 128, X, 128, 1, Y, 64, ws, 16, None,
                            1, None) == EWS
    assert L.qg_tune_lmhead(2, FAKE, FAKE, 64, 128, 65, X, Y, None, ws, 1 << 20, None, 0, None) == ESHAPE
    assert L.qg_tune_lmhead(2, FAKE, FAKE, 64, 128, 64, X, None, None, ws, 1 << 20, None, 1, None) == EINVAL

