"""Bench: achieved HBM GB/s of the block-quantised products on one MI355X.

`value` is the prefill step of the 16-column workload: a 512-token prompt
run as 32 passes of 16 columns, each pass one launch over the four matrices
of the workload (Q4_0 and Q8_0, 5120 -> 17408 and 17408 -> 5120, every
weight block read once per pass for its 16 columns), then the LM head
(Q8_0, 248,320 x 5120) with the GPU argmax.  Algorithmic bytes per step x
steps / time.  The other workloads (the decode FFN step, the decode GEMV
2048 x 2048, verify GEMVs at 4 and 8 columns, single 16-column GEMMs, LM
head top-k, the MoE FFN at 1 and 16 tokens, requantisation) are timed the
same way and reported under "kernels".

Inputs are seeded synthetic tensors at the pages' model shapes, resident in
HBM before timing.  Every timed loop cycles byte-identical, address-distinct
weight copies of >= 1 GiB in all (larger than the 256 MB Infinity Cache), is
captured in a HIP graph (no host launch gaps) and is timed with events on
the stream the kernels run on.

Algorithmic bytes: packed weights (qs + f16 scales) + activations read +
outputs written (+ outputs read when accumulating) + router weights.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
POOL_BYTES = 1 << 30


def qbytes(qtype, rows, cols):
    return rows * cols // 32 * (18 if qtype == 2 else 34)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Bench:
    def __init__(self, torch, qg, dev):
        self.torch, self.qg, self.dev = torch, qg, dev

    def up(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    def matrix(self, qtype, rows, cols, seed, sigma):
        raw = __import__("synth").gen_weights(qtype, rows, cols, sigma, np.random.default_rng(seed))
        return self.qg.qg_repack(qtype, self.up(raw.reshape(-1)), rows, cols), raw

    def pool(self, w, per_copy_bytes):
        """Byte-identical, address-distinct copies totalling >= 1 GiB."""
        n = max(2, -(-POOL_BYTES // per_copy_bytes))
        out = [w]
        for _ in range(n - 1):
            out.append(self.qg.QMatrix(w.qtype, w.rows, w.cols, w.n_mat, w.qs.clone(), w.d.clone()))
        return out

    def graph_time(self, fns, iters, reps=5):
        """Capture `iters` calls (cycling fns) in one HIP graph and replay it
        `reps` times after one warm replay.  Returns the mean time per call in
        seconds over all timed replays and the graph; `self.last` holds the
        per-call time of each replay (for median and min)."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for f in fns[:2]:
                f()                               # eager warm-up on the capture stream (workspace, code objects)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for i in range(iters):
                    fns[i % len(fns)]()
        torch.cuda.current_stream().wait_stream(s)
        g.replay()                                # warm replay
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for r in range(reps):
            g.replay()
            ev[r + 1].record()
        torch.cuda.synchronize()
        self.last = [ev[r].elapsed_time(ev[r + 1]) * 1e-3 / iters for r in range(reps)]
        return ev[0].elapsed_time(ev[reps]) * 1e-3 / (iters * reps), g


def kernel_entry(bytes_per_call, t, extra=None, per_rep=None):
    """One workload: mean time per call, bytes per call, GB/s and fraction of
    the 8 TB/s peak; with per-replay times, their median and minimum."""
    gbs = bytes_per_call / t / 1e9
    d = {"us": round(t * 1e6, 3), "bytes": int(bytes_per_call), "GB_s": round(gbs, 1),
         "frac_peak": round(gbs / PEAK_HBM_GBS, 4)}
    if per_rep:
        d["us_median"] = round(float(np.median(per_rep)) * 1e6, 3)
        d["us_min"] = round(min(per_rep) * 1e6, 3)
    if extra:
        d.update(extra)
    return d


# The prefill workload: four matrices, 16 columns per pass, 32 passes.
PREFILL = ((2, 17408, 5120), (2, 5120, 17408), (8, 17408, 5120), (8, 5120, 17408))
PASSES = 32
LM_ROWS, LM_COLS = 248320, 5120


def pass_bytes():
    return sum(qbytes(qt, N, K) + 64 * (N + K) for qt, N, K in PREFILL)


def step_bytes():
    return PASSES * pass_bytes() + qbytes(8, LM_ROWS, LM_COLS) + 4 * LM_COLS + 8


def run_prefill(B, steps, warmup):
    """The headline step.  Returns (per-step times over `steps` timed steps,
    per-launch time of the pass kernel with its per-replay times, the host
    copies of the matrices for the CPU baseline)."""
    torch, qg = B.torch, B.qg
    import synth
    # four address-distinct sets of the four matrices (4 x 289 MB >= 1 GiB);
    # pass p reads set p % 4
    base, raws = [], []
    for i, (qt, N, K) in enumerate(PREFILL):
        w, raw = B.matrix(qt, N, K, seed=41 + i, sigma=0.005 if qt == 8 else 0.02)
        base.append(w)
        raws.append(raw)
    cl = lambda m: qg.QMatrix(m.qtype, m.rows, m.cols, m.n_mat, m.qs.clone(), m.d.clone())
    sets = [base] + [[cl(m) for m in base] for _ in range(3)]
    # each pass its own 16 columns (the next 16 tokens): one X per input width
    xs = [{K: B.up(synth.gen_x(K, 16, cfg_id=synth.CFG_PREFILL, col0=16 * (2 * p + (K > 5120))).T)
           for K in (5120, 17408)} for p in range(PASSES)]
    ys = [torch.empty((16, N), device=B.dev) for (_, N, _) in PREFILL]
    # the LM head: two copies (1.35 GB each), alternating step by step
    lm, _ = B.matrix(8, LM_ROWS, LM_COLS, seed=51, sigma=0.005)
    lms = [lm, cl(lm)]
    xl = B.up(synth.gen_x(LM_COLS, 1, cfg_id=synth.CFG_PREFILL)[:, 0])
    oi = torch.empty(1, dtype=torch.int32, device=B.dev)
    ov = torch.empty(1, dtype=torch.float32, device=B.dev)

    def one_pass(p):
        st = sets[p % 4]
        qg.qgemm16_batch([(st[j], xs[p][PREFILL[j][2]], ys[j], 0) for j in range(4)])

    def step(c):
        for p in range(PASSES):
            one_pass(p)
        qg.lmhead_argmax(lms[c], xl, None, oi, ov)

    # one graph per LM-head copy, replayed alternately; each timed step is
    # bracketed by events on the launch stream (median and min over steps)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(s):
        step(0)                                   # eager warm-up on the capture stream
        step(1)
        torch.cuda.synchronize()
        for c in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step(c)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    for w in range(warmup):
        graphs[w % 2].replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for k in range(steps):
        graphs[k % 2].replay()
        ev[k + 1].record()
    torch.cuda.synchronize()
    per_step = [ev[k].elapsed_time(ev[k + 1]) * 1e-3 for k in range(steps)]
    total = ev[0].elapsed_time(ev[steps]) * 1e-3
    del graphs
    # the pass kernel alone: 4 x 32 launches (set and inputs cycling), 5 replays
    t_pass, _ = B.graph_time([lambda p=p: one_pass(p) for p in range(PASSES)], 4 * PASSES)
    pass_reps = list(B.last)
    # the same pass as four single-matrix launches, for comparison
    def four(p):
        st = sets[p % 4]
        for j in range(4):
            qg.qgemm16(st[j], xs[p][PREFILL[j][2]], ys[j])
    t_four, _ = B.graph_time([lambda p=p: four(p) for p in range(PASSES)], 4 * PASSES)
    four_reps = list(B.last)
    # each matrix alone (single 16-column GEMM launches over its 4 copies)
    singles = {}
    for j, (qt, N, K) in enumerate(PREFILL):
        t1, _ = B.graph_time([lambda p=p: qg.qgemm16(sets[p % 4][j], xs[p][K], ys[j]) for p in range(PASSES)],
                             4 * PASSES)
        singles[f"gemm16_{'q4_0' if qt == 2 else 'q8_0'}_{K}to{N}"] = kernel_entry(
            qbytes(qt, N, K) + 64 * (N + K), t1, {"tokens_per_s": round(16 / t1, 1)}, list(B.last))
    t_lm, _ = B.graph_time([lambda c=c: qg.lmhead_argmax(lms[c], xl, None, oi, ov) for c in range(2)], 20)
    lm_reps = list(B.last)
    del sets, lms
    return {"per_step": per_step, "total": total, "t_pass": t_pass, "pass_reps": pass_reps,
            "t_four": t_four, "four_reps": four_reps, "singles": singles, "t_lm": t_lm, "lm_reps": lm_reps,
            "raws": raws}


def run_ffn(B, kernels):
    """The decode-FFN step of a 27B-like layer at batch 1 (gate/up with SiLU,
    then down accumulated into the residual), its two launches, and the
    RMSNorm folded into gate/up against its own launch first."""
    torch, qg = B.torch, B.qg
    Q4 = qg.Q4_0
    N, K = 17408, 5120
    wg, _ = B.matrix(Q4, N, K, seed=21, sigma=0.02)
    wu, _ = B.matrix(Q4, N, K, seed=22, sigma=0.02)
    wd, _ = B.matrix(Q4, K, N, seed=23, sigma=0.02)
    set_bytes = 3 * qbytes(Q4, N, K)
    n = max(2, -(-POOL_BYTES // set_bytes))
    pg, pu, pd = B.pool(wg, set_bytes)[:n], B.pool(wu, set_bytes)[:n], B.pool(wd, set_bytes)[:n]
    import synth
    x = B.up(synth.gen_x(K, 1, cfg_id=2).T)
    y = B.up(synth.rng(2, 90).standard_normal((1, K)).astype(np.float32))
    h = torch.empty((1, N), dtype=torch.float32, device=B.dev)
    gu_bytes = 2 * qbytes(Q4, N, K) + 4 * K + 4 * N
    dn_bytes = qbytes(Q4, K, N) + 4 * N + 8 * K

    def step(i):
        qg.gateup_silu(pg[i], pu[i], x, h)
        qg.qgemv(pd[i], h, y, accumulate=True)

    t, _ = B.graph_time([lambda i=i: step(i) for i in range(n)], 4 * n)
    kernels["decode_ffn_step_q4_0_5120x17408"] = kernel_entry(gu_bytes + dn_bytes, t,
                                                               {"tokens_per_s": round(1 / t, 1)}, B.last)
    t, _ = B.graph_time([lambda i=i: qg.gateup_silu(pg[i], pu[i], x, h) for i in range(n)], 4 * n)
    kernels["gateup_silu_q4_0_5120to2x17408"] = kernel_entry(gu_bytes, t, None, B.last)
    t, _ = B.graph_time([lambda i=i: qg.qgemv(pd[i], h, y, accumulate=True) for i in range(n)], 4 * n)
    kernels["qgemv_q4_0_17408to5120_acc"] = kernel_entry(dn_bytes, t, None, B.last)
    # RMSNorm ahead of gate/up: folded into the call, and as its own launch
    # first (the same algorithmic bytes: weights, x, gamma, h)
    gam = B.up(synth.rng(3, K).uniform(0.5, 1.5, K).astype(np.float32))
    xn = torch.empty_like(x)
    t, _ = B.graph_time([lambda i=i: qg.gateup_silu_rmsnorm(pg[i], pu[i], x, gam, 1e-6, h) for i in range(n)],
                        4 * n)
    kernels["gateup_rmsnorm_fused_q4_0_5120to2x17408"] = kernel_entry(gu_bytes + 4 * K, t, None, B.last)

    def norm_then_gu(i):
        qg.rmsnorm(x, gam, 1e-6, xn)
        qg.gateup_silu(pg[i], pu[i], xn, h)

    t, _ = B.graph_time([lambda i=i: norm_then_gu(i) for i in range(n)], 4 * n)
    kernels["rmsnorm_then_gateup_q4_0_5120to2x17408"] = kernel_entry(gu_bytes + 4 * K, t, None, B.last)
    del pg, pu, pd


def run_extras(B, kernels):
    torch, qg = B.torch, B.qg
    import synth
    Q4, Q8 = qg.Q4_0, qg.Q8_0

    # decode GEMV, 2048 x 2048 Q4_0 (a parity-size matrix; launch-bound)
    w, _ = B.matrix(Q4, 2048, 2048, seed=11, sigma=0.02)
    p = B.pool(w, qbytes(Q4, 2048, 2048))
    x = B.up(synth.gen_x(2048, 1, cfg_id=1).T)
    y = torch.empty((1, 2048), device=B.dev)
    t, _ = B.graph_time([lambda m=m: qg.qgemv(m, x, y) for m in p], 2 * len(p))
    kernels["gemv_q4_0_2048x2048_1col"] = kernel_entry(qbytes(Q4, 2048, 2048) + 8192 * 2, t, None, B.last)
    del p
    log("  gemv 2048 done")

    # verify GEMVs at 4 and 8 columns
    for qtype, N, K, name in ((Q8, 5120, 5120, "q8_0_5120x5120"), (Q4, 17408, 5120, "q4_0_5120to17408")):
        w, _ = B.matrix(qtype, N, K, seed=31, sigma=0.005 if qtype == Q8 else 0.02)
        p = B.pool(w, qbytes(qtype, N, K))
        for nc in (4, 8):
            x = B.up(synth.gen_x(K, nc, cfg_id=3).T)
            y = torch.empty((nc, N), device=B.dev)
            t, _ = B.graph_time([lambda m=m: qg.qgemv(m, x, y) for m in p], 2 * len(p))
            kernels[f"verify_{name}_{nc}col"] = kernel_entry(qbytes(qtype, N, K) + 4 * nc * (N + K), t,
                                                             {"tokens_per_s": round(nc / t, 1)}, B.last)
        del p
    log("  verify done")

    # LM head + top-10 (the Three.js page's example asks for top-k 10):
    # Q8_0 248,320 x 5120, two address-distinct copies
    N, K = 248320, 5120
    w, _ = B.matrix(Q8, N, K, seed=51, sigma=0.005)
    p = [w, qg.QMatrix(w.qtype, w.rows, w.cols, 1, w.qs.clone(), w.d.clone())]
    x = B.up(synth.gen_x(K, 1, cfg_id=4)[:, 0])
    # the same head returning the 10 best (value, row) pairs (the Three.js
    # page's example asks for top-k 10)
    ti = torch.empty(10, dtype=torch.int32, device=B.dev)
    tv = torch.empty(10, dtype=torch.float32, device=B.dev)
    t, _ = B.graph_time([lambda m=m: qg.lmhead_topk(m, x, 10, None, ti, tv) for m in p], 20)
    kernels["lmhead_topk10_q8_0_5120to248320"] = kernel_entry(qbytes(Q8, N, K) + 4 * K + 80, t, None, B.last)
    del p, w
    log("  lmhead done")

    # load-time requantisation of a Q4_1 17408 x 5120 matrix to Q8_0 (bytes
    # read + written), over 8 address-distinct source / destination pairs
    # (8 x 151 MB >= 1 GiB)
    nbk = 17408 * 5120 // 32
    src0 = torch.randint(0, 256, (nbk * 20,), dtype=torch.uint8, device=B.dev)
    src0.view(nbk, 20)[:, 1] = 0x3C        # finite scales near 1 (f16 high byte)
    src0.view(nbk, 20)[:, 3] = 0xBC        # offsets near -1
    pairs = [(src0 if i == 0 else src0.clone(), torch.empty(nbk * 34, dtype=torch.uint8, device=B.dev))
             for i in range(8)]
    t, _ = B.graph_time([lambda sd=sd: qg.requant_q8_0(qg.Q4_1, sd[0], nbk, sd[1]) for sd in pairs], 32)
    kernels["requant_q4_1_to_q8_0_17408x5120"] = kernel_entry(nbk * (20 + 34), t, None, B.last)
    del src0, pairs
    # the same matrix as Q4_K and Q6_K super-blocks (256 values each), random
    # bytes with finite f16 scales near 1 (and mins near 1 for Q4_K)
    for st, name, bs, doff in ((qg.Q4_K, "q4_k", 144, 0), (qg.Q6_K, "q6_k", 210, 208)):
        nsb = 17408 * 5120 // 256
        src0 = torch.randint(0, 256, (nsb * bs,), dtype=torch.uint8, device=B.dev)
        src0.view(nsb, bs)[:, doff + 1] = 0x3C
        if st == qg.Q4_K:
            src0.view(nsb, bs)[:, 3] = 0x3C
        pairs = [(src0 if i == 0 else src0.clone(), torch.empty(nsb * 8 * 34, dtype=torch.uint8, device=B.dev))
                 for i in range(8)]
        t, _ = B.graph_time([lambda sd=sd: qg.requant_q8_0(st, sd[0], nsb, sd[1]) for sd in pairs], 32)
        kernels[f"requant_{name}_to_q8_0_17408x5120"] = kernel_entry(nsb * (bs + 8 * 34), t, None, B.last)
        del src0, pairs
    log("  requant done")

    # MoE FFN, 256 experts (8 active) + shared, hidden 2048, ffn 512
    moes, (E, H, F, k), copies = moe_layers(B)
    eb = qbytes(Q4, F, H) * 3
    NX = 17  # distinct inputs per token count, cycled against the layer copies
    for T in (1, 16):
        Xs = [B.up(synth.gen_x(H, T, cfg_id=5, col0=T * i).T) for i in range(NX)]
        Y = torch.zeros((T, H), device=B.dev)
        tidx = torch.empty((T, k), dtype=torch.int32, device=B.dev)
        # algorithmic bytes of each input's call: the experts its routing reads
        us = []
        for X in Xs:
            qg.moe_ffn(moes[0], X, Y, tidx)
            torch.cuda.synchronize()
            us.append(len(np.unique(tidx.cpu().numpy())))
        calls = NX * copies
        fn = [lambda i=i: qg.moe_ffn(moes[i % copies], Xs[i % NX], Y) for i in range(calls)]
        nbytes = 4 * E * H + eb * (float(np.mean(us)) + 1) + 4 * H * T + 8 * H * T
        t, _ = B.graph_time(fn, calls)
        kernels[f"moe_ffn_{T}tok"] = kernel_entry(nbytes, t, {"distinct_experts_mean": round(float(np.mean(us)), 2),
                                                             "tokens_per_s": round(T / t, 1),
                                                             "inputs": NX, "layer_copies": copies}, B.last)
        # the RMSNorm ahead of router and experts: folded into the layer, and
        # as its own launch first (the same algorithmic bytes plus the weights)
        gam = B.up(synth.rng(63, H).uniform(0.5, 1.5, H).astype(np.float32))
        for m in moes:
            m.norm_weight, m.norm_eps = gam, 1e-6
        t_nf, _ = B.graph_time(fn, calls)
        reps_nf = list(B.last)
        for m in moes:
            m.norm_weight = None
        Xn = torch.empty_like(Xs[0])

        def norm_then_moe(i):
            qg.rmsnorm(Xs[i % NX], gam, 1e-6, Xn)
            qg.moe_ffn(moes[i % copies], Xn, Y)

        t_nu, _ = B.graph_time([lambda i=i: norm_then_moe(i) for i in range(calls)], calls)
        kernels[f"moe_ffn_rmsnorm_fused_{T}tok"] = kernel_entry(nbytes + 4 * H, t_nf, None, reps_nf)
        kernels[f"rmsnorm_then_moe_ffn_{T}tok"] = kernel_entry(nbytes + 4 * H, t_nu, None, B.last)
    del moes
    log("  moe done")


def run_plans(B, kernels):
    """Each launch plan timed at the benchmarked decode shapes (the built-in
    choice, 4 / 8 / 12 / 16 waves per workgroup, K segments inside one
    workgroup, and K splits of 1 to 12 segments with the built-in layout),
    and the plans the tuner keeps there (without and with splits)."""
    torch, qg = B.torch, B.qg
    import synth
    Q4 = qg.Q4_0
    cands = [4, 8, 12, 16, qg.PLAN_SW]

    splits = [qg.PLAN_SPLIT(s) for s in (1, 2, 3, 4, 6, 8, 12)]

    def sweep(op, w, ncols, mk_fns, iters, plans):
        us = {}
        for pl in [0] + plans + splits:
            qg.plan_reset()
            if pl:
                qg.plan_set(op, w.qtype, w.rows, w.cols, ncols, pl | qg.PLAN_STRICT)
            key = ("builtin" if pl == 0 else "sw" if pl == qg.PLAN_SW else
                   f"split{pl >> 12}" if pl >= 1 << 12 else str(pl))
            try:
                t, _ = B.graph_time(mk_fns(), iters)   # a refused plan raises in the eager warm-up
                us[key] = round(t * 1e6, 2)
            except qg.QGError:
                us[key] = None
        qg.plan_reset()
        return us

    N, K = 17408, 5120
    for nm, rows, cols, ncols in (("gateup_silu_q4_0_5120to2x17408_1col", N, K, 1),
                                  ("down_q4_0_17408to5120_1col", K, N, 1),
                                  ("verify_q4_0_5120to17408_4col", N, K, 4),
                                  ("verify_q4_0_5120to17408_8col", N, K, 8),
                                  ("gemm16_q4_0_5120to17408", N, K, 16)):
        w, _ = B.matrix(Q4, rows, cols, seed=61, sigma=0.02)
        gate = nm.startswith("gateup")
        p = B.pool(w, qbytes(Q4, rows, cols))     # gate/up: distinct pairs (2i, 2i + 1)
        x = B.up(synth.gen_x(cols, ncols, cfg_id=6).T)
        y = torch.empty((ncols, rows), device=B.dev)
        if gate:
            fns = lambda: [lambda i=i: qg.gateup_silu(p[2 * i], p[2 * i + 1], x, y) for i in range(len(p) // 2)]
            us = sweep(qg.OP_GATEUP, w, ncols, fns, len(p), cands)
            tuned = qg.tune_gateup(p[0], p[1], x, y)
            qg.plan_reset()
            tuned_s = qg.tune_gateup(p[0], p[1], x, y, split=True)
        elif ncols == 16:
            fns = lambda: [lambda m=m: qg.qgemm16(m, x, y) for m in p]
            us = sweep(qg.OP_GEMV, w, ncols, fns, 2 * len(p), [8, 12, 16])
            tuned = qg.tune_gemv(p[0], x, y)
            qg.plan_reset()
            tuned_s = qg.tune_gemv(p[0], x, y, split=True)
        else:
            fns = lambda: [lambda m=m: qg.qgemv(m, x, y) for m in p]
            us = sweep(qg.OP_GEMV, w, ncols, fns, 2 * len(p), cands)
            tuned = qg.tune_gemv(p[0], x, y)
            qg.plan_reset()
            tuned_s = qg.tune_gemv(p[0], x, y, split=True)
        qg.plan_reset()
        kernels[f"plans_{nm}"] = {"us": us, "tuned_plan": tuned, "tuned_plan_with_splits": tuned_s}
        del p
    log("  plans done")


def ceilings(B):
    """Measured denominators beside the 8 TB/s spec, timed the same way:
    a plain device copy of 1 GiB (read + write), and the library's
    streaming-read probe over 1 GiB (reads every byte once, the way the
    product kernels stream weights).  A 100 MB read (the decode gate/up
    size, 10 address-distinct slices of the 1 GiB buffer) shows what launch
    and ramp leave at that size."""
    torch, qg = B.torch, B.qg
    a = torch.empty(POOL_BYTES // 4, dtype=torch.float32, device=B.dev).normal_()
    b = torch.empty_like(a)
    sink = torch.zeros(1, dtype=torch.int32, device=B.dev)
    t_copy, _ = B.graph_time([lambda: b.copy_(a)], 10)
    t_read, _ = B.graph_time([lambda: qg.read_probe(a, sink)], 10)
    n = 100_000_000 // 4
    slices = [a[i * n:(i + 1) * n] for i in range(POOL_BYTES // 4 // n)]
    t_small, _ = B.graph_time([lambda s=s: qg.read_probe(s, sink) for s in slices], 2 * len(slices))
    return (2 * POOL_BYTES / t_copy / 1e9, POOL_BYTES / t_read / 1e9, n * 4 / t_small / 1e9)


# the sources of the pass kernel whose counters the traffic summary holds
TRAFFIC_SOURCES = ("gemm_q4_q8_amd/csrc/qmv.hip", "gemm_q4_q8_amd/csrc/dot_unit.h",
                   "gemm_q4_q8_amd/csrc/common.h")
TRAFFIC_FILE = "gemm16_batch_prefill_pass_traffic.txt"


def source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per pass launch from the committed counter summary, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILE)
    try:
        fields = dict(l.split()[0:2] for l in open(path) if l.strip() and not l.startswith("#")
                      and len(l.split()) == 2)
    except OSError:
        return None
    if fields.get("kernel_source_hash") != source_hash():
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def cpu_baseline(raws, min_seconds=12.0):
    """The oracle, as it stands, on full prefill passes of the headline step
    (the four 16-column GEMMs over all their rows), repeated until at least
    `min_seconds` of host work."""
    import synth
    from oracle import ops
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = 1
    host_cores = len(os.sched_getaffinity(0))
    xs = {K: synth.gen_x(K, 16, cfg_id=synth.CFG_PREFILL, col0=16 * (K > 5120)) for K in (5120, 17408)}
    reps = 0
    t0 = time.perf_counter()
    while True:
        for raw, (qt, N, K) in zip(raws, PREFILL):
            ops.gemv(qt, raw, xs[K])
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    return {"value": round(pass_bytes() / dt / 1e9, 3), "unit": "GB/s", "cores": int(min(threads, host_cores)),
            "kind": "oracle",
            "sample": f"{reps} full prefill passes (Q4_0 and Q8_0, 5120->17408 and 17408->5120, 16 columns, all "
                      f"rows; the step is 32 such passes plus the LM head), {dt * reps:.1f} s, {dt:.2f} s per pass; "
                      f"f64 numpy: BLAS products on {threads} threads, dequantisation on one; "
                      f"host cores available: {host_cores}"}


def moe_layers(B, copies=None):
    """The benchmarked MoE layer (256 Q4_0 experts, 8 active, plus a shared
    expert; hidden 2048, expert FFN 512) in `copies` address-distinct copies
    of its experts (default: enough for >= 1 GiB of expert weights)."""
    import synth
    torch, qg = B.torch, B.qg
    Q4 = qg.Q4_0
    E, H, F, k = 256, 2048, 512, 8
    g = np.random.default_rng(61)

    def stack(rows, cols):
        raw = np.stack([synth.gen_weights(Q4, rows, cols, 0.02, g) for _ in range(E)])
        return qg.qg_repack(Q4, B.up(raw.reshape(-1)), rows, cols, E)
    gate, upm, down = stack(F, H), stack(F, H), stack(H, F)
    sh = [B.matrix(Q4, r, c, seed=62 + i, sigma=0.02)[0] for i, (r, c) in enumerate(((F, H), (F, H), (H, F)))]
    router = B.up(synth.gen_f32((E, H), 0.02, g))
    layer_bytes = 3 * E * qbytes(Q4, F, H)
    if copies is None:
        copies = max(2, -(-POOL_BYTES // layer_bytes))
    cl = lambda m: qg.QMatrix(m.qtype, m.rows, m.cols, m.n_mat, m.qs.clone(), m.d.clone())
    moes = []
    for c in range(copies):
        gg, uu, dd = (gate, upm, down) if c == 0 else (cl(gate), cl(upm), cl(down))
        moes.append(qg.MoE(hidden=H, ffn=F, n_expert=E, top_k=k, router=router, gate=gg, up=uu,
                           down=dd, sh_gate=sh[0], sh_up=sh[1], sh_down=sh[2]))
    return moes, (E, H, F, k), copies


def traffic_run(B):
    """Fixed launches for hardware-counter runs (rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE): 5 element-wise copies of exactly 1 GiB (read 1 GiB, write
    1 GiB) as the scale reference, then 8 prefill-pass launches over 4
    address-distinct weight sets, then 8 launches of each single 16-column
    GEMM, 4 of the LM head with argmax, 16 decode gate/up and 16 decode down
    launches, 16 verify launches (Q8_0 5120 x 5120) at 4 and at 8 columns,
    and 8 MoE layers at 16 tokens, over address-distinct weights."""
    torch, qg = B.torch, B.qg
    Q4, Q8 = qg.Q4_0, qg.Q8_0
    import synth
    a = torch.empty(POOL_BYTES // 4, dtype=torch.float32, device=B.dev).normal_()
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    del a, b
    sets = [[B.matrix(qt, N, K, seed=41 + 10 * s + i, sigma=0.005 if qt == 8 else 0.02)[0]
             for i, (qt, N, K) in enumerate(PREFILL)] for s in range(4)]
    xs = {K: B.up(synth.gen_x(K, 16, cfg_id=synth.CFG_PREFILL).T) for K in (5120, 17408)}
    ys = [torch.empty((16, N), device=B.dev) for (_, N, _) in PREFILL]
    torch.cuda.synchronize()
    for r in range(8):
        qg.qgemm16_batch([(sets[r % 4][j], xs[PREFILL[j][2]], ys[j], 0) for j in range(4)])
    torch.cuda.synchronize()
    for j in range(4):
        for r in range(8):
            qg.qgemm16(sets[r % 4][j], xs[PREFILL[j][2]], ys[j])
    torch.cuda.synchronize()
    del sets
    lm = [B.matrix(8, LM_ROWS, LM_COLS, seed=51 + i, sigma=0.005)[0] for i in range(2)]
    xl = B.up(synth.gen_x(LM_COLS, 1, cfg_id=synth.CFG_PREFILL)[:, 0])
    torch.cuda.synchronize()
    for r in range(4):
        qg.lmhead_argmax(lm[r % 2], xl)
    torch.cuda.synchronize()
    del lm
    N, K = 17408, 5120
    ws = [(B.matrix(2, N, K, seed=21 + i, sigma=0.02)[0], B.matrix(2, N, K, seed=61 + i, sigma=0.02)[0],
           B.matrix(2, K, N, seed=81 + i, sigma=0.02)[0]) for i in range(6)]
    x = B.up(synth.gen_x(K, 1, cfg_id=2).T)
    h = torch.empty((1, N), dtype=torch.float32, device=B.dev)
    y = torch.zeros((1, K), dtype=torch.float32, device=B.dev)
    torch.cuda.synchronize()
    for i in range(16):
        qg.gateup_silu(ws[i % 6][0], ws[i % 6][1], x, h)
    torch.cuda.synchronize()
    for i in range(16):
        qg.qgemv(ws[i % 6][2], h, y, accumulate=True)
    torch.cuda.synchronize()
    del ws
    # verify Q8_0 5120 x 5120 at 4 and 8 columns, 8 address-distinct copies
    w, _ = B.matrix(Q8, 5120, 5120, seed=31, sigma=0.005)
    vp = [w] + [qg.QMatrix(w.qtype, w.rows, w.cols, 1, w.qs.clone(), w.d.clone()) for _ in range(7)]
    for nc in (4, 8):
        xv = B.up(synth.gen_x(5120, nc, cfg_id=3).T)
        yv = torch.empty((nc, 5120), device=B.dev)
        torch.cuda.synchronize()
        for i in range(16):
            qg.qgemv(vp[i % 8], xv, yv)
        torch.cuda.synchronize()
    del vp, w
    # the MoE layer at 16 tokens: 8 calls, each on a fresh input and the next
    # of 4 copies of the experts; the algorithmic bytes of each call (router,
    # the experts its routing reads, the shared expert, activations in and
    # out) printed for the summary
    moes, (E, H, F, k), copies = moe_layers(B, 4)
    eb = qbytes(Q4, F, H) * 3
    T = 16
    Y = torch.zeros((T, H), device=B.dev)
    tidx = torch.empty((T, k), dtype=torch.int32, device=B.dev)
    nb = []
    for i in range(8):
        X = B.up(synth.gen_x(H, T, cfg_id=5, col0=T * i).T)
        torch.cuda.synchronize()
        qg.moe_ffn(moes[i % copies], X, Y, tidx)
        torch.cuda.synchronize()
        nb.append(4 * E * H + eb * (len(np.unique(tidx.cpu().numpy())) + 1) + 12 * H * T)
    print(f"moe_16tok_algorithmic_bytes_per_call {float(np.mean(nb)):.0f}", flush=True)
    print("traffic run done", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--suite", choices=["all", "main", "plans"], default="all",
                    help="main: the headline step only; all: every workload; plans: all plus the launch-plan sweep")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--traffic", action="store_true",
                    help="only the fixed launches used for HBM traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_q4_q8_amd as qg
    dev = torch.device("cuda:0")
    B = Bench(torch, qg, dev)
    if args.traffic:
        traffic_run(B)
        return

    log("bench: prefill step (32 passes of 16 columns + LM head)")
    r = run_prefill(B, args.steps, args.warmup)
    sb = step_bytes()
    t_step = r["total"] / args.steps
    value = sb / t_step / 1e9
    kernels = {
        "prefill_pass_batch_4x16col": kernel_entry(pass_bytes(), r["t_pass"], {"tokens_per_s": round(16 / r["t_pass"], 1)},
                                                   r["pass_reps"]),
        "prefill_pass_4_single_launches": kernel_entry(pass_bytes(), r["t_four"], None, r["four_reps"]),
        "lmhead_argmax_q8_0_5120to248320": kernel_entry(qbytes(8, LM_ROWS, LM_COLS) + 4 * LM_COLS + 8, r["t_lm"],
                                                        None, r["lm_reps"]),
    }
    kernels.update(r["singles"])
    copy_gbs, read_gbs, read100_gbs = ceilings(B)
    clock_khz, bus_bits = qg.device_memory(0)
    if args.suite in ("all", "plans"):
        log("bench: other workloads")
        run_ffn(B, kernels)
        run_extras(B, kernels)
    if args.suite == "plans":
        run_plans(B, kernels)
    achieved = pass_bytes() / r["t_pass"] / 1e9
    ps = r["per_step"]
    out = {
        "metric": "Q4_0/Q8_0 GEMV+GEMM achieved HBM GB/s and % of MI355X peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0/q8_0 weights, f16 activation operands (16-column tiles), f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "prefill: 512-token prompt as 32 passes of 16 columns over Q4_0 and Q8_0 "
                               "5120->17408 and 17408->5120 (one launch per pass), then the LM head Q8_0 "
                               "5120->248320 with GPU argmax",
                   "bytes_per_step": int(sb), "passes": PASSES, "tokens_per_s": round(16 * PASSES / t_step, 1),
                   "ms_per_step_median": round(float(np.median(ps)) * 1e3, 5),
                   "ms_per_step_min": round(min(ps) * 1e3, 5),
                   "frac_peak": round(value / PEAK_HBM_GBS, 4),
                   "copy_ceiling_GB_s": round(copy_gbs, 1),
                   "read_ceiling_GB_s": round(read_gbs, 1),
                   "read_100MB_GB_s": round(read100_gbs, 1),
                   "device_memory_clock_kHz": clock_khz, "device_memory_bus_bits": bus_bits,
                   "device_peak_GB_s": round(2 * clock_khz * 1e3 * bus_bits / 8 / 1e9, 1)},
        "roofline": {"bound": "hbm", "kernel": "gemm16_batch_kernel (one prefill pass: 4 matrices x 16 columns)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": int(pass_bytes()), "us_per_launch": round(r["t_pass"] * 1e6, 3),
                     "frac_of_read_ceiling": round(achieved / read_gbs, 4)},
        "kernels": kernels,
        # the pages' own figures (WebGPU on a GB10, a 27B model): context, not targets
        "context": {"pages_gb10_webgpu": {"gemv_stream_GB_s": 183, "prefill_batched_tok_s": "3 -> 39",
                                          "gemm16_prefill_tok_s": "34.6 -> 56.7",
                                          "verify_tok_s": "12.8 -> 15.4"}},
    }
    if not args.no_cpu:
        log("bench: cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(r["raws"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
