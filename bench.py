"""Bench: achieved HBM GB/s of the block-quantised products on one MI355X.

`value` is the decode-FFN step of a 27B-like layer at batch 1 (fused gate/up
Q4_0 5120 -> 2 x 17408 with SiLU, then down Q4_0 17408 -> 5120 accumulated
into the residual): algorithmic bytes per step x steps / time.  The other
workloads (decode GEMV 2048 x 2048, verify GEMVs at 4 and 8 columns, the
16-column prefill GEMMs, the LM head + argmax, the MoE FFN at 1 and 16
tokens) are timed the same way and reported under "kernels".

Inputs are seeded synthetic tensors at the pages' model shapes, resident in
HBM before timing.  Every timed loop cycles a pool of byte-identical,
address-distinct weight copies of >= 1 GiB (larger than the 256 MB
Infinity Cache), is captured in a HIP graph (no host launch gaps) and is
timed with events on the stream the kernels run on.

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

    def graph_time(self, fns, iters):
        """Capture `iters` calls (cycling fns) in one HIP graph; return the
        mean time per call in seconds over one timed replay."""
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / iters, g


def kernel_entry(bytes_per_call, t, extra=None):
    gbs = bytes_per_call / t / 1e9
    d = {"us": round(t * 1e6, 3), "bytes": int(bytes_per_call), "GB_s": round(gbs, 1),
         "frac_peak": round(gbs / PEAK_HBM_GBS, 4)}
    if extra:
        d.update(extra)
    return d


def run_ffn(B, steps, warmup):
    """The decode-FFN step: returns (bytes/step, step time, gate/up time, down time)."""
    torch, qg = B.torch, B.qg
    Q4 = qg.Q4_0
    N, K = 17408, 5120
    wg, graw = B.matrix(Q4, N, K, seed=21, sigma=0.02)
    wu, uraw = B.matrix(Q4, N, K, seed=22, sigma=0.02)
    wd, draw = B.matrix(Q4, K, N, seed=23, sigma=0.02)
    set_bytes = 3 * qbytes(Q4, N, K)
    n = max(2, -(-POOL_BYTES // set_bytes))
    pg, pu, pd = B.pool(wg, set_bytes)[:n], B.pool(wu, set_bytes)[:n], B.pool(wd, set_bytes)[:n]
    import synth
    x = B.up(synth.gen_x(K, 1, cfg_id=2).T)
    y = B.up(synth.rng(2, 90).standard_normal((1, K)).astype(np.float32))
    h = torch.empty((1, N), dtype=torch.float32, device=B.dev)
    gu_bytes = 2 * qbytes(Q4, N, K) + 4 * K + 4 * N
    dn_bytes = qbytes(Q4, K, N) + 4 * N + 8 * K
    step_bytes = gu_bytes + dn_bytes

    def step(i):
        qg.gateup_silu(pg[i], pu[i], x, h)
        qg.qgemv(pd[i], h, y, accumulate=True)

    steps_fns = [lambda i=i: step(i) for i in range(n)]
    # W warm-up steps, then exactly K timed steps, barrier + sync on both sides
    if warmup > 0:
        _, gw = B.graph_time(steps_fns, warmup)
    t_step, _ = B.graph_time(steps_fns, steps)
    t_gu, _ = B.graph_time([lambda i=i: qg.gateup_silu(pg[i], pu[i], x, h) for i in range(n)], 4 * n)
    t_dn, _ = B.graph_time([lambda i=i: qg.qgemv(pd[i], h, y, accumulate=True) for i in range(n)], 4 * n)
    # RMSNorm ahead of gate/up: folded into the call, and as its own launch
    # first (the same algorithmic bytes: weights, x, gamma, h)
    gam = B.up(synth.rng(3, K).uniform(0.5, 1.5, K).astype(np.float32))
    xn = torch.empty_like(x)
    t_gun, _ = B.graph_time([lambda i=i: qg.gateup_silu_rmsnorm(pg[i], pu[i], x, gam, 1e-6, h) for i in range(n)],
                            4 * n)

    def norm_then_gu(i):
        qg.rmsnorm(x, gam, 1e-6, xn)
        qg.gateup_silu(pg[i], pu[i], xn, h)

    t_ngu, _ = B.graph_time([lambda i=i: norm_then_gu(i) for i in range(n)], 4 * n)
    norm = {"gateup_rmsnorm_fused_q4_0_5120to2x17408": (gu_bytes + 4 * K, t_gun),
            "rmsnorm_then_gateup_q4_0_5120to2x17408": (gu_bytes + 4 * K, t_ngu)}
    raws = (graw, uraw, draw)
    del pg, pu, pd
    return step_bytes, t_step, gu_bytes, t_gu, dn_bytes, t_dn, raws, norm


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
    kernels["gemv_q4_0_2048x2048_1col"] = kernel_entry(qbytes(Q4, 2048, 2048) + 8192 * 2, t)
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
                                                             {"tokens_per_s": round(nc / t, 1)})
        del p
    log("  verify done")

    # 16-column prefill GEMMs
    for qtype in (Q4, Q8):
        for N, K in ((17408, 5120), (5120, 17408)):
            w, _ = B.matrix(qtype, N, K, seed=41, sigma=0.005 if qtype == Q8 else 0.02)
            p = B.pool(w, qbytes(qtype, N, K))
            x = B.up(synth.gen_x(K, 16, cfg_id=4).T)
            y = torch.empty((16, N), device=B.dev)
            t, _ = B.graph_time([lambda m=m: qg.qgemm16(m, x, y) for m in p], 2 * len(p))
            nm = f"gemm16_{'q4_0' if qtype == Q4 else 'q8_0'}_{K}to{N}"
            kernels[nm] = kernel_entry(qbytes(qtype, N, K) + 64 * (N + K), t,
                                       {"tokens_per_s": round(16 / t, 1)})
            del p
    log("  gemm16 done")

    # LM head + argmax, Q8_0 248,320 x 5120
    N, K = 248320, 5120
    w, _ = B.matrix(Q8, N, K, seed=51, sigma=0.005)
    p = [w, qg.QMatrix(w.qtype, w.rows, w.cols, 1, w.qs.clone(), w.d.clone())]
    x = B.up(synth.gen_x(K, 1, cfg_id=4)[:, 0])
    oi = torch.empty(1, dtype=torch.int32, device=B.dev)
    ov = torch.empty(1, dtype=torch.float32, device=B.dev)
    t, _ = B.graph_time([lambda m=m: qg.lmhead_argmax(m, x, None, oi, ov) for m in p], 20)
    kernels["lmhead_argmax_q8_0_5120to248320"] = kernel_entry(qbytes(Q8, N, K) + 4 * K + 8, t)
    # the same head returning the 10 best (value, row) pairs (the Three.js
    # page's example asks for top-k 10)
    ti = torch.empty(10, dtype=torch.int32, device=B.dev)
    tv = torch.empty(10, dtype=torch.float32, device=B.dev)
    t, _ = B.graph_time([lambda m=m: qg.lmhead_topk(m, x, 10, None, ti, tv) for m in p], 20)
    kernels["lmhead_topk10_q8_0_5120to248320"] = kernel_entry(qbytes(Q8, N, K) + 4 * K + 80, t)
    del p, w
    log("  lmhead done")

    # load-time requantisation of a Q4_1 17408 x 5120 matrix to Q8_0 (bytes
    # read + written)
    nbk = 17408 * 5120 // 32
    src = torch.randint(0, 256, (nbk * 20,), dtype=torch.uint8, device=B.dev)
    src.view(nbk, 20)[:, 1] = 0x3C        # finite scales near 1 (f16 high byte)
    src.view(nbk, 20)[:, 3] = 0xBC        # offsets near -1
    dst = torch.empty(nbk * 34, dtype=torch.uint8, device=B.dev)
    t, _ = B.graph_time([lambda: qg.requant_q8_0(qg.Q4_1, src, nbk, dst)], 20)
    kernels["requant_q4_1_to_q8_0_17408x5120"] = kernel_entry(nbk * (20 + 34), t)
    del src, dst
    log("  requant done")

    # MoE FFN, 256 experts (8 active) + shared, hidden 2048, ffn 512
    E, H, F, k = 256, 2048, 512, 8
    g = np.random.default_rng(61)
    def stack(rows, cols):
        raw = np.stack([synth.gen_weights(Q4, rows, cols, 0.02, g) for _ in range(E)])
        return qg.qg_repack(Q4, B.up(raw.reshape(-1)), rows, cols, E)
    gate, upm, down = stack(F, H), stack(F, H), stack(H, F)
    sh = [B.matrix(Q4, r, c, seed=62 + i, sigma=0.02)[0] for i, (r, c) in enumerate(((F, H), (F, H), (H, F)))]
    router = B.up(synth.gen_f32((E, H), 0.02, g))
    layer_bytes = 3 * E * qbytes(Q4, F, H)
    copies = max(2, -(-POOL_BYTES // layer_bytes))
    cl = lambda m: qg.QMatrix(m.qtype, m.rows, m.cols, m.n_mat, m.qs.clone(), m.d.clone())
    moes = []
    for c in range(copies):
        gg, uu, dd = (gate, upm, down) if c == 0 else (cl(gate), cl(upm), cl(down))
        moes.append(qg.MoE(hidden=H, ffn=F, n_expert=E, top_k=k, router=router, gate=gg, up=uu,
                           down=dd, sh_gate=sh[0], sh_up=sh[1], sh_down=sh[2]))
    eb = qbytes(Q4, F, H) * 3
    for T in (1, 16):
        X = B.up(synth.gen_x(H, T, cfg_id=5).T)
        Y = torch.zeros((T, H), device=B.dev)
        tidx = torch.empty((T, k), dtype=torch.int32, device=B.dev)
        qg.moe_ffn(moes[0], X, Y, tidx)
        torch.cuda.synchronize()
        U = len(np.unique(tidx.cpu().numpy()))
        nbytes = 4 * E * H + eb * (U + 1) + 4 * H * T + 8 * H * T
        t, _ = B.graph_time([lambda m=m: qg.moe_ffn(m, X, Y) for m in moes], 4 * copies)
        kernels[f"moe_ffn_{T}tok"] = kernel_entry(nbytes, t, {"distinct_experts": U,
                                                             "tokens_per_s": round(T / t, 1)})
        # the RMSNorm ahead of router and experts: folded into the layer, and
        # as its own launch first (the same algorithmic bytes plus the weights)
        gam = B.up(synth.rng(63, H).uniform(0.5, 1.5, H).astype(np.float32))
        for m in moes:
            m.norm_weight, m.norm_eps = gam, 1e-6
        t_nf, _ = B.graph_time([lambda m=m: qg.moe_ffn(m, X, Y) for m in moes], 4 * copies)
        for m in moes:
            m.norm_weight = None
        Xn = torch.empty_like(X)

        def norm_then_moe(m):
            qg.rmsnorm(X, gam, 1e-6, Xn)
            qg.moe_ffn(m, Xn, Y)

        t_nu, _ = B.graph_time([lambda m=m: norm_then_moe(m) for m in moes], 4 * copies)
        kernels[f"moe_ffn_rmsnorm_fused_{T}tok"] = kernel_entry(nbytes + 4 * H, t_nf)
        kernels[f"rmsnorm_then_moe_ffn_{T}tok"] = kernel_entry(nbytes + 4 * H, t_nu)
    del moes, gate, upm, down
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


# the sources of the gate/up kernel whose counters the traffic summary holds
TRAFFIC_SOURCES = ("gemm_q4_q8_amd/csrc/qmv.hip", "gemm_q4_q8_amd/csrc/dot_unit.h",
                   "gemm_q4_q8_amd/csrc/common.h")


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, or
    None when the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gateup_silu_q4_0_decode_ffn_traffic.txt")
    try:
        fields = dict(l.split()[0:2] for l in open(path) if l.strip() and not l.startswith("#")
                      and len(l.split()) == 2)
    except OSError:
        return None
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("kernel_source_hash") != h.hexdigest()[:16]:
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def cpu_baseline(raws, min_seconds=12.0):
    """The oracle, as it stands, on full decode-FFN steps, repeated until at
    least `min_seconds` of host work."""
    import synth
    from oracle import ops
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = 1
    graw, uraw, draw = raws
    x = synth.gen_x(5120, 1, cfg_id=2)[:, 0]
    y_in = synth.rng(2, 90).standard_normal(5120).astype(np.float32)
    reps = 0
    t0 = time.perf_counter()
    while True:
        h, _, _, _ = ops.gateup_silu(2, graw, uraw, x)
        ops.gemv(2, draw, h.astype(np.float32), y_in=y_in)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    nbytes = 3 * qbytes(2, 17408, 5120) + 4 * 5120 + 4 * 17408 + 4 * 17408 + 8 * 5120
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"full decode-FFN steps (gate/up 17408x5120 + down 5120x17408, Q4_0, batch 1), "
                      f"{reps} repetitions in {dt * reps:.1f} s, {dt:.2f} s per step; f64 numpy, "
                      f"BLAS threads={threads}"}


def traffic_run(B):
    """Fixed launches for hardware-counter runs (rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE): 5 element-wise copies of exactly 1 GiB (read 1 GiB, write
    1 GiB) as the scale reference, then 16 fused gate/up launches of the
    decode FFN shape over 8 address-distinct weight sets."""
    torch, qg = B.torch, B.qg
    a = torch.empty(POOL_BYTES // 4, dtype=torch.float32, device=B.dev).normal_()
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    del a, b
    N, K = 17408, 5120
    ws = [(B.matrix(2, N, K, seed=21 + i, sigma=0.02)[0], B.matrix(2, N, K, seed=41 + i, sigma=0.02)[0])
          for i in range(8)]
    import synth
    x = B.up(synth.gen_x(K, 1, cfg_id=2).T)
    h = torch.empty((1, N), dtype=torch.float32, device=B.dev)
    torch.cuda.synchronize()
    for i in range(16):
        qg.gateup_silu(ws[i % 8][0], ws[i % 8][1], x, h)
    torch.cuda.synchronize()
    print("traffic run done", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--suite", choices=["all", "main"], default="all")
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

    log("bench: decode FFN step")
    step_bytes, t_step, gu_bytes, t_gu, dn_bytes, t_dn, raws, norm = run_ffn(B, args.steps, args.warmup)
    value = step_bytes / t_step / 1e9
    kernels = {
        "gateup_silu_q4_0_5120to2x17408": kernel_entry(gu_bytes, t_gu),
        "qgemv_q4_0_17408to5120_acc": kernel_entry(dn_bytes, t_dn),
    }
    for nm, (nb, tt) in norm.items():
        kernels[nm] = kernel_entry(nb, tt)
    copy_gbs, read_gbs, read100_gbs = ceilings(B)
    if args.suite == "all":
        log("bench: other workloads")
        run_extras(B, kernels)
        run_plans(B, kernels)
    achieved = gu_bytes / t_gu / 1e9
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
        "dtype": "q4_0 weights, f16 activation operands, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "27B-like decode FFN layer, batch 1: gate/up Q4_0 5120->2x17408 + SiLU, "
                               "down Q4_0 17408->5120 y+=W.h",
                   "bytes_per_step": int(step_bytes), "tokens_per_s": round(1.0 / t_step, 1),
                   "frac_peak": round(value / PEAK_HBM_GBS, 4),
                   "copy_ceiling_GB_s": round(copy_gbs, 1),
                   "read_ceiling_GB_s": round(read_gbs, 1),
                   "read_100MB_GB_s": round(read100_gbs, 1)},
        "roofline": {"bound": "hbm", "kernel": "gateup_silu (Q4_0, 1 column)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": int(gu_bytes), "us_per_launch": round(t_gu * 1e6, 3),
                     "frac_of_read_ceiling": round(achieved / read_gbs, 4)},
        "kernels": kernels,
        # the pages' own figures (WebGPU on a GB10, a 27B model): context, not targets
        "context": {"pages_gb10_webgpu": {"gemv_stream_GB_s": 183, "prefill_batched_tok_s": "3 -> 39",
                                          "gemm16_prefill_tok_s": "34.6 -> 56.7",
                                          "verify_tok_s": "12.8 -> 15.4"}},
    }
    if not args.no_cpu:
        log("bench: cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(raws)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
