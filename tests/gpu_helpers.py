"""Helpers shared by the GPU parity tests (no GPU work at import time)."""
import sys

import numpy as np

from oracle import ops

# Relative error an activation operand may carry into the products of 1..8
# columns: each value enters as an f16 hi / lo pair under a power of two,
# 22 significant bits (the rounding count of the sums is covered by the
# gamma_K factor, whose term count is far above the roundings any path
# takes).  Certification of argmax, top-k and routing uses it.
EPS_OP = 2.0 ** -22


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def up(env, a):
    torch, _, dev = env
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def assert_tol(got, ref, tol, what):
    err = np.abs(got - ref)
    ratio = float(np.max(err / tol)) if err.size else 0.0
    say(f"  {what}: max err/tol = {ratio:.3g}")
    assert np.all(err <= tol), f"{what}: {int(np.sum(err > tol))} elements out of tolerance, worst ratio {ratio}"


def check_routing(idx_gpu, w_gpu, res, top_k, hidden):
    """Router top-k of every token against the oracle.  The selected set must
    be certified (the caller searched for such inputs) and is compared
    exactly; the order inside it is compared exactly where the error bound
    forces it, else the (index, weight) pairs are compared as a set."""
    lg, la = res["logits"], res["logit_a"]
    assert np.all(ops.routing_certified(lg, la, top_k, hidden)), "routing not certified"
    ordered = ops.routing_certified(lg, la, top_k, hidden, order=True)
    for t in range(idx_gpu.shape[0]):
        gi, gw = idx_gpu[t].astype(np.int64), w_gpu[t]
        oi, ow = res["idx"][t], res["p"][t]
        if ordered[t]:
            assert np.array_equal(gi, oi), (t, gi, oi)
            assert np.all(np.abs(gw - ow) <= 1e-5), (t, gw, ow)
        else:
            sg, so = np.argsort(gi), np.argsort(oi)
            assert np.array_equal(gi[sg], oi[so]), (t, gi, oi)
            assert np.all(np.abs(gw[sg] - ow[so]) <= 1e-5), (t, gw, ow)
    return int(np.sum(ordered))


def check_topk_order(idx, val, want, ref, a, k_terms):
    """GPU top-k against the oracle's when the error bound forces the set:
    the same rows; values within the bound; the GPU's own list ordered by
    its values (then rows); and the oracle's order wherever the bound
    separates two of its rows."""
    got = np.asarray(idx).astype(np.int64)
    v = np.asarray(val).astype(np.float64)
    assert sorted(got) == sorted(want)
    assert np.all(np.abs(v - ref[got]) <= ops.tol_dot(a[got]))
    assert all(v[i] > v[i + 1] or (v[i] == v[i + 1] and got[i] < got[i + 1]) for i in range(len(got) - 1))
    gam = k_terms * ops.U32 / (1 - k_terms * ops.U32)
    bound = (gam + EPS_OP * (1 + gam)) * a
    pos = {int(r): i for i, r in enumerate(got)}
    for i, ri in enumerate(want):
        for rj in want[i + 1:]:
            if ref[ri] - bound[ri] > ref[rj] + bound[rj]:
                assert pos[int(ri)] < pos[int(rj)], (ri, rj)
