"""lmhead_argmax_noalloc (the LM head on the library-owned scratch, for
callers that cannot allocate) through the C-ABI: the same index and the
same value bits as lmhead_argmax with a caller workspace, on two calls in a
row (the second on a smaller head, so stale scratch from the first would
show), and inside a captured HIP graph, replayed with eager calls between."""
import numpy as np
import pytest

import synth
from gpu_helpers import say, up

pytestmark = pytest.mark.gpu

Q4, Q8 = synth.Q4_0, synth.Q8_0


def _head(env, qtype, rows, cols, seed):
    torch, qg, dev = env
    raw = synth.gen_weights(qtype, rows, cols, 0.02 if qtype == Q4 else 0.005, np.random.default_rng(seed))
    return qg.qg_repack(qtype, up(env, raw.reshape(-1)), rows, cols)


def _with_ws(env, W, x, n_rows):
    torch, qg, dev = env
    L = qg.lib
    idx = torch.full((1,), -1, dtype=torch.int32, device=dev)
    val = torch.zeros(1, dtype=torch.float32, device=dev)
    ws = qg.workspace(L.qg_lmhead_ws_bytes(W.rows, W.cols), dev)
    st = L.lmhead_argmax(W.qtype, W.qs.data_ptr(), W.d.data_ptr(), W.rows, W.cols, n_rows, x.data_ptr(),
                         idx.data_ptr(), val.data_ptr(), ws.data_ptr(), ws.numel(),
                         torch.cuda.current_stream(dev).cuda_stream)
    assert st == 0, st
    return idx, val


def _noalloc(env, W, x, n_rows, idx, val):
    torch, qg, dev = env
    return qg.lib.lmhead_argmax_noalloc(W.qtype, W.qs.data_ptr(), W.d.data_ptr(), W.rows, W.cols, n_rows,
                                        x.data_ptr(), idx.data_ptr(), val.data_ptr(),
                                        torch.cuda.current_stream(dev).cuda_stream)


def test_noalloc_equals_workspace_call(env):
    torch, qg, dev = env
    cases = [(Q8, 70000, 1024, 70000, 81), (Q4, 3000, 512, 2900, 82)]   # the second call is smaller
    for qtype, rows, cols, n_rows, seed in cases:
        say(f"noalloc lm head qtype={qtype} {rows}x{cols} n_rows={n_rows}")
        W = _head(env, qtype, rows, cols, seed)
        x = up(env, synth.gen_x(cols, 1, cfg_id=seed)[:, 0])
        idx_a, val_a = _with_ws(env, W, x, n_rows)
        idx_b = torch.full((1,), -1, dtype=torch.int32, device=dev)
        val_b = torch.zeros(1, dtype=torch.float32, device=dev)
        assert _noalloc(env, W, x, n_rows, idx_b, val_b) == 0
        torch.cuda.synchronize()
        assert int(idx_b.item()) == int(idx_a.item())
        assert val_b.cpu().numpy().view(np.uint32)[0] == val_a.cpu().numpy().view(np.uint32)[0]


def test_noalloc_in_graph(env):
    torch, qg, dev = env
    W = _head(env, Q8, 20000, 2048, 83)
    xs = [up(env, synth.gen_x(2048, 1, cfg_id=84 + i)[:, 0]) for i in range(2)]
    x = xs[0].clone()
    idx = torch.full((1,), -1, dtype=torch.int32, device=dev)
    val = torch.zeros(1, dtype=torch.float32, device=dev)
    want = [_with_ws(env, W, xi, 20000) for xi in xs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            assert _noalloc(env, W, x, 20000, idx, val) == 0
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(4):
        x.copy_(xs[r % 2])
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        wi, wv = want[r % 2]
        assert int(idx.item()) == int(wi.item()), r
        assert val.cpu().numpy().view(np.uint32)[0] == wv.cpu().numpy().view(np.uint32)[0], r
        # an eager call between replays (a smaller head, same scratch)
        Ws = _head(env, Q4, 1000, 512, 85 + r)
        xe = up(env, synth.gen_x(512, 1, cfg_id=90 + r)[:, 0])
        ie = torch.full((1,), -1, dtype=torch.int32, device=dev)
        ve = torch.zeros(1, dtype=torch.float32, device=dev)
        assert _noalloc(env, Ws, xe, 1000, ie, ve) == 0
        ia, va = _with_ws(env, Ws, xe, 1000)
        torch.cuda.synchronize()
        assert int(ie.item()) == int(ia.item())
