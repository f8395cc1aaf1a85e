"""Python binding of libqgemm (block-quantised Q4_0 / Q8_0 products, gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  The functions carry
the C-ABI names declared in include/qgemm.h; `lib` is the raw ctypes handle.

Importing fails loudly when the built library is missing: there is no
fallback.  Build it with `python gemm_q4_q8_amd/build.py`.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemm.so")

Q4_0 = 2
Q8_0 = 8
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34}
STATUS = {0: "QG_OK", -1: "QG_EINVAL", -2: "QG_ESHAPE", -3: "QG_EALIGN",
          -4: "QG_EUNSUPPORTED", -5: "QG_EWORKSPACE", -6: "QG_EHIP"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built (python gemm_q4_q8_amd/build.py)")
# torch ships its own HIP runtime.  Load it first so that the library binds to
# the same runtime instance: streams and events are runtime objects, and a
# second runtime in the process would not know torch's streams.
import torch  # noqa: E402,F401
lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class qg_moe(ctypes.Structure):
    _fields_ = [
        ("hidden", _i64), ("ffn", _i64),
        ("n_expert", _i32), ("top_k", _i32), ("normalize_topk", _i32),
        ("qtype", _i32),
        ("router", _vp),
        ("gate_qs", _vp), ("up_qs", _vp), ("down_qs", _vp),
        ("gate_d", _vp), ("up_d", _vp), ("down_d", _vp),
        ("sh_ffn", _i64),
        ("sh_gate_qs", _vp), ("sh_up_qs", _vp), ("sh_down_qs", _vp),
        ("sh_gate_d", _vp), ("sh_up_d", _vp), ("sh_down_d", _vp),
        ("norm_weight", _vp), ("norm_eps", ctypes.c_float),
    ]


class qg_gemm16_problem(ctypes.Structure):
    _fields_ = [
        ("qtype", _i32), ("accumulate", _i32),
        ("qs", _vp), ("d", _vp),
        ("rows", _i64), ("cols", _i64),
        ("X", _vp), ("ldx", _i64),
        ("Y", _vp), ("ldy", _i64),
    ]


BATCH_MAX = 8

_SIGS = {
    "qg_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "qg_last_hip_error": (ctypes.c_char_p, []),
    "qg_packed_bytes": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64,
                                       ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "qg_repack": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "qg_gemv_ws_bytes": (_sz, [_i64, _i64]),
    "qgemv_q4_0": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _i64, _i32, _vp, _i64, _i32,
                                  _vp, _sz, _vp]),
    "qgemv_q8_0": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _i64, _i32, _vp, _i64, _i32,
                                  _vp, _sz, _vp]),
    "qg_gemm16_ws_bytes": (_sz, [ctypes.c_int, _i64, _i64]),
    "qgemm16": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i32,
                               _vp, _sz, _vp]),
    "qg_gemm16_batch_ws_bytes": (_sz, [ctypes.POINTER(qg_gemm16_problem), _i32]),
    "qg_gemm16_batch_splits": (ctypes.c_int, [ctypes.POINTER(qg_gemm16_problem), _i32, ctypes.POINTER(ctypes.c_int32)]),
    "qgemm16_batch": (ctypes.c_int, [ctypes.POINTER(qg_gemm16_problem), _i32, _vp, _sz, _vp]),
    "qg_gateup_ws_bytes": (_sz, [_i64, _i64]),
    "gateup_silu": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i64, _i32,
                                   _vp, _i64, _vp, _sz, _vp]),
    "gateup_silu_rmsnorm": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i64, _i32,
                                           _vp, ctypes.c_float, _vp, _i64, _vp, _sz, _vp]),
    "qg_rmsnorm": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, ctypes.c_float, _vp, _i64, _vp]),
    "qg_requant_q8_0": (ctypes.c_int, [ctypes.c_int, _i64, _vp, _vp, _vp]),
    "qg_lmhead_ws_bytes": (_sz, [_i64, _i64]),
    "qg_lmhead_topk_ws_bytes": (_sz, [_i64, _i64, _i32]),
    "lmhead_topk": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp,
                                   _vp, _sz, _vp]),
    "lmhead_argmax_noalloc": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "lmhead_argmax": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                                     _vp, _sz, _vp]),
    "qg_moe_ws_bytes": (_sz, [ctypes.POINTER(qg_moe), _i32]),
    "moe_ffn": (ctypes.c_int, [ctypes.POINTER(qg_moe), _vp, _i64, _i32, _vp, _i64, _vp, _vp,
                               _vp, _sz, _vp]),
    "qg_read_probe": (ctypes.c_int, [_vp, _sz, _vp, _vp]),
    "qg_device_memory": (ctypes.c_int, [_i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "qg_tune_gemv": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _i64, _i64, _vp, _i64, _i32, _vp, _i64,
                                    _vp, _sz, _vp, _i32, _vp]),
    "qg_tune_gateup": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i64, _i32,
                                      _vp, _i64, _vp, _sz, _vp, _i32, _vp]),
    "qg_tune_lmhead": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                                      _vp, _sz, _vp, _i32, _vp]),
    "qg_plan_set": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, _i64, _i32, _i32]),
    "qg_plan_get": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, _i64, _i32, _vp]),
    "qg_plan_reset": (None, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class QGError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = f"{what}: {STATUS.get(status, status)} ({lib.qg_strerror(status).decode()})"
        if status == -6:
            msg += f" [{lib.qg_last_hip_error().decode()}]"
        super().__init__(msg)
        self.status = status


def _check(status: int, what: str):
    if status != 0:
        raise QGError(status, what)


# ---------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


_WS = {}
_WS_RETIRED = []


def workspace(nbytes: int, device, key: str = "default"):
    """A zero-filled device workspace, cached per (device, current stream,
    key).  Its leading counters are zero again after every completed call,
    so one workspace serves any sequence of calls on one stream; calls on
    different streams, which may overlap, get different workspaces.  A
    larger request replaces it with a new zero-filled one, and the old one
    stays allocated for the life of the process: a HIP graph captured
    earlier still holds its address.  Inside a graph capture the workspace
    cannot be created or grown (its zero fill would only run at replay):
    make one eager call of the largest shape on the capture stream first."""
    torch = _torch()
    dev = torch.device(device)
    k = (dev.index, torch.cuda.current_stream(dev).cuda_stream, key)
    ws = _WS.get(k)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("the library workspace of this stream would have to be created or grown "
                               "during graph capture; make one eager call of the largest shape on the "
                               "capture stream first")
        new = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
        if ws is not None:
            _WS_RETIRED.append(ws)
        _WS[k] = new
        ws = new
    return ws


def _check_dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


@dataclass
class QMatrix:
    """A repacked matrix (or a stack of n_mat matrices) on the GPU."""
    qtype: int
    rows: int
    cols: int
    n_mat: int
    qs: object
    d: object


def packed_bytes(qtype: int, rows: int, cols: int, n_mat: int = 1):
    qb, db = _sz(), _sz()
    _check(lib.qg_packed_bytes(qtype, n_mat, rows, cols, ctypes.byref(qb), ctypes.byref(db)),
           "qg_packed_bytes")
    return qb.value, db.value


def qg_repack(qtype: int, blocks, rows: int, cols: int, n_mat: int = 1) -> QMatrix:
    """blocks: uint8 tensor on the GPU holding n_mat*rows*cols/32 GGUF blocks."""
    torch = _torch()
    _check_dev(blocks)
    qb, db = packed_bytes(qtype, rows, cols, n_mat)
    qs = torch.empty(qb, dtype=torch.uint8, device=blocks.device)
    d = torch.empty(db, dtype=torch.uint8, device=blocks.device)
    _check(lib.qg_repack(qtype, n_mat, rows, cols, blocks.data_ptr(), qs.data_ptr(),
                         d.data_ptr(), _stream(blocks.device)), "qg_repack")
    return QMatrix(qtype, rows, cols, n_mat, qs, d)


def _ld(t) -> int:
    """Leading dimension of a column-major [len, ncols] matrix stored as a
    row-major torch tensor of shape [ncols, len] (column j = t[j]).  The stride
    of a size-1 leading axis is meaningless, so a single column gets len."""
    if t.dim() == 1:
        return t.shape[0]
    if t.stride(1) != 1:
        raise ValueError("columns must be contiguous (stride 1 along the last axis)")
    return t.shape[1] if t.shape[0] == 1 else t.stride(0)


def qgemv(w: QMatrix, X, Y=None, accumulate: bool = False):
    """Y[j] = (acc ? Y[j] : 0) + W X[j]; X: [ncols, cols] f32 (ncols 1..8)."""
    torch = _torch()
    _check_dev(X)
    X2 = X if X.dim() == 2 else X.view(1, -1)
    ncols = X2.shape[0]
    if Y is None:
        Y = torch.empty((ncols, w.rows), dtype=torch.float32, device=X.device)
    Y2 = Y if Y.dim() == 2 else Y.view(1, -1)
    ws_b = lib.qg_gemv_ws_bytes(w.rows, w.cols)
    ws = workspace(ws_b, X.device)
    fn = lib.qgemv_q4_0 if w.qtype == Q4_0 else lib.qgemv_q8_0
    _check(fn(w.qs.data_ptr(), w.d.data_ptr(), w.rows, w.cols, X2.data_ptr(), _ld(X2), ncols,
              Y2.data_ptr(), _ld(Y2), int(accumulate), ws.data_ptr(), ws.numel(),
              _stream(X.device)), "qgemv")
    return Y


def qgemv_q4_0(w: QMatrix, X, Y=None, accumulate: bool = False):
    assert w.qtype == Q4_0
    return qgemv(w, X, Y, accumulate)


def qgemv_q8_0(w: QMatrix, X, Y=None, accumulate: bool = False):
    assert w.qtype == Q8_0
    return qgemv(w, X, Y, accumulate)


def qgemm16(w: QMatrix, X, Y=None, accumulate: bool = False):
    """Y = (acc ? Y : 0) + W X; X: [16, cols] f32, Y: [16, rows]."""
    torch = _torch()
    _check_dev(X)
    if X.shape[0] != 16:
        raise ValueError("qgemm16 takes exactly 16 columns")
    if Y is None:
        Y = torch.empty((16, w.rows), dtype=torch.float32, device=X.device)
    ws_b = lib.qg_gemm16_ws_bytes(w.qtype, w.rows, w.cols)
    ws = workspace(ws_b, X.device)
    _check(lib.qgemm16(w.qtype, w.qs.data_ptr(), w.d.data_ptr(), w.rows, w.cols, X.data_ptr(),
                       _ld(X), Y.data_ptr(), _ld(Y), int(accumulate), ws.data_ptr(), ws.numel(),
                       _stream(X.device)), "qgemm16")
    return Y


def _batch_array(items):
    torch = _torch()
    n = len(items)
    arr = (qg_gemm16_problem * max(n, 1))()
    outs = []
    for i, (w, X, Y, acc) in enumerate(items):
        _check_dev(X)
        if X.shape[0] != 16:
            raise ValueError("qgemm16_batch takes exactly 16 columns per problem")
        if Y is None:
            Y = torch.empty((16, w.rows), dtype=torch.float32, device=X.device)
        outs.append(Y)
        arr[i] = qg_gemm16_problem(w.qtype, int(acc), w.qs.data_ptr(), w.d.data_ptr(), w.rows, w.cols,
                                   X.data_ptr(), _ld(X), Y.data_ptr(), _ld(Y))
    dev = items[0][1].device if n else torch.device("cuda:0")
    return arr, n, outs, dev


def qgemm16_batch(items):
    """One launch over several 16-column problems: items is a list of
    (w: QMatrix, X [16, cols], Y [16, rows] or None, accumulate).  Each Y is
    bitwise equal to qgemm16 on that problem with the K split of
    gemm16_batch_splits(items) pinned.  Returns the list of Y."""
    arr, n, outs, dev = _batch_array(items)
    ws = workspace(lib.qg_gemm16_batch_ws_bytes(arr, n), dev)
    _check(lib.qgemm16_batch(arr, n, ws.data_ptr(), ws.numel(), _stream(dev)), "qgemm16_batch")
    return outs


def gemm16_batch_splits(items):
    """The K segments qgemm16_batch uses for each problem of `items` (same
    form as qgemm16_batch's; a None output is allocated for the query)."""
    arr, n, _, _ = _batch_array(items)
    out = (ctypes.c_int32 * max(n, 1))()
    _check(lib.qg_gemm16_batch_splits(arr, n, out), "qg_gemm16_batch_splits")
    return [int(out[i]) for i in range(n)]


def gateup_silu(wg: QMatrix, wu: QMatrix, X, H=None):
    """H[j] = silu(Wg X[j]) * (Wu X[j]); X: [ncols, cols] (ncols 1..8)."""
    torch = _torch()
    _check_dev(X)
    X2 = X if X.dim() == 2 else X.view(1, -1)
    ncols = X2.shape[0]
    if H is None:
        H = torch.empty((ncols, wg.rows), dtype=torch.float32, device=X.device)
    H2 = H if H.dim() == 2 else H.view(1, -1)
    ws = workspace(lib.qg_gateup_ws_bytes(wg.rows, wg.cols), X.device)
    _check(lib.gateup_silu(wg.qtype, wg.qs.data_ptr(), wg.d.data_ptr(), wu.qs.data_ptr(),
                           wu.d.data_ptr(), wg.rows, wg.cols, X2.data_ptr(), _ld(X2), ncols,
                           H2.data_ptr(), _ld(H2), ws.data_ptr(), ws.numel(),
                           _stream(X.device)), "gateup_silu")
    return H


Q4_1, Q5_0, Q5_1 = 3, 6, 7
Q4_K, Q5_K, Q6_K = 12, 13, 14
_REQUANT_RUNS = {Q4_1: 1, Q5_0: 1, Q5_1: 1, Q4_K: 8, Q5_K: 8, Q6_K: 8}


def requant_q8_0(src_type: int, blocks, n_blocks: int, out=None):
    """Q4_1 / Q5_0 / Q5_1 / Q4_K / Q5_K / Q6_K blocks (device uint8) ->
    canonical Q8_0 blocks (device uint8, 34 bytes per 32 values: n_blocks *
    34 bytes, or n_blocks * 8 * 34 for the 256-value K-quant blocks), on the
    GPU."""
    torch = _torch()
    _check_dev(blocks)
    if out is None:
        n_out = n_blocks * _REQUANT_RUNS.get(src_type, 1)
        out = torch.empty(n_out * 34, dtype=torch.uint8, device=blocks.device)
    _check(lib.qg_requant_q8_0(src_type, n_blocks, blocks.data_ptr(), out.data_ptr(), _stream(blocks.device)),
           "qg_requant_q8_0")
    return out


def gateup_silu_rmsnorm(wg: QMatrix, wu: QMatrix, X, gamma, eps: float, H=None):
    """H[j] = silu(Wg n(X[j])) * (Wu n(X[j])), n = RMSNorm with weights gamma
    (cols floats) and eps, folded into the gate/up call."""
    torch = _torch()
    _check_dev(X, gamma)
    X2 = X if X.dim() == 2 else X.view(1, -1)
    ncols = X2.shape[0]
    if H is None:
        H = torch.empty((ncols, wg.rows), dtype=torch.float32, device=X.device)
    H2 = H if H.dim() == 2 else H.view(1, -1)
    ws = workspace(lib.qg_gateup_ws_bytes(wg.rows, wg.cols), X.device)
    _check(lib.gateup_silu_rmsnorm(wg.qtype, wg.qs.data_ptr(), wg.d.data_ptr(), wu.qs.data_ptr(),
                                   wu.d.data_ptr(), wg.rows, wg.cols, X2.data_ptr(), _ld(X2), ncols,
                                   gamma.data_ptr(), float(eps), H2.data_ptr(), _ld(H2), ws.data_ptr(),
                                   ws.numel(), _stream(X.device)), "gateup_silu_rmsnorm")
    return H


def rmsnorm(X, gamma, eps: float, Y=None):
    """Y[j] = X[j] * gamma / sqrt(mean(X[j]^2) + eps); X: [ncols, cols]; Y may be X."""
    torch = _torch()
    _check_dev(X, gamma)
    X2 = X if X.dim() == 2 else X.view(1, -1)
    if Y is None:
        Y = torch.empty_like(X2)
    Y2 = Y if Y.dim() == 2 else Y.view(1, -1)
    _check(lib.qg_rmsnorm(X2.data_ptr(), _ld(X2), X2.shape[1], X2.shape[0], gamma.data_ptr(), float(eps),
                          Y2.data_ptr(), _ld(Y2), _stream(X.device)), "qg_rmsnorm")
    return Y


def read_probe(t, sink=None):
    """Measurement aid: read every byte of device tensor `t` once (the
    bench's streaming-read ceiling).  Returns the sink tensor."""
    torch = _torch()
    _check_dev(t)
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=t.device)
    _check(lib.qg_read_probe(t.data_ptr(), t.numel() * t.element_size(), sink.data_ptr(),
                             _stream(t.device)), "qg_read_probe")
    return sink

def device_memory(device: int = 0):
    """(memory clock in kHz, bus width in bits) as the HIP runtime reports them."""
    c, w = _i32(), _i32()
    _check(lib.qg_device_memory(device, ctypes.byref(c), ctypes.byref(w)), "qg_device_memory")
    return c.value, w.value


def lmhead_argmax(w: QMatrix, x, n_rows: Optional[int] = None, out_idx=None, out_val=None):
    """Returns (idx int32 [1], val f32 [1]) on the GPU (no host sync)."""
    torch = _torch()
    _check_dev(x)
    if out_idx is None:
        out_idx = torch.empty(1, dtype=torch.int32, device=x.device)
    if out_val is None:
        out_val = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = workspace(lib.qg_lmhead_ws_bytes(w.rows, w.cols), x.device, "lmhead")
    _check(lib.lmhead_argmax(w.qtype, w.qs.data_ptr(), w.d.data_ptr(), w.rows, w.cols,
                             w.rows if n_rows is None else n_rows, x.data_ptr(),
                             out_idx.data_ptr(), out_val.data_ptr(), ws.data_ptr(), ws.numel(),
                             _stream(x.device)), "lmhead_argmax")
    return out_idx, out_val


def lmhead_topk(w: QMatrix, x, k: int, n_rows: Optional[int] = None, out_idx=None, out_val=None):
    """The k largest logits of W x over rows < n_rows, value descending then
    row ascending: (idx int32 [k], val f32 [k]) on the GPU (no host sync)."""
    torch = _torch()
    _check_dev(x)
    if out_idx is None:
        out_idx = torch.empty(k, dtype=torch.int32, device=x.device)
    if out_val is None:
        out_val = torch.empty(k, dtype=torch.float32, device=x.device)
    ws = workspace(lib.qg_lmhead_topk_ws_bytes(w.rows, w.cols, k), x.device, "lmhead_topk")
    _check(lib.lmhead_topk(w.qtype, w.qs.data_ptr(), w.d.data_ptr(), w.rows, w.cols,
                           w.rows if n_rows is None else n_rows, x.data_ptr(), k,
                           out_idx.data_ptr(), out_val.data_ptr(), ws.data_ptr(), ws.numel(),
                           _stream(x.device)), "lmhead_topk")
    return out_idx, out_val


# ------------------------------------------------------------ launch plans
OP_GEMV, OP_GATEUP, OP_LMHEAD = 0, 1, 2
PLAN_SW = 0x100
PLAN_STRICT = 0x200
TUNE_SPLIT = 1


def PLAN_SPLIT(s: int) -> int:
    """Plan bits for s K segments instead of the shape's own."""
    return s << 12


def tune_gemv(w: QMatrix, X, Y=None, split: bool = False) -> int:
    """Times the launch plans of qgemv (1..8 columns) or qgemm16 (16) on
    these buffers (with split: K splits too), keeps the winner for this
    shape and column count, and returns it; Y ends holding W X."""
    torch = _torch()
    _check_dev(X)
    X2 = X if X.dim() == 2 else X.view(1, -1)
    ncols = X2.shape[0]
    if Y is None:
        Y = torch.empty((ncols, w.rows), dtype=torch.float32, device=X.device)
    Y2 = Y if Y.dim() == 2 else Y.view(1, -1)
    ws_b = lib.qg_gemm16_ws_bytes(w.qtype, w.rows, w.cols) if ncols == 16 else lib.qg_gemv_ws_bytes(w.rows, w.cols)
    ws = workspace(ws_b, X.device)
    plan = ctypes.c_int32(-1)
    _check(lib.qg_tune_gemv(w.qtype, w.qs.data_ptr(), w.d.data_ptr(), w.rows, w.cols, X2.data_ptr(), _ld(X2),
                            ncols, Y2.data_ptr(), _ld(Y2), ws.data_ptr(), ws.numel(), _stream(X.device),
                            int(split), ctypes.addressof(plan)), "qg_tune_gemv")
    return plan.value


def tune_gateup(wg: QMatrix, wu: QMatrix, X, H=None, split: bool = False) -> int:
    """As tune_gemv for gateup_silu; H ends holding the gated product."""
    torch = _torch()
    _check_dev(X)
    X2 = X if X.dim() == 2 else X.view(1, -1)
    ncols = X2.shape[0]
    if H is None:
        H = torch.empty((ncols, wg.rows), dtype=torch.float32, device=X.device)
    H2 = H if H.dim() == 2 else H.view(1, -1)
    ws = workspace(lib.qg_gateup_ws_bytes(wg.rows, wg.cols), X.device)
    plan = ctypes.c_int32(-1)
    _check(lib.qg_tune_gateup(wg.qtype, wg.qs.data_ptr(), wg.d.data_ptr(), wu.qs.data_ptr(), wu.d.data_ptr(),
                              wg.rows, wg.cols, X2.data_ptr(), _ld(X2), ncols, H2.data_ptr(), _ld(H2),
                              ws.data_ptr(), ws.numel(), _stream(X.device), int(split), ctypes.addressof(plan)),
           "qg_tune_gateup")
    return plan.value


def tune_lmhead(w: QMatrix, x, n_rows: Optional[int] = None, split: bool = False) -> int:
    """As tune_gemv for lmhead_argmax (the entry serves lmhead_topk too)."""
    torch = _torch()
    _check_dev(x)
    out_idx = torch.empty(1, dtype=torch.int32, device=x.device)
    out_val = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = workspace(lib.qg_lmhead_ws_bytes(w.rows, w.cols), x.device, "lmhead")
    plan = ctypes.c_int32(-1)
    _check(lib.qg_tune_lmhead(w.qtype, w.qs.data_ptr(), w.d.data_ptr(), w.rows, w.cols,
                              w.rows if n_rows is None else n_rows, x.data_ptr(), out_idx.data_ptr(),
                              out_val.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device),
                              int(split), ctypes.addressof(plan)), "qg_tune_lmhead")
    return plan.value


def plan_set(op: int, qtype: int, rows: int, cols: int, ncols: int, plan: int) -> None:
    _check(lib.qg_plan_set(op, qtype, rows, cols, ncols, plan), "qg_plan_set")


def plan_get(op: int, qtype: int, rows: int, cols: int, ncols: int) -> int:
    plan = ctypes.c_int32(-1)
    _check(lib.qg_plan_get(op, qtype, rows, cols, ncols, ctypes.addressof(plan)), "qg_plan_get")
    return plan.value


def plan_reset() -> None:
    lib.qg_plan_reset()


@dataclass
class MoE:
    """Role-stacked experts (gate / up / down stacks) plus optional shared expert."""
    hidden: int
    ffn: int
    n_expert: int
    top_k: int
    router: object            # f32 [n_expert, hidden]
    gate: QMatrix             # n_mat = n_expert, ffn x hidden
    up: QMatrix
    down: QMatrix             # n_mat = n_expert, hidden x ffn
    sh_gate: Optional[QMatrix] = None
    sh_up: Optional[QMatrix] = None
    sh_down: Optional[QMatrix] = None
    normalize_topk: bool = True
    norm_weight: object = None  # f32 [hidden]: RMSNorm ahead of router and experts
    norm_eps: float = 0.0

    @property
    def qtype(self) -> int:
        return self.gate.qtype

    def struct(self) -> qg_moe:
        s = qg_moe()
        s.hidden, s.ffn = self.hidden, self.ffn
        s.n_expert, s.top_k, s.normalize_topk = self.n_expert, self.top_k, int(self.normalize_topk)
        s.qtype = self.gate.qtype
        s.router = self.router.data_ptr()
        s.gate_qs, s.up_qs, s.down_qs = (m.qs.data_ptr() for m in (self.gate, self.up, self.down))
        s.gate_d, s.up_d, s.down_d = (m.d.data_ptr() for m in (self.gate, self.up, self.down))
        if self.sh_gate is not None:
            s.sh_ffn = self.sh_gate.rows
            s.sh_gate_qs, s.sh_up_qs, s.sh_down_qs = (
                m.qs.data_ptr() for m in (self.sh_gate, self.sh_up, self.sh_down))
            s.sh_gate_d, s.sh_up_d, s.sh_down_d = (
                m.d.data_ptr() for m in (self.sh_gate, self.sh_up, self.sh_down))
        else:
            s.sh_ffn = 0
        s.norm_weight = self.norm_weight.data_ptr() if self.norm_weight is not None else None
        s.norm_eps = float(self.norm_eps)
        return s


def moe_ffn(moe: MoE, X, Y, topk_idx=None, topk_w=None):
    """Y[t] += MoE(X[t]) for the ntok = X.shape[0] tokens (<= 16)."""
    _check_dev(X, Y)
    s = moe.struct()
    ntok = X.shape[0]
    ws = workspace(lib.qg_moe_ws_bytes(ctypes.byref(s), ntok), X.device, "moe")
    _check(lib.moe_ffn(ctypes.byref(s), X.data_ptr(), _ld(X), ntok, Y.data_ptr(), _ld(Y),
                       _ptr(topk_idx), _ptr(topk_w), ws.data_ptr(), ws.numel(),
                       _stream(X.device)), "moe_ffn")
    return Y
