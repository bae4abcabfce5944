"""ctypes binding of libhsmla.so (include/hsmla.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and the current HIP stream to
the C entry point of the same name, and raises HsmlaError on a non-zero
status.  No computation happens here, and there is no fallback: if the
library is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhsmla.so")

HSMLA_F32, HSMLA_BF16 = 0, 1
HSMLA_OP_QKV, HSMLA_OP_LINEAR, HSMLA_OP_FORWARD, HSMLA_OP_BLOCK = 0, 1, 2, 3
(HSMLA_OK, HSMLA_ERR_NULL, HSMLA_ERR_SHAPE, HSMLA_ERR_DTYPE, HSMLA_ERR_ALIGN,
 HSMLA_ERR_WORKSPACE, HSMLA_ERR_HIP, HSMLA_ERR_ARG,
 HSMLA_ERR_SCRATCH) = 0, -1, -2, -3, -4, -5, -6, -7, -8
HSMLA_ROUTE_TOPK, HSMLA_ROUTE_THRESHOLD, HSMLA_ROUTE_HEAD_THRESHOLD, HSMLA_ROUTE_SOFT = 0, 1, 2, 3

# Every symbol include/hsmla.h declares.
EXPORTED = (
    "hsmla_workspace_bytes",
    "hsmla_workspace_views",
    "hsmla_prepare",
    "hsmla_qkv_branches",
    "hsmla_linear_attn",
    "hsmla_linear_attn_noalloc",
    "hsmla_gate_select",
    "hsmla_gate_threshold",
    "hsmla_gate_head_threshold",
    "hsmla_sparse_softmax",
    "hsmla_sparse_softmax_counted",
    "hsmla_sparse_softmax_weighted",
    "hsmla_forward",
    "hsmla_block_forward",
    "hsmla_block_forward_split",
    "hsmla_forward_timed",
    "hsmla_block_forward_timed",
    "hsmla_status_string",
)


class HsmlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class hsmla_desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32), ("channels", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_branches", ctypes.c_int32), ("branch_k", ctypes.c_int32 * 3),
        ("block", ctypes.c_int32), ("window", ctypes.c_int32),
        ("keep_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("routing", ctypes.c_int32), ("tau", ctypes.c_float),
        ("prepared", ctypes.c_int32),
    ]


class hsmla_weights(ctypes.Structure):
    _fields_ = [
        ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
        ("dw", ctypes.c_void_p * 3), ("gate_w", ctypes.c_void_p),
        ("gate_b", ctypes.c_void_p), ("gate_dw", ctypes.c_void_p),
    ]


class hsmla_ffn_weights(ctypes.Structure):
    _fields_ = [
        ("ln1_g", ctypes.c_void_p), ("ln1_b", ctypes.c_void_p),
        ("ln2_g", ctypes.c_void_p), ("ln2_b", ctypes.c_void_p),
        ("w1", ctypes.c_void_p), ("dw_ffn", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
    ]


class hsmla_views(ctypes.Structure):
    _fields_ = [
        ("qkv", ctypes.c_void_p), ("qkv_hat", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("kv", ctypes.c_void_p),
        ("ksum", ctypes.c_void_p), ("scores", ctypes.c_void_p),
        ("sel", ctypes.c_void_p), ("counts", ctypes.c_void_p),
        ("head_scores", ctypes.c_void_p), ("x1", ctypes.c_void_p),
    ]


_lib = None


def library():
    """Load libhsmla.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m efficient_vision_attention_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, VP, I32, SZ = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lib.hsmla_status_string.restype = ctypes.c_char_p
        lib.hsmla_status_string.argtypes = [I32]
        sigs = {
            "hsmla_workspace_bytes": [P(hsmla_desc), I32, P(SZ)],
            "hsmla_workspace_views": [P(hsmla_desc), I32, VP, P(hsmla_views)],
            "hsmla_prepare": [P(hsmla_desc), I32, P(hsmla_weights), P(hsmla_ffn_weights),
                              VP, SZ, VP],
            "hsmla_qkv_branches": [P(hsmla_desc), P(hsmla_weights), VP, VP, VP, VP, SZ, VP],
            "hsmla_linear_attn": [P(hsmla_desc), VP, VP, VP, VP, VP, SZ, VP],
            "hsmla_linear_attn_noalloc": [P(hsmla_desc), VP, VP, VP, VP, VP],
            "hsmla_gate_select": [P(hsmla_desc), VP, VP, VP, VP, VP, VP, VP, VP],
            "hsmla_gate_threshold": [P(hsmla_desc), VP, VP, VP, VP, VP, VP, VP, VP, VP],
            "hsmla_gate_head_threshold": [P(hsmla_desc), VP, VP, VP, VP, VP, VP, VP, VP, VP],
            "hsmla_sparse_softmax": [P(hsmla_desc), VP, VP, VP, VP, VP],
            "hsmla_sparse_softmax_counted": [P(hsmla_desc), VP, VP, VP, VP, VP, VP],
            "hsmla_sparse_softmax_weighted": [P(hsmla_desc), VP, VP, VP, VP, VP],
            "hsmla_forward": [P(hsmla_desc), P(hsmla_weights), VP, VP, VP, SZ, VP],
            "hsmla_block_forward": [P(hsmla_desc), P(hsmla_weights), P(hsmla_ffn_weights),
                                    VP, VP, VP, SZ, VP],
            "hsmla_block_forward_split": [P(hsmla_desc), P(hsmla_weights),
                                          P(hsmla_ffn_weights), VP, VP, VP, SZ, VP,
                                          VP, VP, VP],
            "hsmla_forward_timed": [P(hsmla_desc), P(hsmla_weights), VP, VP, VP, SZ, VP,
                                    P(VP), P(ctypes.c_char_p), I32, P(I32)],
            "hsmla_block_forward_timed": [P(hsmla_desc), P(hsmla_weights),
                                          P(hsmla_ffn_weights), VP, VP, VP, SZ, VP,
                                          P(VP), P(ctypes.c_char_p), I32, P(I32)],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int32
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().hsmla_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise HsmlaError(status, where)


def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def make_desc(*, batch, grid_h, grid_w, channels, heads, branches, block,
              window, keep_blocks, dtype, head_dim=32, tau=None, per_head=False,
              soft=False, prepared=False):
    """tau=None: top-k routing (keep_blocks per image); a number: threshold
    routing (every block with score > tau), per head when per_head; soft:
    the training-time mixture (every block, residual scaled by its score);
    prepared: the workspace holds what hsmla_prepare wrote."""
    d = hsmla_desc()
    d.batch, d.grid_h, d.grid_w = batch, grid_h, grid_w
    d.channels, d.heads, d.head_dim = channels, heads, head_dim
    d.n_branches = len(branches)
    for i, k in enumerate(branches):
        d.branch_k[i] = k
    d.block, d.window, d.keep_blocks = block, window, keep_blocks
    d.dtype = {"f32": HSMLA_F32, "bf16": HSMLA_BF16}.get(dtype, dtype)
    d.routing = (HSMLA_ROUTE_SOFT if soft else HSMLA_ROUTE_TOPK if tau is None else
                 HSMLA_ROUTE_HEAD_THRESHOLD if per_head else HSMLA_ROUTE_THRESHOLD)
    d.tau = 0.0 if tau is None else float(tau)
    d.prepared = 1 if prepared else 0
    return d


def make_weights(w_qkv, w_o, dw, gate_w, gate_b, gate_dw=None):
    w = hsmla_weights()
    w.w_qkv, w.w_o = _ptr(w_qkv), _ptr(w_o)
    for i, t in enumerate(dw):
        w.dw[i] = _ptr(t)
    w.gate_w, w.gate_b = _ptr(gate_w), _ptr(gate_b)
    w.gate_dw = _ptr(gate_dw)
    return w


def make_ffn_weights(ln1_g, ln1_b, ln2_g, ln2_b, w1, dw_ffn, w2):
    f = hsmla_ffn_weights()
    f.ln1_g, f.ln1_b, f.ln2_g, f.ln2_b = map(_ptr, (ln1_g, ln1_b, ln2_g, ln2_b))
    f.w1, f.dw_ffn, f.w2 = _ptr(w1), _ptr(dw_ffn), _ptr(w2)
    return f


def hsmla_workspace_bytes(desc, op) -> int:
    n = ctypes.c_size_t(0)
    _check(library().hsmla_workspace_bytes(ctypes.byref(desc), op, ctypes.byref(n)),
           "hsmla_workspace_bytes")
    return n.value


def hsmla_workspace_views(desc, op, ws):
    """Byte offsets of the intermediates inside workspace tensor `ws`."""
    v = hsmla_views()
    _check(library().hsmla_workspace_views(ctypes.byref(desc), op, _ptr(ws),
                                           ctypes.byref(v)),
           "hsmla_workspace_views")
    base = ws.data_ptr()
    return {name: (getattr(v, name) - base) if getattr(v, name) else None
            for name, _ in hsmla_views._fields_}


def hsmla_prepare(desc, op, weights, ffn, ws):
    _check(library().hsmla_prepare(ctypes.byref(desc), op, ctypes.byref(weights),
                                   ctypes.byref(ffn) if ffn is not None else None,
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream()),
           "hsmla_prepare")


def hsmla_qkv_branches(desc, weights, x, qkv, qkv_hat, ws):
    _check(library().hsmla_qkv_branches(ctypes.byref(desc), ctypes.byref(weights),
                                        _ptr(x), _ptr(qkv), _ptr(qkv_hat), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream()),
           "hsmla_qkv_branches")


def hsmla_linear_attn(desc, qkv_hat, o, kv, ksum, ws):
    _check(library().hsmla_linear_attn(ctypes.byref(desc), _ptr(qkv_hat), _ptr(o),
                                       _ptr(kv), _ptr(ksum), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream()),
           "hsmla_linear_attn")


def hsmla_linear_attn_noalloc(desc, qkv_hat, o, kv, ksum):
    _check(library().hsmla_linear_attn_noalloc(ctypes.byref(desc), _ptr(qkv_hat),
                                               _ptr(o), _ptr(kv), _ptr(ksum),
                                               _stream()),
           "hsmla_linear_attn_noalloc")


def hsmla_gate_select(desc, qkv_hat, gate_w, gate_b, scores_in, scores_out, sel,
                      gate_dw=None):
    _check(library().hsmla_gate_select(ctypes.byref(desc), _ptr(qkv_hat),
                                       _ptr(gate_w), _ptr(gate_b), _ptr(gate_dw),
                                       _ptr(scores_in), _ptr(scores_out), _ptr(sel),
                                       _stream()),
           "hsmla_gate_select")


def hsmla_gate_threshold(desc, qkv_hat, gate_w, gate_b, scores_in, scores_out,
                         sel, counts, gate_dw=None):
    _check(library().hsmla_gate_threshold(ctypes.byref(desc), _ptr(qkv_hat),
                                          _ptr(gate_w), _ptr(gate_b), _ptr(gate_dw),
                                          _ptr(scores_in), _ptr(scores_out),
                                          _ptr(sel), _ptr(counts), _stream()),
           "hsmla_gate_threshold")


def hsmla_gate_head_threshold(desc, qkv_hat, gate_w, gate_b, head_scores_in,
                              head_scores_out, sel, counts, gate_dw=None):
    _check(library().hsmla_gate_head_threshold(
        ctypes.byref(desc), _ptr(qkv_hat), _ptr(gate_w), _ptr(gate_b), _ptr(gate_dw),
        _ptr(head_scores_in), _ptr(head_scores_out), _ptr(sel), _ptr(counts),
        _stream()), "hsmla_gate_head_threshold")


def hsmla_sparse_softmax_counted(desc, qkv, qkv_hat, sel, counts, o):
    _check(library().hsmla_sparse_softmax_counted(ctypes.byref(desc), _ptr(qkv),
                                                  _ptr(qkv_hat), _ptr(sel),
                                                  _ptr(counts), _ptr(o), _stream()),
           "hsmla_sparse_softmax_counted")


def hsmla_sparse_softmax(desc, qkv, qkv_hat, sel, o):
    _check(library().hsmla_sparse_softmax(ctypes.byref(desc), _ptr(qkv),
                                          _ptr(qkv_hat), _ptr(sel), _ptr(o),
                                          _stream()),
           "hsmla_sparse_softmax")


def hsmla_sparse_softmax_weighted(desc, qkv, qkv_hat, weights, o):
    _check(library().hsmla_sparse_softmax_weighted(ctypes.byref(desc), _ptr(qkv),
                                                   _ptr(qkv_hat), _ptr(weights),
                                                   _ptr(o), _stream()),
           "hsmla_sparse_softmax_weighted")


def hsmla_forward(desc, weights, x, y, ws):
    _check(library().hsmla_forward(ctypes.byref(desc), ctypes.byref(weights),
                                   _ptr(x), _ptr(y), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream()),
           "hsmla_forward")


def hsmla_block_forward(desc, weights, ffn, x, out, ws):
    _check(library().hsmla_block_forward(ctypes.byref(desc), ctypes.byref(weights),
                                         ctypes.byref(ffn), _ptr(x), _ptr(out),
                                         _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream()),
           "hsmla_block_forward")


class SplitStreams:
    """The second stream and the fork/join events hsmla_block_forward_split
    takes (default stream priority; events without timing)."""

    def __init__(self):
        self.aux = torch.cuda.Stream()
        self.fork = torch.cuda.Event()
        self.join = torch.cuda.Event()
        # torch creates the underlying events on their first record
        self.fork.record()
        self.join.record()


def hsmla_block_forward_split(desc, weights, ffn, x, out, ws, split: SplitStreams):
    _check(library().hsmla_block_forward_split(
        ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(ffn), _ptr(x),
        _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(),
        split.aux.cuda_stream, split.fork.cuda_event, split.join.cuda_event),
        "hsmla_block_forward_split")


def _timed(fn, where, args, events):
    n = len(events)
    ev = (ctypes.c_void_p * n)(*events)
    names = (ctypes.c_char_p * n)()
    count = ctypes.c_int32(0)
    _check(fn(*args, ev, names, n, ctypes.byref(count)), where)
    return [names[i].decode() for i in range(count.value + 1)]


def hsmla_forward_timed(desc, weights, x, y, ws, events):
    """hsmla_forward with an event recorded before every launch and after the
    last; `events` are raw hipEvent_t handles.  Returns the launch names."""
    lib = library()
    return _timed(lib.hsmla_forward_timed, "hsmla_forward_timed",
                  (ctypes.byref(desc), ctypes.byref(weights), _ptr(x), _ptr(y),
                   _ptr(ws), ws.numel() * ws.element_size(), _stream()), events)


def hsmla_block_forward_timed(desc, weights, ffn, x, out, ws, events):
    lib = library()
    return _timed(lib.hsmla_block_forward_timed, "hsmla_block_forward_timed",
                  (ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(ffn),
                   _ptr(x), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                   _stream()), events)
