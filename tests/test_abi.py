"""Host-side checks of the C ABI: the library loads, exports every function
include/hsmla.h declares, and rejects bad arguments with the documented
status before any HIP call.

The argument-error cases pass placeholder device addresses; they run only
where no GPU is visible, so a validation bug can never turn into a launch
on real memory.
"""

import ctypes
import os
import re

import pytest

from efficient_vision_attention_amd import hsmla as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(hsmla_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    lib = H.library()
    declared = _declared_functions()
    assert declared == set(H.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(0, -9, -1):
        assert H.status_string(code)
    assert H.status_string(-99) == "unknown status"


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


cpu_only = pytest.mark.skipif(not _no_gpu(), reason="argument-error cases run on hosts without a GPU")

FAKE = 0x10000  # 16-byte aligned placeholder address, never dereferenced


def _desc(**kw):
    base = dict(batch=2, grid_h=16, grid_w=32, channels=64, heads=2,
                branches=(3, 5), block=4, window=8, keep_blocks=4, dtype="bf16")
    base.update(kw)
    return H.make_desc(**base)


def _ws_bytes(desc, op):
    n = ctypes.c_size_t(0)
    st = H.library().hsmla_workspace_bytes(ctypes.byref(desc), op, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("change,status", [
    (dict(head_dim=16, channels=32), -2),
    (dict(channels=96), -2),              # heads * head_dim != channels
    (dict(grid_w=30), -2),                # not a multiple of the block
    (dict(window=9), -2),                 # (window - block) odd
    (dict(window=2), -2),                 # window smaller than block
    (dict(keep_blocks=33), -2),           # keep > T = 32
    (dict(keep_blocks=-1), -2),
    (dict(block=32, grid_h=32, window=32), -2),  # block > 16
    (dict(branches=(4,)), -2),            # even kernel size
    (dict(branches=(9,)), -2),            # kernel > 7
    (dict(dtype=7), -3),
    (dict(batch=0), -2),
    # maximum sizes: just past each limit of the header
    (dict(channels=2080, heads=65), -2),                      # channels > 2048
    (dict(grid_h=368, grid_w=368, window=8), -2),             # 92 x 92 blocks > 8192
    (dict(batch=1024, grid_h=1024, grid_w=2048, block=16,     # 2^31 tokens in one call
          window=16, keep_blocks=4), -2),
])
def test_desc_validation(change, status):
    d = _desc(**{k: v for k, v in change.items() if k != "head_dim"})
    if "head_dim" in change:
        d.head_dim = change["head_dim"]
    st, _ = _ws_bytes(d, H.HSMLA_OP_FORWARD)
    assert st == status


@pytest.mark.parametrize("change", [
    dict(channels=2048, heads=64),                            # channels at the limit
    dict(grid_h=512, grid_w=256, window=8),                   # 128 x 64 = 8192 blocks
    dict(batch=511, grid_h=1024, grid_w=2048, block=16,       # just under 2^30 tokens
         window=16, keep_blocks=4),
])
def test_desc_at_the_limits(change):
    """Descriptors exactly at the header's size limits are accepted (the
    workspace size is formed without overflow)."""
    st, n = _ws_bytes(_desc(**change), H.HSMLA_OP_BLOCK)
    assert st == 0 and n > 0


def test_routing_validation():
    d = _desc()
    d.routing = 4
    assert _ws_bytes(d, H.HSMLA_OP_FORWARD)[0] == -7
    # the soft mixture does not look at tau
    d = _desc(soft=True)
    d.tau = float("nan")
    assert _ws_bytes(d, H.HSMLA_OP_FORWARD)[0] == 0
    assert _ws_bytes(_desc(tau=float("nan"), per_head=True), H.HSMLA_OP_FORWARD)[0] == -7
    assert _ws_bytes(_desc(tau=float("nan")), H.HSMLA_OP_FORWARD)[0] == -7
    # tau is not looked at under top-k routing
    d = _desc()
    d.tau = float("nan")
    assert _ws_bytes(d, H.HSMLA_OP_FORWARD)[0] == 0
    # threshold: sel rows are T wide and the counts follow them
    st_k, n_k = _ws_bytes(_desc(keep_blocks=4), H.HSMLA_OP_FORWARD)
    st_t, n_t = _ws_bytes(_desc(tau=0.5), H.HSMLA_OP_FORWARD)
    assert st_k == 0 and st_t == 0 and n_t > n_k


def test_workspace_bytes_and_bad_op():
    d = _desc()
    st, n = _ws_bytes(d, H.HSMLA_OP_FORWARD)
    assert st == 0 and n > 0
    st_b, nb = _ws_bytes(d, H.HSMLA_OP_BLOCK)
    assert st_b == 0 and nb > n
    assert _ws_bytes(d, 9)[0] == -7
    lib = H.library()
    assert lib.hsmla_workspace_bytes(None, 2, ctypes.byref(ctypes.c_size_t())) == -1
    assert lib.hsmla_workspace_bytes(ctypes.byref(d), 2, None) == -1


def _weights():
    w = H.hsmla_weights()
    w.w_qkv = w.w_o = FAKE
    w.dw[0] = w.dw[1] = FAKE
    w.gate_w = w.gate_b = FAKE
    return w


@cpu_only
def test_forward_argument_errors():
    lib = H.library()
    d = _desc()
    st, need = _ws_bytes(d, H.HSMLA_OP_FORWARD)
    w = _weights()
    f = lib.hsmla_forward
    assert f(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, FAKE, need - 1, None) == -5
    assert f(ctypes.byref(d), ctypes.byref(w), None, FAKE, FAKE, need, None) == -1
    assert f(ctypes.byref(d), ctypes.byref(w), FAKE + 2, FAKE, FAKE, need, None) == -4
    assert f(ctypes.byref(d), None, FAKE, FAKE, FAKE, need, None) == -1
    w.gate_dw = FAKE + 8
    assert f(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, FAKE, need, None) == -4
    w.gate_dw = None
    w.dw[1] = None
    assert f(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, FAKE, need, None) == -1
    bad = _desc(window=7)
    assert f(ctypes.byref(bad), ctypes.byref(_weights()), FAKE, FAKE, FAKE, need, None) == -2


@cpu_only
def test_stage_argument_errors():
    lib = H.library()
    d = _desc()
    st, need = _ws_bytes(d, H.HSMLA_OP_LINEAR)
    assert lib.hsmla_linear_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE,
                                 need - 1, None) == -5
    assert lib.hsmla_linear_attn(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE,
                                 need, None) == -1
    assert lib.hsmla_linear_attn(ctypes.byref(d), FAKE, FAKE, FAKE + 2, FAKE, FAKE,
                                 need, None) == -4
    # gate: pooled scores need qkv_hat, weights and scores_out
    assert lib.hsmla_gate_select(ctypes.byref(d), None, FAKE, FAKE, None, None, FAKE,
                                 FAKE, None) == -1
    assert lib.hsmla_gate_select(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, None,
                                 FAKE, None) == -1
    assert lib.hsmla_gate_select(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE,
                                 None, None) == -1
    assert lib.hsmla_gate_select(ctypes.byref(d), FAKE + 8, FAKE, FAKE, None, None, FAKE,
                                 FAKE, None) == -4
    # the gate's depthwise kernel must be 16-byte aligned
    assert lib.hsmla_gate_select(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE + 8, None,
                                 FAKE, FAKE, None) == -4
    assert lib.hsmla_sparse_softmax(ctypes.byref(d), FAKE, FAKE, None, FAKE, None) == -1
    assert lib.hsmla_sparse_softmax(ctypes.byref(d), FAKE, FAKE + 4, FAKE, FAKE,
                                    None) == -4
    st, need_q = _ws_bytes(d, H.HSMLA_OP_QKV)
    assert lib.hsmla_qkv_branches(ctypes.byref(d), ctypes.byref(_weights()), FAKE,
                                  FAKE, FAKE, FAKE, need_q - 1, None) == -5
    # routing must match the entry point
    dt = _desc(tau=0.5)
    assert lib.hsmla_gate_select(ctypes.byref(dt), FAKE, FAKE, FAKE, None, None, FAKE,
                                 FAKE, None) == -7
    assert lib.hsmla_sparse_softmax(ctypes.byref(dt), FAKE, FAKE, FAKE, FAKE,
                                    None) == -7
    assert lib.hsmla_gate_threshold(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE,
                                    FAKE, FAKE, None) == -7
    assert lib.hsmla_sparse_softmax_counted(ctypes.byref(d), FAKE, FAKE, FAKE,
                                            FAKE, FAKE, None) == -7
    ds = _desc(soft=True)
    assert lib.hsmla_sparse_softmax_weighted(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE,
                                             None) == -7
    assert lib.hsmla_sparse_softmax_weighted(ctypes.byref(ds), FAKE, FAKE, None, FAKE,
                                             None) == -1
    assert lib.hsmla_sparse_softmax_weighted(ctypes.byref(ds), FAKE, FAKE, FAKE + 2,
                                             FAKE, None) == -4
    assert lib.hsmla_sparse_softmax(ctypes.byref(ds), FAKE, FAKE, FAKE, FAKE, None) == -7
    assert lib.hsmla_gate_select(ctypes.byref(ds), FAKE, FAKE, FAKE, None, None, FAKE,
                                 FAKE, None) == -7
    dh = _desc(tau=0.5, per_head=True)
    assert lib.hsmla_gate_threshold(ctypes.byref(dh), FAKE, FAKE, FAKE, None, None,
                                    FAKE, FAKE, FAKE, None) == -7
    assert lib.hsmla_gate_head_threshold(ctypes.byref(dt), FAKE, FAKE, FAKE, None,
                                         None, FAKE, FAKE, FAKE, None) == -7
    assert lib.hsmla_gate_head_threshold(ctypes.byref(dh), FAKE, FAKE, FAKE, None,
                                         None, None, FAKE, FAKE, None) == -1
    assert lib.hsmla_gate_head_threshold(ctypes.byref(dh), FAKE, FAKE, FAKE, None,
                                         None, FAKE, FAKE + 2, FAKE, None) == -4
    assert lib.hsmla_gate_threshold(ctypes.byref(dt), FAKE, FAKE, FAKE, None, None, FAKE,
                                    FAKE, None, None) == -1
    assert lib.hsmla_gate_threshold(ctypes.byref(dt), FAKE, FAKE, FAKE, None, None, FAKE,
                                    FAKE + 2, FAKE, None) == -4
    assert lib.hsmla_sparse_softmax_counted(ctypes.byref(dt), FAKE, FAKE, FAKE,
                                            None, FAKE, None) == -1
    assert lib.hsmla_sparse_softmax_counted(ctypes.byref(dt), FAKE, FAKE, FAKE + 2,
                                            FAKE, FAKE, None) == -4
    ffn = H.hsmla_ffn_weights()
    st, need_b = _ws_bytes(d, H.HSMLA_OP_BLOCK)
    assert lib.hsmla_block_forward(ctypes.byref(d), ctypes.byref(_weights()),
                                   ctypes.byref(ffn), FAKE, FAKE, FAKE, need_b,
                                   None) == -1


@cpu_only
def test_prepare_argument_errors():
    lib = H.library()
    d = _desc()
    st, need = _ws_bytes(d, H.HSMLA_OP_FORWARD)
    w = _weights()
    f = lib.hsmla_prepare
    assert f(ctypes.byref(d), H.HSMLA_OP_LINEAR, ctypes.byref(w), None, FAKE, need,
             None) == -7
    assert f(ctypes.byref(d), 9, ctypes.byref(w), None, FAKE, need, None) == -7
    assert f(ctypes.byref(d), H.HSMLA_OP_FORWARD, ctypes.byref(w), None, FAKE,
             need - 1, None) == -5
    assert f(ctypes.byref(d), H.HSMLA_OP_FORWARD, ctypes.byref(w), None, None,
             need, None) == -1
    assert f(ctypes.byref(d), H.HSMLA_OP_FORWARD, ctypes.byref(w), None, FAKE + 4,
             need, None) == -4
    assert f(ctypes.byref(d), H.HSMLA_OP_FORWARD, None, None, FAKE, need, None) == -1
    st, need_b = _ws_bytes(d, H.HSMLA_OP_BLOCK)
    # the block needs the FFN weights
    assert f(ctypes.byref(d), H.HSMLA_OP_BLOCK, ctypes.byref(w), None, FAKE, need_b,
             None) == -1
    ffn = H.hsmla_ffn_weights()
    ffn.w1 = ffn.w2 = ffn.dw_ffn = FAKE
    assert f(ctypes.byref(d), H.HSMLA_OP_BLOCK, ctypes.byref(w), ctypes.byref(ffn),
             FAKE, need, None) == -5
    ffn.w2 = FAKE + 8
    assert f(ctypes.byref(d), H.HSMLA_OP_BLOCK, ctypes.byref(w), ctypes.byref(ffn),
             FAKE, need_b, None) == -4


def test_workspace_views_layout():
    d = _desc()
    st, need = _ws_bytes(d, H.HSMLA_OP_FORWARD)
    v = H.hsmla_views()
    base = 1 << 20
    assert H.library().hsmla_workspace_views(ctypes.byref(d), H.HSMLA_OP_FORWARD,
                                             base, ctypes.byref(v)) == 0
    offs = [getattr(v, n) - base for n in ("qkv", "qkv_hat", "o", "kv", "ksum",
                                           "scores", "sel")]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and offs[-1] < need
    assert v.x1 is None and v.counts is None
    dt = _desc(tau=0.5)
    st, need_t = _ws_bytes(dt, H.HSMLA_OP_FORWARD)
    assert H.library().hsmla_workspace_views(ctypes.byref(dt), H.HSMLA_OP_FORWARD,
                                             base, ctypes.byref(v)) == 0
    T = (16 // 4) * (32 // 4)
    assert v.counts - v.sel >= 2 * T * 4 and (v.counts - base) % 256 == 0
    assert v.counts - base < need_t and v.head_scores is None
    # per head: sel [B][H][T], counts [B][H], head scores [B][T][H]
    dh = _desc(tau=0.5, per_head=True)
    st, need_h = _ws_bytes(dh, H.HSMLA_OP_FORWARD)
    assert H.library().hsmla_workspace_views(ctypes.byref(dh), H.HSMLA_OP_FORWARD,
                                             base, ctypes.byref(v)) == 0
    assert v.counts - v.sel >= 2 * 2 * T * 4
    assert v.head_scores - v.counts >= 2 * 2 * 4
    assert v.head_scores + 2 * T * 2 * 4 - base <= need_h
