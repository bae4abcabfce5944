"""The two-stream block (hsmla_block_forward_split) against the one-stream
block: the output and every workspace view must be equal bit for bit, for
each routing, odd batches (ranges of unequal size), ragged shapes, one-image
batches and float32 (which runs on one stream)."""

import numpy as np
import pytest
import torch

from efficient_vision_attention_amd import hsmla as H
from efficient_vision_attention_amd.device import DeviceModel, to_device
from workloads import WORKLOADS, make_inputs, scaled

from gpu_harness import announce, shape_of, tau_between

pytestmark = pytest.mark.gpu

_B = WORKLOADS["block"]
SPLIT_CASES = {
    "block_b2": (scaled(_B, batch=2, grid_h=32, grid_w=64), {}),
    "block_b3_ragged": (scaled(_B, name="block_ragged", batch=3, grid_h=20,
                               grid_w=36, channels=96, heads=3, block=4,
                               window=10, keep=0.3), {}),
    "block_b1": (scaled(_B, batch=1, grid_h=16, grid_w=32), {}),
    "block_b4_keep0": (scaled(_B, batch=4, grid_h=16, grid_w=32, keep=0.0), {}),
    "block_b3_threshold": (scaled(_B, batch=3, grid_h=24, grid_w=40),
                           {"tau_q": 0.8}),
    "block_b3_per_head": (scaled(_B, batch=3, grid_h=24, grid_w=40),
                          {"tau_q": 0.7, "per_head": True}),
    "block_b2_soft": (scaled(_B, batch=2, grid_h=24, grid_w=40), {"soft": True}),
    "block_b2_exact_gate": (scaled(_B, batch=2, grid_h=24, grid_w=40,
                                   branches=(3, 5, 7), gate_conv=True), {}),
    # 160 blocks per image: the gate's top-k runs inside the K/V-state
    # launches of each image range
    "block_b3_ranked": (scaled(_B, name="block_ranked", batch=3, grid_h=40,
                               grid_w=64, channels=96, heads=3, block=4,
                               window=10, keep=0.15), {}),
    "block_f32": (scaled(_B, name="block_f32", batch=2, grid_h=12, grid_w=28,
                         channels=96, heads=3, dtype="f32", block=4, window=10,
                         keep=0.4), {}),
}


def _tau(wl, inp, q, per_head):
    # a threshold between two (head) scores of a one-stream run
    m = DeviceModel(shape_of(wl, tau=0.5 if per_head else None,
                             per_head=per_head), inp)
    ws = m.workspace(H.HSMLA_OP_BLOCK)
    out = m.act()
    x = to_device(inp["x"], wl.dtype)
    H.hsmla_block_forward(m.desc, m.weights, m.ffn, x, out, ws)
    torch.cuda.synchronize()
    v = m.views(H.HSMLA_OP_BLOCK, ws)
    return tau_between(v["head_scores" if per_head else "scores"].cpu().numpy(), q)


def _same(a, b, what):
    assert a.dtype == b.dtype and a.shape == b.shape, what
    ai = a.contiguous().view(torch.uint8)
    bi = b.contiguous().view(torch.uint8)
    if not torch.equal(ai, bi):
        n = int((ai != bi).sum())
        raise AssertionError(f"{what}: {n} bytes differ")


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_split_matches_one_stream(name):
    wl, opt = SPLIT_CASES[name]
    inp = make_inputs(wl)
    tau = None
    if "tau_q" in opt:
        announce(f"pilot hsmla_block_forward {name}")
        tau = _tau(wl, inp, opt["tau_q"], opt.get("per_head", False))
    m = DeviceModel(shape_of(wl, tau=tau, per_head=opt.get("per_head", False),
                             soft=opt.get("soft", False)), inp)
    x = to_device(inp["x"], wl.dtype)
    ws1, ws2 = m.workspace(H.HSMLA_OP_BLOCK), m.workspace(H.HSMLA_OP_BLOCK)
    ws1.fill_(0x5A)
    ws2.fill_(0xC3)  # different stale contents: nothing may read them
    out1, out2 = m.act(), m.act()
    out2.fill_(7)
    announce(f"hsmla_block_forward {name} B={wl.batch} {wl.grid_h}x{wl.grid_w}")
    H.hsmla_block_forward(m.desc, m.weights, m.ffn, x, out1, ws1)
    torch.cuda.synchronize()
    split = H.SplitStreams()
    announce(f"hsmla_block_forward_split {name}")
    H.hsmla_block_forward_split(m.desc, m.weights, m.ffn, x, out2, ws2, split)
    # no device-wide sync: the join must order this copy after both halves
    seen = out2.clone()
    torch.cuda.synchronize()
    _same(out1, seen, "out (read on the calling stream after the join)")
    _same(out1, out2, "out")
    v1 = m.views(H.HSMLA_OP_BLOCK, ws1)
    v2 = m.views(H.HSMLA_OP_BLOCK, ws2)
    for key in ("qkv", "qkv_hat", "o", "kv", "ksum", "scores", "x1",
                "head_scores", "counts"):
        if key in v1:
            _same(v1[key], v2[key], key)
    counts = v1.get("counts")
    if counts is None:
        if not opt.get("soft"):
            _same(v1["sel"], v2["sel"], "sel")
    else:
        c = counts.cpu().numpy()
        s1, s2 = v1["sel"].cpu().numpy(), v2["sel"].cpu().numpy()
        for idx in np.ndindex(c.shape):
            n = int(c[idx])
            assert np.array_equal(s1[idx][:n], s2[idx][:n]), f"sel {idx}"


def test_split_rejects_same_stream():
    wl, _ = SPLIT_CASES["block_b2"]
    inp = make_inputs(wl)
    m = DeviceModel(shape_of(wl), inp)
    x = to_device(inp["x"], wl.dtype)
    ws, out = m.workspace(H.HSMLA_OP_BLOCK), m.act()
    split = H.SplitStreams()
    split.aux = torch.cuda.current_stream()
    announce("hsmla_block_forward_split with aux == stream (host-side error)")
    with pytest.raises(H.HsmlaError) as e:
        H.hsmla_block_forward_split(m.desc, m.weights, m.ffn, x, out, ws, split)
    assert e.value.status == H.HSMLA_ERR_ARG
