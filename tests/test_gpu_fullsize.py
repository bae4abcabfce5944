"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (hsmla_forward / hsmla_block_forward over the whole batch).

The oracle cannot afford every output at these sizes, so each stage is
checked on the GPU's own inputs to that stage (stage-wise): Z, D and the gate
scores over everything, the selection exactly, and sampled tokens / blocks
for the projections, the depthwise branches, the linear readout, the
refinement and the FFN.  Tolerances as in the other parity tests.
"""

import numpy as np
import pytest

import oracle as O
from workloads import WORKLOADS, make_inputs, scaled

from gpu_harness import (Run, assert_close, routed_lists, selection_band_check,
                         threshold_band_check)

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(1234)


def _rows(n, count):
    return np.sort(RNG.choice(n, size=min(n, count), replace=False))


def _border_tokens(gh, gw, count):
    """The four corners plus tokens drawn from the two outermost rows and
    columns on each side (the 5x5 and 7x7 branches' zero padding reaches
    three tokens in)."""
    toks = {0, gw - 1, (gh - 1) * gw, gh * gw - 1}
    for _ in range(count):
        side = RNG.integers(4)
        depth = int(RNG.integers(3))
        if side < 2:  # top or bottom rows
            y = depth if side == 0 else gh - 1 - depth
            x = int(RNG.integers(gw))
        else:
            x = depth if side == 2 else gw - 1 - depth
            y = int(RNG.integers(gh))
        toks.add(y * gw + x)
    return np.array(sorted(toks))


def _sampled_branches(qkv, kernels, gh, gw, b, tokens):
    """qkv + sum of depthwise branches at the given tokens of image b, from
    zero-padded crops around each token (same result as the full grid)."""
    kmax = max([k.shape[-1] for k in kernels] + [1])
    r = (kmax - 1) // 2
    side = 2 * r + 1
    img = qkv[b].reshape(gh, gw, -1)
    crops = np.zeros((len(tokens), side, side, img.shape[-1]))
    for i, n in enumerate(tokens):
        y, x = divmod(int(n), gw)
        y0, y1 = max(0, y - r), min(gh, y + r + 1)
        x0, x1 = max(0, x - r), min(gw, x + r + 1)
        crops[i, y0 - (y - r):y1 - (y - r), x0 - (x - r):x1 - (x - r)] = img[y0:y1, x0:x1]
    out = O.multiscale_branches(crops.reshape(len(tokens), side * side, -1),
                                kernels, side, side)
    return out[:, r * side + r]


def _check_module_fullsize(wl, inp, g, tau=None):
    B, N, C = wl.batch, wl.tokens, wl.channels
    rnd = O.round_bf16
    x = inp["x"]
    # S1 on sampled rows
    for b in range(B):
        rows = _rows(N, 256)
        assert_close(g["qkv"][b, rows], rnd(x[b, rows] @ inp["w_qkv"]), "bf16",
                     f"qkv image {b}")
    # S2 on sampled tokens (GPU qkv in)
    for b in range(B):
        toks = np.union1d(_rows(N, 96), _border_tokens(wl.grid_h, wl.grid_w, 64))
        ref = rnd(_sampled_branches(g["qkv"], inp["dw"], wl.grid_h, wl.grid_w, b, toks))
        assert_close(g["qkv_hat"][b, toks], ref, "bf16", f"qkv_hat image {b}")
    # S3a over everything (GPU qkv_hat in)
    Z, D = O.kv_state(g["qkv_hat"][..., C:2 * C], g["qkv_hat"][..., 2 * C:],
                      wl.heads)
    np.testing.assert_allclose(g["kv"], Z, rtol=1e-4, atol=1e-5 * np.abs(Z).max())
    np.testing.assert_allclose(g["ksum"], D, rtol=1e-5, atol=1e-5)
    # S4 over everything
    scores = O.gate_scores(g["qkv_hat"], inp["gate_w"], inp["gate_b"], wl.grid_h,
                           wl.grid_w, wl.block, wl.heads, gate_dw=inp.get("gate_dw"))
    np.testing.assert_allclose(g["scores"], scores, rtol=0, atol=2e-6)
    if tau is None:
        k = wl.keep_blocks
        sel_g = g["sel"][:, :k]
        np.testing.assert_array_equal(
            sel_g, O.select_blocks(g["scores"].astype(np.float32), k))
        sel_ref = O.select_blocks(scores.astype(np.float32), k)
        if not np.array_equal(sel_g, sel_ref):
            selection_band_check(scores, g["scores"], sel_ref, sel_g, k)
        lists = list(sel_g)
    else:
        lists = routed_lists(g["sel"], g["counts"])
        own_sel, own_cnt = O.select_threshold(g["scores"].astype(np.float32),
                                              np.float32(tau))
        np.testing.assert_array_equal(g["counts"], own_cnt)
        for b in range(B):
            np.testing.assert_array_equal(lists[b], own_sel[b, :own_cnt[b]])
        ref_sel, ref_cnt = O.select_threshold(scores.astype(np.float32),
                                              np.float32(tau))
        threshold_band_check(scores, g["scores"], tau,
                             routed_lists(ref_sel, ref_cnt), lists)
    # S3b on sampled unselected tokens
    nbc = wl.grid_w // wl.block
    ys, xs = np.divmod(np.arange(N), wl.grid_w)
    tblk = (ys // wl.block) * nbc + xs // wl.block
    for b in range(B):
        unsel = np.nonzero(~np.isin(tblk, lists[b]))[0]
        toks = np.sort(RNG.choice(unsel, size=min(256, unsel.size), replace=False))
        ref = rnd(O.linear_readout(g["qkv_hat"][b:b + 1, toks, :C], Z[b:b + 1],
                                   D[b:b + 1], wl.heads))[0]
        assert_close(g["o"][b, toks], ref, "bf16", f"o_lin image {b}")
    # S5 on sampled selected blocks (GPU qkv, qkv_hat in; O_lin recomputed)
    for b in range(B):
        if len(lists[b]) == 0:
            continue
        pick = np.sort(RNG.choice(lists[b], size=min(6, len(lists[b])), replace=False))
        toks = np.nonzero(np.isin(tblk, pick))[0]
        o_lin = np.zeros((1, N, C))
        o_lin[0, toks] = rnd(O.linear_readout(g["qkv_hat"][b:b + 1, toks, :C],
                                              Z[b:b + 1], D[b:b + 1], wl.heads))[0]
        ref = O.refine_selected(g["qkv"][b:b + 1], g["qkv_hat"][b:b + 1], o_lin,
                                pick[None], wl.grid_h, wl.grid_w, wl.heads,
                                wl.block, wl.window, rnd=rnd)
        assert_close(g["o"][b, toks], ref[0, toks], "bf16", f"o refined image {b}")
    return tblk


@pytest.mark.parametrize("name", ["street", "ct", "pathology"])
def test_forward_full_size(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    g = Run(wl, inp).forward()
    _check_module_fullsize(wl, inp, g)
    for b in range(wl.batch):
        rows = _rows(wl.tokens, 256)
        assert_close(g["y"][b, rows], O.round_bf16(g["o"][b, rows] @ inp["w_o"]),
                     "bf16", f"y image {b}")


@pytest.mark.parametrize("keep", [0.0, 0.05, 0.10, 0.25, 0.50])
def test_block_forward_full_size(keep):
    wl = scaled(WORKLOADS["block"], keep=keep)
    inp = make_inputs(wl)
    g = Run(wl, inp).block_forward()
    rnd = O.round_bf16
    C, N = wl.channels, wl.tokens
    # the module runs on LN1(x): check LN1 on sampled rows through qkv
    xn1 = rnd(O.layer_norm(inp["x"], inp["ln1_g"], inp["ln1_b"]))
    inp_mod = dict(inp, x=xn1)
    _check_module_fullsize(wl, inp_mod, g)
    for b in range(wl.batch):
        rows = _rows(N, 256)
        ref = rnd(inp["x"][b, rows] + g["o"][b, rows] @ inp["w_o"])
        assert_close(g["x1"][b, rows], ref, "bf16", f"x1 image {b}")
        # FFN at sampled tokens from the GPU's x1 (3x3 neighbourhood)
        toks = _rows(N, 48)
        x1 = g["x1"][b].reshape(wl.grid_h, wl.grid_w, C)
        outs = []
        for n in toks:
            y, x = divmod(int(n), wl.grid_w)
            crop = np.zeros((3, 3, C))
            y0, y1 = max(0, y - 1), min(wl.grid_h, y + 2)
            x0, x1c = max(0, x - 1), min(wl.grid_w, x + 2)
            crop[y0 - (y - 1):y1 - (y - 1), x0 - (x - 1):x1c - (x - 1)] = x1[y0:y1, x0:x1c]
            valid = np.zeros((3, 3, 1))
            valid[y0 - (y - 1):y1 - (y - 1), x0 - (x - 1):x1c - (x - 1)] = 1.0
            xn2 = rnd(O.layer_norm(crop.reshape(9, C), inp["ln2_g"], inp["ln2_b"]))
            h1 = rnd(xn2 @ inp["w1"]) * valid.reshape(9, 1)  # zero padding
            h2 = rnd(O.gelu(O.dwconv_same(h1[None], inp["dw_ffn"], 3, 3)))[0, 4]
            outs.append(rnd(x1[y, x] + h2 @ inp["w2"]))
        assert_close(g["out"][b, toks], np.array(outs), "bf16", f"out image {b}")


def test_block_forward_full_size_exact_gate_three_branches():
    """The benchmark's block workload with the gate's depthwise 3x3 and the
    identity + 3x3 + 5x5 + 7x7 branches, stage-wise as above."""
    wl = scaled(WORKLOADS["block"], branches=(3, 5, 7), gate_conv=True)
    inp = make_inputs(wl)
    g = Run(wl, inp).block_forward()
    xn1 = O.round_bf16(O.layer_norm(inp["x"], inp["ln1_g"], inp["ln1_b"]))
    _check_module_fullsize(wl, dict(inp, x=xn1), g)


def test_block_forward_full_size_every_element():
    """The benchmark's block workload (keep 10%), each projection and the FFN
    checked on every element, stage-wise on the GPU's own inputs (FT 3.5
    block equation): qkv = LN1(x) W_qkv on every row (every output tile of
    the projection), x1 = x + O W_o on every row, and out = x1 +
    FFN(LN2(x1)) on every token from the GPU's x1."""
    wl = scaled(WORKLOADS["block"], keep=0.10)
    inp = make_inputs(wl)
    g = Run(wl, inp).block_forward()
    rnd = O.round_bf16
    B, C = wl.batch, wl.channels
    xn1 = rnd(O.layer_norm(inp["x"], inp["ln1_g"], inp["ln1_b"]))
    assert_close(g["qkv"], rnd(xn1 @ inp["w_qkv"]), "bf16", "qkv, every row")
    assert_close(g["x1"], rnd(inp["x"] + g["o"] @ inp["w_o"]), "bf16", "x1, every row")
    for b in range(B):  # one image at a time keeps the host arrays small
        x1 = g["x1"][b:b + 1]
        xn2 = rnd(O.layer_norm(x1, inp["ln2_g"], inp["ln2_b"]))
        h1 = rnd(xn2 @ inp["w1"])
        h2 = rnd(O.gelu(O.dwconv_same(h1, inp["dw_ffn"], wl.grid_h, wl.grid_w)))
        del h1
        assert_close(g["out"][b:b + 1], rnd(x1 + h2 @ inp["w2"]), "bf16",
                     f"out image {b}, every token")


def test_block_forward_full_size_every_element_attention():
    """The same block workload, the attention stages on every element,
    stage-wise on the GPU's own inputs (FT 3.1 and 3.3): Q^K^V^ = the
    depthwise branches of the GPU's qkv on every token of both images, and
    O = the linear readout of the GPU's Q^K^V^ with the GPU-selected blocks
    refined (two-path residual over the window) on every token."""
    wl = scaled(WORKLOADS["block"], keep=0.10)
    inp = make_inputs(wl)
    g = Run(wl, inp).block_forward()
    rnd = O.round_bf16
    C = wl.channels
    for b in range(wl.batch):
        ref = rnd(O.multiscale_branches(g["qkv"][b:b + 1], inp["dw"], wl.grid_h, wl.grid_w))
        assert_close(g["qkv_hat"][b:b + 1], ref, "bf16", f"qkv_hat image {b}, every token")
        del ref
    Z, D = O.kv_state(g["qkv_hat"][..., C:2 * C], g["qkv_hat"][..., 2 * C:], wl.heads)
    o_lin = rnd(O.linear_readout(g["qkv_hat"][..., :C], Z, D, wl.heads))
    sel = g["sel"][:, :wl.keep_blocks]
    np.testing.assert_array_equal(sel, O.select_blocks(g["scores"].astype(np.float32),
                                                       wl.keep_blocks))
    ref_o = O.refine_selected(g["qkv"], g["qkv_hat"], o_lin, sel, wl.grid_h, wl.grid_w,
                              wl.heads, wl.block, wl.window, rnd=rnd)
    assert_close(g["o"], ref_o, "bf16", "o, every token")
