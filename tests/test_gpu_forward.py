"""End-to-end GPU parity of hsmla_forward and hsmla_block_forward against
the oracle (bfloat16-staged for bf16 runs, exact for float32 runs), plus
the degenerate cases of the method."""

import numpy as np
import pytest
import torch

import oracle as O
from efficient_vision_attention_amd import hsmla as H
from efficient_vision_attention_amd.device import to_host
from workloads import WORKLOADS, make_inputs, scaled

from gpu_harness import (TOL, Run, announce, assert_close, oracle_kwargs,
                         selection_band_check, staged)
from test_gpu_stages import STAGE_CASES

pytestmark = pytest.mark.gpu


def _check_module(wl, inp, g, k=None):
    """Compare every forward intermediate with the oracle; a selection that
    differs inside the near-tie band is injected into the oracle."""
    kw = oracle_kwargs(wl, k)
    st = staged(wl)
    ref = O.hsmla_forward(inp["x"], inp, staged=st, **kw)
    kk = kw["keep_blocks"]
    sel_g = g["sel"][:, :kk]
    if not np.array_equal(sel_g, ref["sel"]):
        rep = selection_band_check(ref["scores"], g["scores"], ref["sel"], sel_g, kk)
        print("selection differs inside the tie band:", rep)
        ref = O.hsmla_forward(inp["x"], inp, staged=st, sel=sel_g, **kw)
    for key in ("qkv", "qkv_hat", "o", "y"):
        assert_close(g[key], ref[key], wl.dtype, key)
    np.testing.assert_allclose(g["scores"], ref["scores"], rtol=0, atol=5e-5)
    return ref


@pytest.mark.parametrize("name", list(STAGE_CASES))
def test_forward_end_to_end(name):
    wl = STAGE_CASES[name]
    inp = make_inputs(wl)
    g = Run(wl, inp).forward()
    _check_module(wl, inp, g)


def test_forward_is_bitwise_deterministic():
    wl = STAGE_CASES["street_small"]
    inp = make_inputs(wl)
    r = Run(wl, inp)
    a, b = r.forward(), r.forward()
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("name", ["tiny", "ragged_bf16"])
def test_keep_zero_is_linear_attention(name):
    wl = STAGE_CASES[name]
    inp = make_inputs(wl)
    g = Run(wl, inp, keep_blocks=0).forward()
    ref = _check_module(wl, inp, g, k=0)
    np.testing.assert_array_equal(ref["o"], ref["o_lin"])


_GATE_PARTS = {
    # 5x5 stream conv (16-lane head slices); C = 96: the last 64-channel
    # tile holds one slice inside the channels and one outside
    "branches35_c96": scaled(WORKLOADS["street"], name="gp35", batch=2, grid_h=40,
                             grid_w=48, channels=96, heads=3, block=4, window=10,
                             keep=0.2),
    # 3x3 only: the LDS-staged conv (8-lane head slices)
    "branches3_c128": scaled(WORKLOADS["street"], name="gp3", batch=1, grid_h=32,
                             grid_w=64, channels=128, heads=4, branches=(3,),
                             block=4, window=12, keep=0.15),
    # the upper end: 1024 blocks per image
    "blocks1024": scaled(WORKLOADS["street"], name="gp1024", batch=1, grid_h=128,
                         grid_w=128, channels=64, heads=2, block=4, window=8,
                         keep=0.05),
    # the exact gate (its 3x3 inside the head score) pools no sums in the
    # conv: scores from the gate kernel, ranked over 8 workgroups per image
    "exact_gate_T192": scaled(WORKLOADS["street"], name="gpx", batch=2, grid_h=48,
                              grid_w=64, channels=96, heads=3, block=4, window=10,
                              keep=0.2, gate_conv=True),
    # the lower end (72 blocks: runs of 16 keys) over three images, whose
    # rank workgroups precede the K/V partial-sum workgroups in one launch
    "blocks72_b3": scaled(WORKLOADS["street"], name="gp72", batch=3, grid_h=24,
                          grid_w=48, channels=64, heads=2, block=4, window=8,
                          keep=0.25),
}


@pytest.mark.parametrize("name", list(_GATE_PARTS))
def test_topk_over_workgroups(name):
    """Top-k routing over 65..1024 blocks per image, ranked over several
    workgroups per image; with the conv's pooled sums reduced into the
    gate's partial logits, or (exact gate) from the gate kernel's scores:
    scores within 5e-5 of the oracle and the selection as the oracle ranks
    the GPU's own scores."""
    wl = _GATE_PARTS[name]
    assert 64 < wl.num_blocks <= 1024
    inp = make_inputs(wl)
    g = Run(wl, inp).forward()
    _check_module(wl, inp, g)
    kk = wl.keep_blocks
    np.testing.assert_array_equal(g["sel"][:, :kk],
                                  O.select_blocks(g["scores"].astype(np.float32), kk))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("grid,block,window", [(4, 4, 8), (8, 8, 16)])
def test_single_block_images(dtype, grid, block, window):
    """Images of a single block (T = 1) with it selected: the gate ranks one
    score, the refinement's window is the whole image, and the forward
    matches the oracle end to end."""
    wl = scaled(WORKLOADS["street"], name=f"one{grid}", batch=2, grid_h=grid, grid_w=grid,
                channels=64, heads=2, block=block, window=window, keep=1.0, dtype=dtype)
    assert wl.num_blocks == 1 and wl.keep_blocks == 1
    inp = make_inputs(wl)
    announce(f"hsmla_forward single-block images {dtype} {grid}x{grid}")
    g = Run(wl, inp).forward()
    _check_module(wl, inp, g)
    assert np.array_equal(g["sel"][:, :1], np.zeros((2, 1), np.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_keep_all_covering_window_is_full_softmax(dtype):
    """Every block refined with a window covering the grid: the linear terms
    cancel and the module output is softmax attention over raw Q, K, V."""
    wl = scaled(WORKLOADS["tiny"], dtype=dtype, window=4 + 2 * 16, keep=1.0)
    inp = make_inputs(wl)
    g = Run(wl, inp).forward()
    ref = _check_module(wl, inp, g)
    qkv = torch.from_numpy(g["qkv"])
    B, N, C3 = qkv.shape
    C = C3 // 3
    q, k, v = (qkv[..., s * C:(s + 1) * C].reshape(B, N, 2, 32).transpose(1, 2)
               for s in range(3))
    full = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    full = full.transpose(1, 2).reshape(B, N, C).numpy()
    tol = 5e-2 if dtype == "bf16" else 1e-4
    np.testing.assert_allclose(g["o"], full, rtol=tol, atol=tol)
    assert ref["sel"].shape[1] == wl.num_blocks


def test_window_equal_block_keep_all():
    wl = scaled(STAGE_CASES["ragged_bf16"], window=4, keep=1.0)
    inp = make_inputs(wl)
    _check_module(wl, inp, Run(wl, inp).forward())


def _check_block(wl, inp, g):
    """The block against the oracle end to end (FT 3.5 block equation):
    every module intermediate and X1 within the bf16 bound, and `out` within
    the same bound element by element.  An element of `out` outside it is
    accepted only for its stated cause: the GPU's X1 differs from the
    oracle's (by its own bf16 rounding, inside the bound) somewhere in that
    token's 3x3 neighbourhood -- the FFN conv's reach -- and the FFN applied
    to the GPU's own X1 matches there.  The stage-wise FFN check holds on
    every element in any case."""
    kw = oracle_kwargs(wl)
    ref = O.hsmla_block_forward(inp["x"], inp, staged=True, **kw)
    kk = kw["keep_blocks"]
    if not np.array_equal(g["sel"][:, :kk], ref["sel"]):
        selection_band_check(ref["scores"], g["scores"], ref["sel"],
                             g["sel"][:, :kk], kk)
        ref = O.hsmla_block_forward(inp["x"], inp, staged=True,
                                    sel=g["sel"][:, :kk], **kw)
    for key in ("qkv", "qkv_hat", "o", "x1"):
        assert_close(g[key], ref[key], wl.dtype, key)
    assert_close(g["out"], _oracle_ffn(g["x1"], inp, wl), wl.dtype, "out (FFN of GPU x1)")
    atol, rtol = TOL[wl.dtype]
    bad = np.abs(g["out"] - ref["out"]) > atol + rtol * np.abs(ref["out"])
    n_bad = int(bad.sum())
    if n_bad:
        B, gh, gw = wl.batch, wl.grid_h, wl.grid_w
        x1_diff = np.any(g["x1"] != ref["x1"], axis=-1).reshape(B, gh, gw)
        near = np.zeros_like(x1_diff)
        pad = np.pad(x1_diff, ((0, 0), (1, 1), (1, 1)))
        for dy in range(3):
            for dx in range(3):
                near |= pad[:, dy:dy + gh, dx:dx + gw]
        bad_tok = bad.any(axis=-1).reshape(B, gh, gw)
        assert np.all(near[bad_tok]), (
            f"{int((bad_tok & ~near).sum())} tokens of out outside the bound "
            f"with X1 equal to the oracle's in their 3x3 neighbourhood")
        print(f"[block] {n_bad} of {bad.size} out elements outside the bound, "
              f"each next to an X1 rounding difference", flush=True)
    return ref


@pytest.mark.parametrize("keep", [0.0, 0.05, 0.5, 1.0])
def test_block_forward(keep):
    wl = scaled(STAGE_CASES["block_small"], keep=keep)
    inp = make_inputs(wl)
    _check_block(wl, inp, Run(wl, inp).block_forward())


def test_block_forward_layernorm_params():
    """LayerNorm scale and shift away from 1 and 0 in both norms (the
    synthetic block has 1 and 0): the per-channel gamma and beta reach the
    tile-blocked outputs that feed the projections."""
    wl = STAGE_CASES["block_small"]
    inp = dict(make_inputs(wl))
    rng = np.random.default_rng(7)
    C = wl.channels
    for k in ("ln1", "ln2"):
        inp[k + "_g"] = rng.uniform(0.5, 1.5, C)
        inp[k + "_b"] = rng.normal(0.0, 0.3, C)
    _check_block(wl, inp, Run(wl, inp).block_forward())


# More block shapes at C = 384: a 256-wide grid (two images, the rows at
# the top and bottom of each; the planar FFN hidden-tensor path) and a
# 128-wide one.
_BLOCK_SHAPES = {
    "w256_b2": scaled(WORKLOADS["block"], name="bs256", batch=2, grid_h=8, grid_w=256,
                      keep=0.25),
    "w128_b1": scaled(WORKLOADS["block"], name="bs128", batch=1, grid_h=24, grid_w=128,
                      keep=0.1),
    # channel-planar FFN path with two 32-row strips, the second ragged (40
    # rows), and eight 64-column conv tiles per row
    "w512_h40": scaled(WORKLOADS["block"], name="bs512", batch=1, grid_h=40, grid_w=512,
                       keep=0.1),
}


@pytest.mark.parametrize("name", sorted(_BLOCK_SHAPES))
def test_block_forward_shapes(name):
    wl = _BLOCK_SHAPES[name]
    inp = make_inputs(wl)
    print(f"[case] block forward {name}", flush=True)
    _check_block(wl, inp, Run(wl, inp).block_forward())


def test_block_forward_prepared_weights():
    """hsmla_prepare once, then blocks with desc.prepared: bit for bit the
    output of the block that prepares its own operands, twice in a row."""
    wl = _BLOCK_SHAPES["w256_b2"]
    inp = make_inputs(wl)
    r = Run(wl, inp)
    ref = r.block_forward()
    m = r.model
    ws = m.workspace(H.HSMLA_OP_BLOCK)
    announce("hsmla_prepare + hsmla_block_forward(prepared) w256_b2")
    H.hsmla_prepare(m.desc, H.HSMLA_OP_BLOCK, m.weights, m.ffn, ws)
    d = H.make_desc(**dict(m.shape, prepared=True))
    for _ in range(2):
        out = m.act()
        H.hsmla_block_forward(d, m.weights, m.ffn, r.x, out, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(out), ref["out"])


@pytest.mark.parametrize("name", ["street_small", "ragged_f32"])
def test_forward_and_qkv_prepared_weights(name):
    """hsmla_prepare for the module and for the QKV step, then calls with
    desc.prepared: bit for bit the outputs of the calls that prepare their
    own operands (tile-blocked copies for the whole-tile bf16 shape,
    row-major ones for the ragged float32 shape)."""
    wl = STAGE_CASES[name]
    inp = make_inputs(wl)
    r = Run(wl, inp)
    ref = r.forward()
    m = r.model
    d = H.make_desc(**dict(m.shape, prepared=True))
    ws = m.workspace(H.HSMLA_OP_FORWARD)
    announce(f"hsmla_prepare + hsmla_forward(prepared) {name}")
    H.hsmla_prepare(m.desc, H.HSMLA_OP_FORWARD, m.weights, None, ws)
    y = m.act()
    H.hsmla_forward(d, m.weights, r.x, y, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(y), ref["y"])
    wq = m.workspace(H.HSMLA_OP_QKV)
    q0, h0, q1, h1 = m.act(3), m.act(3), m.act(3), m.act(3)
    announce(f"hsmla_prepare + hsmla_qkv_branches(prepared) {name}")
    H.hsmla_qkv_branches(m.desc, m.weights, r.x, q0, h0, wq)
    H.hsmla_prepare(m.desc, H.HSMLA_OP_QKV, m.weights, None, wq)
    H.hsmla_qkv_branches(d, m.weights, r.x, q1, h1, wq)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1) and torch.equal(h0, h1)
    np.testing.assert_array_equal(to_host(q1), ref["qkv"])


def _oracle_ffn(x1, inp, wl):
    r = O.round_bf16
    xn2 = r(O.layer_norm(x1, inp["ln2_g"], inp["ln2_b"]))
    h1 = r(xn2 @ inp["w1"])
    h2 = r(O.gelu(O.dwconv_same(h1, inp["dw_ffn"], wl.grid_h, wl.grid_w)))
    return r(x1 + h2 @ inp["w2"])


@pytest.mark.parametrize("block,window,gh,gw", [(12, 16, 24, 36), (16, 20, 32, 48)])
def test_forward_bf16_large_blocks(block, window, gh, gw):
    """bf16 blocks of more than 128 tokens (144 and 256) take the
    refinement's general kernel (one thread per query)."""
    wl = scaled(WORKLOADS["street"], name=f"bf16_block{block}", batch=2, grid_h=gh,
                grid_w=gw, channels=64, heads=2, block=block, window=window, keep=0.34)
    inp = make_inputs(wl)
    assert wl.keep_blocks >= 2
    _check_module(wl, inp, Run(wl, inp).forward())


def test_block_forward_f32():
    wl = scaled(STAGE_CASES["block_small"], dtype="f32", grid_h=16, grid_w=32,
                channels=64, heads=2)
    inp = make_inputs(wl)
    g = Run(wl, inp).block_forward()
    ref = O.hsmla_block_forward(inp["x"], inp, **oracle_kwargs(wl))
    np.testing.assert_array_equal(g["sel"][:, :wl.keep_blocks], ref["sel"])
    assert_close(g["out"], ref["out"], "f32", "out")
