"""GPU parity of the training-time differentiable mixture, forward only
(FT 3.3: O = O_lin + M_b (O_local - O_linloc) on every block): the weighted
refinement entry point against the oracle with arbitrary per-block weights,
the degenerate weights, the whole forward with the block scores as weights,
and the full-size block workload."""

import numpy as np
import pytest
import torch

import oracle as O
from efficient_vision_attention_amd import hsmla as H
from efficient_vision_attention_amd.device import DeviceModel, to_device, to_f32, to_host
from workloads import WORKLOADS, make_inputs, scaled

from gpu_harness import (Run, announce, assert_close, oracle_kwargs, rnd_for,
                         shape_of, staged)
from test_gpu_stages import STAGE_CASES

pytestmark = pytest.mark.gpu


def _stage_inputs(wl, inp):
    rnd = rnd_for(wl)
    qkv = rnd(O.qkv_projection(inp["x"], inp["w_qkv"]))
    qkvh = rnd(O.multiscale_branches(qkv, inp["dw"], wl.grid_h, wl.grid_w))
    o_lin = rnd(O.linear_attention(qkvh, wl.heads)[0])
    return qkv, qkvh, o_lin


@pytest.mark.parametrize("name", list(STAGE_CASES))
def test_sparse_softmax_weighted(name):
    wl = STAGE_CASES[name]
    inp = make_inputs(wl)
    qkv_ref, qkvh_ref, o_lin = _stage_inputs(wl, inp)
    B, T = wl.batch, wl.num_blocks
    w = np.random.default_rng(T).uniform(0, 1, size=(B, T)).astype(np.float32)
    w[0, 0], w[-1, -1] = 0.0, 1.0
    m = DeviceModel(shape_of(wl, soft=True), inp)
    qkv, qkvh = to_device(qkv_ref, wl.dtype), to_device(qkvh_ref, wl.dtype)
    o = to_device(o_lin, wl.dtype)
    o_before = to_host(o)
    announce(f"hsmla_sparse_softmax_weighted {name}")
    H.hsmla_sparse_softmax_weighted(m.desc, qkv, qkvh, to_f32(w), o)
    torch.cuda.synchronize()
    allb = np.tile(np.arange(T), (B, 1))
    ref = O.refine_selected(qkv_ref, qkvh_ref, o_lin, allb, wl.grid_h, wl.grid_w,
                            wl.heads, wl.block, wl.window, rnd=rnd_for(wl),
                            weights=w.astype(np.float64))
    g = to_host(o)
    assert_close(g, ref, wl.dtype, "o soft")
    # a zero weight leaves its block's tokens bitwise unchanged
    nbc = wl.grid_w // wl.block
    ys, xs = np.divmod(np.arange(wl.tokens), wl.grid_w)
    t0 = ((ys // wl.block) * nbc + xs // wl.block) == 0
    assert np.array_equal(g[0][t0], o_before[0][t0])


@pytest.mark.parametrize("name", ["tiny", "street_small", "ragged_bf16", "ragged_f32",
                                  "exact_gate_bf16"])
def test_forward_soft(name):
    wl = STAGE_CASES[name]
    inp = make_inputs(wl)
    g = Run(wl, inp, soft=True).forward()
    ref = O.hsmla_forward(inp["x"], inp, staged=staged(wl), soft=True, **oracle_kwargs(wl))
    np.testing.assert_allclose(g["scores"], ref["scores"], rtol=0, atol=5e-5)
    for key in ("qkv", "qkv_hat", "o", "y"):
        assert_close(g[key], ref[key], wl.dtype, key)


def test_block_forward_soft_full_size():
    """The benchmark's block workload as the training-time forward: every
    block refined, stage-wise on sampled blocks from the GPU's inputs."""
    wl = WORKLOADS["block"]
    inp = make_inputs(wl)
    g = Run(wl, inp, soft=True).block_forward()
    rnd = O.round_bf16
    C, N, Hh = wl.channels, wl.tokens, wl.heads
    scores = O.gate_scores(g["qkv_hat"], inp["gate_w"], inp["gate_b"], wl.grid_h,
                           wl.grid_w, wl.block, Hh)
    np.testing.assert_allclose(g["scores"], scores, rtol=0, atol=2e-6)
    Z, D = O.kv_state(g["qkv_hat"][..., C:2 * C], g["qkv_hat"][..., 2 * C:], Hh)
    nbc = wl.grid_w // wl.block
    ys, xs = np.divmod(np.arange(N), wl.grid_w)
    tblk = (ys // wl.block) * nbc + xs // wl.block
    rng = np.random.default_rng(11)
    for b in range(wl.batch):
        pick = np.sort(rng.choice(wl.num_blocks, size=6, replace=False))
        toks = np.nonzero(np.isin(tblk, pick))[0]
        o_lin = np.zeros((1, N, C))
        o_lin[0, toks] = rnd(O.linear_readout(g["qkv_hat"][b:b + 1, toks, :C],
                                              Z[b:b + 1], D[b:b + 1], Hh))[0]
        ref = O.refine_selected(g["qkv"][b:b + 1], g["qkv_hat"][b:b + 1], o_lin,
                                pick[None], wl.grid_h, wl.grid_w, Hh, wl.block,
                                wl.window, rnd=rnd,
                                weights=g["scores"][b:b + 1].astype(np.float64))
        assert_close(g["o"][b, toks], ref[0, toks], "bf16", f"o soft image {b}")
        rows = np.sort(rng.choice(N, size=256, replace=False))
        assert_close(g["x1"][b, rows], rnd(inp["x"][b, rows] + g["o"][b, rows] @ inp["w_o"]),
                     "bf16", f"x1 image {b}")
