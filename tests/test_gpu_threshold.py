"""GPU parity of threshold routing (the routed set {t : M_t > tau} of the
gating equation in FT 3.2, refined by FT 3.3's sparse residual): the
compaction kernel on injected scores (bit-exact, ties at tau), the pooled
gate, the counted refinement, and the whole forward against the oracle run
with the same tau."""

import numpy as np
import pytest
import torch

import oracle as O
from efficient_vision_attention_amd import hsmla as H
from efficient_vision_attention_amd.device import DeviceModel, to_device, to_host
from workloads import WORKLOADS, make_inputs, scaled

from gpu_harness import (Run, announce, assert_close, oracle_kwargs, padded,
                         routed_lists, rnd_for, shape_of, staged, tau_between,
                         threshold_band_check)
from test_gpu_stages import STAGE_CASES

pytestmark = pytest.mark.gpu


def _token_blocks(wl):
    nbc = wl.grid_w // wl.block
    ys, xs = np.divmod(np.arange(wl.tokens), wl.grid_w)
    return (ys // wl.block) * nbc + xs // wl.block


@pytest.mark.parametrize("T,levels,tau", [
    (16, 4, 0.5),        # scores on a 1/4 grid: tau equal to a score level
    (45, 5, 0.4),
    (1000, 9, 3 / 9),
    (1024, 17, 0.5),
    (2000, 7, 0.0),      # zero scores sit exactly at tau
    (8192, 33, 17 / 33),  # the largest block count
    (300, 3, -1.0),      # every block routed
    (300, 3, 2.0),       # no block routed
])
def test_threshold_injected_scores_exact(T, levels, tau):
    """Exact float32 scores on a coarse grid, many equal to tau: a score equal
    to tau is not routed, and the lists and counts equal the oracle's bit for
    bit."""
    rng = np.random.default_rng(T * 7 + levels)
    B = 3
    scores = (rng.integers(0, levels, size=(B, T)) / levels).astype(np.float32)
    tau32 = np.float32(tau)
    desc = H.make_desc(batch=B, grid_h=1, grid_w=T, channels=32, heads=1,
                       branches=(), block=1, window=1, keep_blocks=0,
                       dtype="bf16", tau=float(tau32))
    s_in = torch.from_numpy(scores).cuda()
    s_out = torch.zeros_like(s_in)
    sel = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    announce(f"hsmla_gate_threshold injected T={T} tau={tau}")
    H.hsmla_gate_threshold(desc, None, None, None, s_in, s_out, sel, counts)
    torch.cuda.synchronize()
    ref_sel, ref_cnt = O.select_threshold(scores, tau32)
    g_sel, g_cnt = sel.cpu().numpy(), counts.cpu().numpy()
    np.testing.assert_array_equal(g_cnt, ref_cnt)
    for b in range(B):
        np.testing.assert_array_equal(g_sel[b, :g_cnt[b]], ref_sel[b, :ref_cnt[b]])
        assert np.all(g_sel[b, g_cnt[b]:] == -7)  # beyond the count: untouched
    assert torch.equal(s_out, s_in)


@pytest.mark.parametrize("name", ["tiny", "street_small", "ragged_bf16", "ragged_f32",
                                  "exact_gate_bf16"])
def test_gate_threshold_pooled(name):
    wl = STAGE_CASES[name]
    inp = make_inputs(wl)
    rnd = rnd_for(wl)
    qkvh_ref = rnd(O.multiscale_branches(rnd(O.qkv_projection(inp["x"], inp["w_qkv"])),
                                         inp["dw"], wl.grid_h, wl.grid_w))
    ref_scores = O.gate_scores(qkvh_ref, inp["gate_w"], inp["gate_b"], wl.grid_h,
                               wl.grid_w, wl.block, wl.heads,
                               gate_dw=inp.get("gate_dw"))
    tau = tau_between(ref_scores, 0.7)
    m = DeviceModel(shape_of(wl, tau=tau), inp)
    qkvh = to_device(qkvh_ref, wl.dtype)
    T = wl.num_blocks
    scores = torch.empty((wl.batch, T), dtype=torch.float32, device="cuda")
    sel = torch.empty((wl.batch, T), dtype=torch.int32, device="cuda")
    counts = torch.empty((wl.batch,), dtype=torch.int32, device="cuda")
    announce(f"hsmla_gate_threshold pooled {name} tau={tau:.6g}")
    H.hsmla_gate_threshold(m.desc, qkvh, m.t["gate_w"], m.t["gate_b"], None,
                           scores, sel, counts, gate_dw=m.t["gate_dw"])
    torch.cuda.synchronize()
    g = to_host(scores)
    np.testing.assert_allclose(g, ref_scores, rtol=0, atol=2e-6)
    g_lists = routed_lists(sel.cpu().numpy(), counts.cpu().numpy())
    # the GPU's own scores thresholded by the oracle give the GPU's lists
    own_sel, own_cnt = O.select_threshold(g.astype(np.float32), np.float32(tau))
    np.testing.assert_array_equal(counts.cpu().numpy(), own_cnt)
    for b in range(wl.batch):
        np.testing.assert_array_equal(g_lists[b], own_sel[b, :own_cnt[b]])
    ref_sel, ref_cnt = O.select_threshold(ref_scores.astype(np.float32), np.float32(tau))
    threshold_band_check(ref_scores, g, tau, routed_lists(ref_sel, ref_cnt), g_lists)


@pytest.mark.parametrize("name", ["street_small", "ragged_bf16", "ragged_f32",
                                  "pathology_small"])
def test_sparse_softmax_counted(name):
    """The counted refinement touches exactly the first counts[b] entries:
    the rest of each sel row holds other valid blocks that must stay
    unrefined."""
    wl = STAGE_CASES[name]
    inp = make_inputs(wl)
    rnd = rnd_for(wl)
    qkv_ref = rnd(O.qkv_projection(inp["x"], inp["w_qkv"]))
    qkvh_ref = rnd(O.multiscale_branches(qkv_ref, inp["dw"], wl.grid_h, wl.grid_w))
    o_lin = rnd(O.linear_attention(qkvh_ref, wl.heads)[0])
    T = wl.num_blocks
    rng = np.random.default_rng(5)
    perm = np.stack([rng.permutation(T) for _ in range(wl.batch)])
    cnt = rng.integers(0, T + 1, size=wl.batch)
    cnt[0] = max(1, T // 3)
    lists = [np.sort(perm[b, :cnt[b]]) for b in range(wl.batch)]
    sel_np = perm.copy()
    for b in range(wl.batch):
        sel_np[b, :cnt[b]] = lists[b]  # routed part ascending, rest other blocks
    m = DeviceModel(shape_of(wl, tau=0.5), inp)
    qkv = to_device(qkv_ref, wl.dtype)
    qkvh = to_device(qkvh_ref, wl.dtype)
    o = to_device(o_lin, wl.dtype)
    o_before = o.clone()
    sel = torch.from_numpy(sel_np.astype(np.int32)).cuda().contiguous()
    counts = torch.from_numpy(cnt.astype(np.int32)).cuda()
    announce(f"hsmla_sparse_softmax_counted {name} counts={cnt.tolist()}")
    H.hsmla_sparse_softmax_counted(m.desc, qkv, qkvh, sel, counts, o)
    torch.cuda.synchronize()
    ref = O.refine_selected(qkv_ref, qkvh_ref, o_lin, padded(lists, T), wl.grid_h,
                            wl.grid_w, wl.heads, wl.block, wl.window, rnd=rnd)
    assert_close(to_host(o), ref, wl.dtype, "o refined (counted)")
    tblk = _token_blocks(wl)
    for b in range(wl.batch):
        untouched = torch.from_numpy(~np.isin(tblk, lists[b])).cuda()
        assert torch.equal(o[b][untouched], o_before[b][untouched])


def _check_threshold_forward(wl, inp, g, tau, block=False):
    kw = oracle_kwargs(wl)
    st = staged(wl)
    fwd = O.hsmla_block_forward if block else O.hsmla_forward
    ref = fwd(inp["x"], inp, staged=st, tau=tau, **kw)
    T = wl.num_blocks
    g_lists = routed_lists(g["sel"], g["counts"])
    ref_lists = routed_lists(ref["sel"], ref["counts"])
    # the GPU's lists are the threshold of its own scores, exactly
    own_sel, own_cnt = O.select_threshold(g["scores"].astype(np.float32), np.float32(tau))
    np.testing.assert_array_equal(g["counts"], own_cnt)
    for b in range(wl.batch):
        np.testing.assert_array_equal(g_lists[b], own_sel[b, :own_cnt[b]])
    if any(not np.array_equal(a, b) for a, b in zip(g_lists, ref_lists)):
        rep = threshold_band_check(ref["scores"], g["scores"], tau, ref_lists, g_lists)
        print("routing differs inside the tie band:", rep)
        ref = fwd(inp["x"], inp, staged=st, sel=padded(g_lists, T), **kw)
    np.testing.assert_allclose(g["scores"], ref["scores"], rtol=0, atol=5e-5)
    keys = ("qkv", "qkv_hat", "o", "x1") if block else ("qkv", "qkv_hat", "o", "y")
    for key in keys:
        assert_close(g[key], ref[key], wl.dtype, key)
    return ref


def _tau_for(wl, inp, quantile):
    """tau between two adjacent oracle scores at the quantile."""
    r = O.hsmla_module(inp["x"], inp, staged=staged(wl), **oracle_kwargs(wl))
    return tau_between(r["scores"], quantile)


@pytest.mark.parametrize("name", list(STAGE_CASES))
def test_forward_threshold(name):
    wl = STAGE_CASES[name]
    inp = make_inputs(wl)
    tau = _tau_for(wl, inp, 0.7)  # about 30% of the blocks routed
    g = Run(wl, inp, tau=tau).forward()
    _check_threshold_forward(wl, inp, g, tau)


def test_threshold_equals_topk_between_kth_and_next():
    """One image: a tau strictly between the k-th and (k+1)-th GPU score
    routes the same blocks, in the same order, as top-k with k, so the two
    forwards are bitwise equal."""
    wl = STAGE_CASES["pathology_small"]
    inp = make_inputs(wl)
    k = wl.keep_blocks
    top = Run(wl, inp).forward()
    s = np.sort(top["scores"][0].astype(np.float32))[::-1]
    assert s[k - 1] > s[k], "k-th and (k+1)-th scores tie; pick another case"
    tau = float(np.float32((np.float64(s[k - 1]) + np.float64(s[k])) / 2))
    assert s[k] < np.float32(tau) < s[k - 1]
    thr = Run(wl, inp, tau=tau).forward()
    assert int(thr["counts"][0]) == k
    np.testing.assert_array_equal(thr["sel"][0, :k], top["sel"][0, :k])
    for key in ("scores", "o", "y"):
        assert np.array_equal(thr[key], top[key]), key


def test_threshold_equals_topk_from_partial_logits():
    """The same with 256 blocks per image, where both routings form their
    scores from the S2 conv's partial logits (top-k inside its ranking
    launch, the threshold routing in a launch of its own, both adding the
    heads' sigmoids in head order): scores, lists and forwards are bitwise
    equal."""
    wl = scaled(WORKLOADS["pathology"], batch=1, grid_h=128, grid_w=128)
    assert wl.num_blocks == 256
    inp = make_inputs(wl)
    k = wl.keep_blocks
    top = Run(wl, inp).forward()
    s = np.sort(top["scores"][0].astype(np.float32))[::-1]
    assert s[k - 1] > s[k], "k-th and (k+1)-th scores tie; pick another case"
    tau = float(np.float32((np.float64(s[k - 1]) + np.float64(s[k])) / 2))
    thr = Run(wl, inp, tau=tau).forward()
    assert int(thr["counts"][0]) == k
    np.testing.assert_array_equal(thr["sel"][0, :k], top["sel"][0, :k])
    for key in ("scores", "o", "y"):
        assert np.array_equal(thr[key], top[key]), key


@pytest.mark.parametrize("name", ["tiny", "ragged_bf16"])
def test_threshold_extremes(name):
    """tau above every score: nothing routed, o is the linear path; tau below
    every score: every block routed, as top-k with k = T."""
    wl = STAGE_CASES[name]
    inp = make_inputs(wl)
    none = Run(wl, inp, tau=2.0).forward()  # sigmoid means lie in (0, 1)
    assert np.all(none["counts"] == 0)
    zero = Run(wl, inp, keep_blocks=0).forward()
    assert np.array_equal(none["o"], zero["o"]) and np.array_equal(none["y"], zero["y"])
    every = Run(wl, inp, tau=-1.0).forward()
    assert np.all(every["counts"] == wl.num_blocks)
    full = Run(wl, inp, keep_blocks=wl.num_blocks).forward()
    assert np.array_equal(every["o"], full["o"]) and np.array_equal(every["y"], full["y"])


def test_block_forward_threshold():
    wl = STAGE_CASES["block_small"]
    inp = make_inputs(wl)
    xn1 = O.round_bf16(O.layer_norm(inp["x"], inp["ln1_g"], inp["ln1_b"]))
    r = O.hsmla_module(xn1, inp, staged=True, **oracle_kwargs(wl))
    tau = tau_between(r["scores"], 0.7)
    g = Run(wl, inp, tau=tau).block_forward()
    _check_threshold_forward(wl, inp, g, tau, block=True)


def test_block_forward_threshold_full_size():
    """The benchmark's block workload under threshold routing at about 30%
    routed blocks (tau from a first top-k run's scores), checked stage-wise
    as the other full-size tests."""
    from test_gpu_fullsize import _check_module_fullsize
    wl = scaled(WORKLOADS["block"], keep=0.3)
    inp = make_inputs(wl)
    pilot = Run(wl, inp).block_forward()
    tau = tau_between(pilot["scores"], 0.7)
    g = Run(wl, inp, tau=tau).block_forward()
    xn1 = O.round_bf16(O.layer_norm(inp["x"], inp["ln1_g"], inp["ln1_b"]))
    _check_module_fullsize(wl, dict(inp, x=xn1), g, tau=tau)
    frac = g["counts"].sum() / (wl.batch * wl.num_blocks)
    assert 0.2 < frac < 0.4, frac
