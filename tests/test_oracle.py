"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something other than itself: a library
routine on the CPU, a closed form, a brute-force formulation written
differently, a hand-worked fixture, or an exhaustive search.  Together they
are chosen so that a dropped term, a wrong sign, a transposed operand or a
wrong index in the oracle fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import WORKLOADS, make_inputs, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# bfloat16 rounding
# ---------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_float32_values():
    rng = _rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        rng.standard_normal(2000) * 1e-39,  # float32 subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38]),
    ]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(vals.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_ties_and_overflow():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even one
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert O.round_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127  # largest finite bfloat16
    assert O.round_bf16(big) == big
    assert np.isinf(O.round_bf16((2.0 - 2.0 ** -8) * 2.0 ** 127))
    assert np.isnan(O.round_bf16(np.nan))
    # fp64 value just above a float32 tie: direct rounding goes up
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert O.round_bf16(x) == 1.0 + 2.0 ** -7


# ---------------------------------------------------------------------------
# projection and depthwise branches
# ---------------------------------------------------------------------------

def test_qkv_projection_is_a_plain_matmul():
    rng = _rng(2)
    x = rng.standard_normal((2, 5, 4))
    w = rng.standard_normal((4, 12))
    got = O.qkv_projection(x, w)
    for b in range(2):
        for n in range(5):
            for c in range(12):
                ref = sum(x[b, n, i] * w[i, c] for i in range(4))
                assert abs(got[b, n, c] - ref) < 1e-12


@pytest.mark.parametrize("k", [3, 5, 7])
def test_dwconv_matches_torch_conv2d(k):
    rng = _rng(3 + k)
    B, gh, gw, Ch = 2, 9, 13, 6
    t = rng.standard_normal((B, gh * gw, Ch))
    w = rng.standard_normal((Ch, k, k))
    got = O.dwconv_same(t, w, gh, gw)
    inp = torch.from_numpy(t.reshape(B, gh, gw, Ch)).permute(0, 3, 1, 2)
    ref = torch.nn.functional.conv2d(inp, torch.from_numpy(w)[:, None],
                                     padding=(k - 1) // 2, groups=Ch)
    ref = ref.permute(0, 2, 3, 1).reshape(B, gh * gw, Ch).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_multiscale_delta_kernels_give_scaled_identity():
    rng = _rng(4)
    B, gh, gw, Ch = 1, 6, 7, 5
    t = rng.standard_normal((B, gh * gw, Ch))
    d3 = np.zeros((Ch, 3, 3)); d3[:, 1, 1] = 1.0
    d5 = np.zeros((Ch, 5, 5)); d5[:, 2, 2] = 1.0
    got = O.multiscale_branches(t, [d3, d5], gh, gw)
    np.testing.assert_allclose(got, 3.0 * t, rtol=0, atol=1e-14)
    # a shifted delta moves every channel by one column, with zero fill
    s3 = np.zeros((Ch, 3, 3)); s3[:, 1, 2] = 1.0
    got = O.dwconv_same(t, s3, gh, gw).reshape(B, gh, gw, Ch)
    img = t.reshape(B, gh, gw, Ch)
    np.testing.assert_array_equal(got[:, :, :-1], img[:, :, 1:])
    np.testing.assert_array_equal(got[:, :, -1], 0.0)


# ---------------------------------------------------------------------------
# global linear attention
# ---------------------------------------------------------------------------

def _brute_linear(qh, kh, vh, heads):
    """sum_m (phi(q_n).phi(k_m)) v_m / sum_m phi(q_n).phi(k_m), O(N^2)."""
    B, N, C = qh.shape
    d = C // heads
    out = np.zeros_like(qh)
    for b in range(B):
        for h in range(heads):
            sl = slice(h * d, (h + 1) * d)
            fq = np.maximum(qh[b, :, sl], 0)
            fk = np.maximum(kh[b, :, sl], 0)
            a = fq @ fk.T  # [N, N] kernel scores
            den = a.sum(axis=1)
            num = a @ vh[b, :, sl]
            for n in range(N):
                out[b, n, sl] = num[n] / den[n] if den[n] > 0 else 0.0
    return out


def test_linear_attention_equals_brute_force_quadratic_form():
    rng = _rng(5)
    B, N, H, d = 2, 37, 3, 8
    C = H * d
    qkvh = rng.standard_normal((B, N, 3 * C))
    qkvh[0, 4, 0:C] = -np.abs(qkvh[0, 4, 0:C])  # a query with phi(q) = 0
    got, Z, D = O.linear_attention(qkvh, H)
    ref = _brute_linear(qkvh[..., :C], qkvh[..., C:2 * C], qkvh[..., 2 * C:], H)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
    assert np.all(got[0, 4] == 0.0)
    assert Z.shape == (B, H, d, d) and D.shape == (B, H, d)


def test_linear_attention_scale_invariance():
    rng = _rng(6)
    B, N, H, d = 1, 20, 2, 4
    C = H * d
    qkvh = rng.standard_normal((B, N, 3 * C))
    base, _, _ = O.linear_attention(qkvh, H)
    for lo, hi, s in [(0, C, 3.5), (C, 2 * C, 0.25)]:
        alt = qkvh.copy()
        alt[..., lo:hi] *= s
        got, _, _ = O.linear_attention(alt, H)
        np.testing.assert_allclose(got, base, rtol=1e-12, atol=1e-13)
    # scaling V scales the output (V enters linearly, without phi)
    alt = qkvh.copy()
    alt[..., 2 * C:] *= -2.0
    got, _, _ = O.linear_attention(alt, H)
    np.testing.assert_allclose(got, -2.0 * base, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# hand-worked fixtures
# ---------------------------------------------------------------------------

def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_fixture_refine_1x3():
    fx = _load("refine_1x3.json")
    qkv = np.array(fx["qkv"])
    qkvh = np.array(fx["qkv_hat"])
    e = fx["expected"]
    o_lin, Z, D = O.linear_attention(qkvh, 1)
    assert abs(Z[0, 0, 0, 0] - e["Z"]) < 1e-12 and abs(D[0, 0, 0] - e["D"]) < 1e-12
    np.testing.assert_allclose(o_lin[0, :, 0], e["o_lin"], atol=1e-12)
    kw = dict(grid_h=1, grid_w=3, heads=1, block=1, window=3)
    o_all = O.refine_selected(qkv, qkvh, o_lin, np.array([[0, 1, 2]]), **kw)
    np.testing.assert_allclose(o_all[0, :, 0], e["o_all_selected"], atol=1e-12)
    o_one = O.refine_selected(qkv, qkvh, o_lin, np.array([[1]]), **kw)
    np.testing.assert_allclose(o_one[0, :, 0], e["o_select_block1"], atol=1e-12)


def test_fixture_gate_2x4():
    fx = _load("gate_2x4.json")
    qkvh = np.array(fx["qkv_hat"])
    m = O.gate_scores(qkvh, np.array(fx["gate_w"]), np.array(fx["gate_b"]),
                      grid_h=2, grid_w=4, block=2, heads=2)
    np.testing.assert_allclose(m[0], fx["expected"]["scores"], atol=1e-14)
    assert O.select_blocks(m, 1)[0].tolist() == fx["expected"]["top1"]


# ---------------------------------------------------------------------------
# gate
# ---------------------------------------------------------------------------

def test_gate_zero_weights_gives_mean_sigmoid_of_bias():
    rng = _rng(7)
    H, d = 3, 4
    qkvh = rng.standard_normal((2, 8 * 8, 3 * H * d))
    b = np.array([0.3, -1.2, 2.0])
    m = O.gate_scores(qkvh, np.zeros((H, 3 * d)), b, 8, 8, 4, H)
    ref = np.mean(1.0 / (1.0 + np.exp(-b)))
    np.testing.assert_allclose(m, ref, rtol=0, atol=1e-15)


def test_gate_block_mean_is_per_block():
    """A feature constant on each block with a one-hot weight reproduces the
    per-block constant as the logit (block numbering and pooling window)."""
    H, d, Bs, gh, gw = 2, 2, 2, 4, 6
    C = H * d
    T = (gh // Bs) * (gw // Bs)
    vals = np.arange(T) * 0.1 - 0.2
    qkvh = np.zeros((1, gh * gw, 3 * C))
    for n in range(gh * gw):
        y, x = divmod(n, gw)
        t = (y // Bs) * (gw // Bs) + x // Bs
        qkvh[0, n, C + 1 * d + 1] = vals[t]  # k channel 1 of head 1
    w = np.zeros((H, 3 * d)); w[1, d + 1] = 1.0  # head 1 weights its k_1
    m = O.gate_scores(qkvh, w, np.zeros(H), gh, gw, Bs, H)
    ref = 0.5 * (0.5 + 1.0 / (1.0 + np.exp(-vals)))
    np.testing.assert_allclose(m[0], ref, atol=1e-15)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def _is_valid_topk(scores, subset):
    inside = set(subset)
    for i in inside:
        for j in range(len(scores)):
            if j in inside:
                continue
            if not (scores[i] > scores[j] or (scores[i] == scores[j] and i < j)):
                return False
    return True


def test_gate_delta_kernel_equals_plain_gate():
    rng = _rng(11)
    H, d, gh, gw, Bs = 2, 4, 8, 12, 4
    qkvh = rng.normal(size=(2, gh * gw, 3 * H * d))
    w, b = rng.normal(size=(H, 3 * d)), rng.normal(size=H)
    delta = np.zeros((3 * H * d, 3, 3))
    delta[:, 1, 1] = 1.0
    np.testing.assert_allclose(
        O.gate_scores(qkvh, w, b, gh, gw, Bs, H, gate_dw=delta),
        O.gate_scores(qkvh, w, b, gh, gw, Bs, H), rtol=1e-14, atol=1e-15)


def test_gate_conv_matches_loops_over_the_definition():
    """G_b^(h) = sigmoid(w . AvgPool_b(DWConv3x3(x)) + b), written as plain
    loops: each token of the block, each tap, zero outside the grid."""
    rng = _rng(12)
    H, d, gh, gw, Bs = 2, 2, 6, 4, 2
    C3 = 3 * H * d
    qkvh = rng.normal(size=(1, gh * gw, C3))
    gdw = rng.normal(size=(C3, 3, 3))
    w, b = rng.normal(size=(H, 3 * d)), rng.normal(size=H)
    got = O.gate_scores(qkvh, w, b, gh, gw, Bs, H, gate_dw=gdw)
    nbc = gw // Bs
    for t in range(got.shape[1]):
        r0, c0 = (t // nbc) * Bs, (t % nbc) * Bs
        gs = []
        for h in range(H):
            feats = []
            for part in range(3):  # q, k, v
                for j in range(d):
                    ch = part * H * d + h * d + j
                    acc = 0.0
                    for y in range(r0, r0 + Bs):
                        for x in range(c0, c0 + Bs):
                            for dy in range(3):
                                for dx in range(3):
                                    yy, xx = y + dy - 1, x + dx - 1
                                    if 0 <= yy < gh and 0 <= xx < gw:
                                        acc += gdw[ch, dy, dx] * qkvh[0, yy * gw + xx, ch]
                    feats.append(acc / (Bs * Bs))
            z = sum(w[h][i] * feats[i] for i in range(3 * d)) + b[h]
            gs.append(1.0 / (1.0 + math.exp(-z)))
        assert abs(got[0, t] - sum(gs) / H) < 1e-12


def test_gate_conv_constant_field_closed_form():
    """All-ones input and kernel on a 4 x 4 grid, 2 x 2 blocks: a token sees
    as many in-grid neighbours (itself included) as its 3x3 window holds, so
    every block averages 4, 6, 6 and 9 -> 25 / 4 (each block touches two
    borders).  On 6 x 6 the centre block's tokens see 9 each, and the
    top-middle block's border row 6 each, its inner row 9 each."""
    H, d = 1, 1
    w = np.array([[1.0, 0.0, 0.0]])  # logit = the q feature
    ones = np.ones((3, 3, 3))
    m4 = O.gate_scores(np.ones((1, 16, 3)), w, np.zeros(1), 4, 4, 2, H, gate_dw=ones)
    np.testing.assert_allclose(m4, 1.0 / (1.0 + np.exp(-6.25)), rtol=1e-14)
    m6 = O.gate_scores(np.ones((1, 36, 3)), w, np.zeros(1), 6, 6, 2, H, gate_dw=ones)
    # centre block (t = 4): 9 per token; corner block: 25/4 as on 4 x 4
    assert abs(m6[0, 4] - 1.0 / (1.0 + math.exp(-9.0))) < 1e-14
    edge = (6 + 6 + 9 + 9) / 4  # top-middle block: border row 6 each, inner row 9 each
    assert abs(m6[0, 1] - 1.0 / (1.0 + math.exp(-edge))) < 1e-14
    assert abs(m6[0, 0] - 1.0 / (1.0 + math.exp(-6.25))) < 1e-14


@pytest.mark.parametrize("seed", range(6))
def test_select_blocks_exhaustive(seed):
    rng = _rng(100 + seed)
    T = 9
    # few distinct values so ties are frequent
    scores = rng.integers(0, 4, size=(3, T)).astype(np.float64) / 4.0
    for k in range(T + 1):
        sel = O.select_blocks(scores, k)
        for b in range(3):
            valid = [s for s in itertools.combinations(range(T), k)
                     if _is_valid_topk(scores[b], s)]
            assert len(valid) == 1
            assert tuple(sel[b].tolist()) == valid[0]


# ---------------------------------------------------------------------------
# refinement
# ---------------------------------------------------------------------------

def _window_member(t, n, grid_w, block, window):
    """Key token n lies in block t's window iff its row and column are each
    within p tokens of the block's extent (Chebyshev-style distance)."""
    p = (window - block) // 2
    nbc = grid_w // block
    r0, c0 = (t // nbc) * block, (t % nbc) * block
    y, x = divmod(n, grid_w)
    dy = max(0, r0 - y, y - (r0 + block - 1))
    dx = max(0, c0 - x, x - (c0 + block - 1))
    return dy <= p and dx <= p


def _dense_refine(qkv, qkvh, o_lin, sel, gh, gw, H, Bs, w):
    """Refinement written over the full token set with a mask per query."""
    B, N, C3 = qkv.shape
    C = C3 // 3
    d = C // H
    out = o_lin.copy()
    for b in range(B):
        for t in sel[b]:
            mask = np.array([_window_member(t, n, gw, Bs, w) for n in range(N)])
            queries = [n for n in range(N)
                       if (n // gw) // Bs * (gw // Bs) + (n % gw) // Bs == t]
            for h in range(H):
                sl = slice(h * d, (h + 1) * d)
                q = qkv[b, :, sl]
                k = qkv[b, :, C + h * d:C + (h + 1) * d]
                v = qkv[b, :, 2 * C + h * d:2 * C + (h + 1) * d]
                fq = np.maximum(qkvh[b, :, sl], 0)
                fk = np.maximum(qkvh[b, :, C + h * d:C + (h + 1) * d], 0)
                vh = qkvh[b, :, 2 * C + h * d:2 * C + (h + 1) * d]
                for i in queries:
                    s = np.where(mask, k @ q[i] / math.sqrt(d), -np.inf)
                    p = np.exp(s - s.max())
                    loc = (p / p.sum()) @ v
                    a = np.where(mask, fk @ fq[i], 0.0)
                    ll = (a @ vh) / a.sum() if a.sum() > 0 else np.zeros(d)
                    out[b, i, sl] = o_lin[b, i, sl] + loc - ll
    return out


@pytest.mark.parametrize("Bs,w,gh,gw", [(2, 6, 6, 8), (2, 2, 4, 6), (3, 7, 9, 6)])
def test_refine_matches_masked_dense_form(Bs, w, gh, gw):
    rng = _rng(8 + w)
    B, H, d = 2, 2, 3
    C = H * d
    N = gh * gw
    qkv = rng.standard_normal((B, N, 3 * C))
    qkvh = rng.standard_normal((B, N, 3 * C))
    o_lin, _, _ = O.linear_attention(qkvh, H)
    T = (gh // Bs) * (gw // Bs)
    sel = np.stack([np.sort(rng.choice(T, size=T // 2, replace=False))
                    for _ in range(B)])
    got = O.refine_selected(qkv, qkvh, o_lin, sel, gh, gw, H, Bs, w)
    ref = _dense_refine(qkv, qkvh, o_lin, sel, gh, gw, H, Bs, w)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_window_bounds_against_membership():
    for (gh, gw, Bs, w) in [(8, 12, 4, 8), (16, 16, 4, 12), (9, 9, 3, 3)]:
        T = (gh // Bs) * (gw // Bs)
        for t in range(T):
            r_lo, r_hi, c_lo, c_hi = O.window_bounds(t, gh, gw, Bs, w)
            for n in range(gh * gw):
                y, x = divmod(n, gw)
                inside = r_lo <= y < r_hi and c_lo <= x < c_hi
                assert inside == _window_member(t, n, gw, Bs, w)


def _module_kwargs(gh, gw, H, Bs, w, k):
    return dict(grid_h=gh, grid_w=gw, heads=H, block=Bs, window=w,
                keep_blocks=k)


def test_keep_zero_is_pure_linear_attention():
    wl = scaled(WORKLOADS["tiny"], keep=0.0)
    inp = make_inputs(wl)
    r = O.hsmla_forward(inp["x"], inp, **wl.kwargs())
    assert r["sel"].shape == (1, 0)
    np.testing.assert_array_equal(r["o"], r["o_lin"])
    np.testing.assert_allclose(r["y"], r["o_lin"] @ inp["w_o"], atol=1e-13)


def test_keep_all_with_covering_window_is_full_softmax():
    """Z_W = Z when the window covers the grid, so the linear terms cancel
    and the output is textbook softmax attention over raw Q, K, V."""
    wl = scaled(WORKLOADS["tiny"], keep=1.0, window=4 + 2 * 16)
    inp = make_inputs(wl)
    r = O.hsmla_module(inp["x"], inp, **wl.kwargs())
    assert r["sel"].shape == (1, wl.num_blocks)
    qkv = torch.from_numpy(r["qkv"])
    B, N, C3 = qkv.shape
    C = C3 // 3
    H, d = wl.heads, wl.head_dim
    q, k, v = (qkv[..., s * C:(s + 1) * C].reshape(B, N, H, d).transpose(1, 2)
               for s in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    ref = ref.transpose(1, 2).reshape(B, N, C).numpy()
    np.testing.assert_allclose(r["o"], ref, rtol=1e-10, atol=1e-11)


def test_keep_all_window_equal_block_is_block_local():
    """window = block: every block attends only to itself, and the linear
    correction is the linear attention restricted to the block."""
    rng = _rng(9)
    gh, gw, Bs, H, d = 8, 8, 4, 2, 4
    C = H * d
    qkv = rng.standard_normal((1, gh * gw, 3 * C))
    qkvh = rng.standard_normal((1, gh * gw, 3 * C))
    o_lin, _, _ = O.linear_attention(qkvh, H)
    T = 4
    got = O.refine_selected(qkv, qkvh, o_lin, np.arange(T)[None], gh, gw, H,
                            Bs, Bs)
    # reference: per block, gather its tokens and apply textbook formulas
    ref = o_lin.copy()
    for t in range(T):
        ys, xs = (t // 2) * 4 + np.arange(4), (t % 2) * 4 + np.arange(4)
        ids = (ys[:, None] * gw + xs[None, :]).reshape(-1)
        sub = qkv[:, ids]
        subh = qkvh[:, ids]
        qq, kk, vv = (torch.from_numpy(sub[..., s * C:(s + 1) * C])
                      .reshape(1, 16, H, d).transpose(1, 2) for s in range(3))
        soft = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)
        soft = soft.transpose(1, 2).reshape(1, 16, C).numpy()
        lin = _brute_linear(subh[..., :C], subh[..., C:2 * C], subh[..., 2 * C:], H)
        ref[:, ids] = o_lin[:, ids] + soft - lin
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


# ---------------------------------------------------------------------------
# block wrapper pieces and staging
# ---------------------------------------------------------------------------

def test_layer_norm_and_gelu_match_torch():
    rng = _rng(10)
    x = rng.standard_normal((3, 7, 24)) * 3 + 1
    g = rng.standard_normal(24)
    b = rng.standard_normal(24)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (24,),
                                         torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(O.layer_norm(x, g, b), ref, atol=1e-12)
    ref = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(O.gelu(x), ref, atol=1e-13)


def test_staged_mode_rounds_and_stays_close():
    wl = scaled(WORKLOADS["street"], batch=1, grid_h=16, grid_w=32)
    inp = make_inputs(wl)
    ex = O.hsmla_forward(inp["x"], inp, **wl.kwargs())
    st = O.hsmla_forward(inp["x"], inp, staged=True, sel=ex["sel"],
                         **wl.kwargs())
    for key in ("qkv", "qkv_hat", "o_lin", "o", "y"):
        np.testing.assert_array_equal(O.round_bf16(st[key]), st[key])
        np.testing.assert_allclose(st[key], ex[key], rtol=3e-2, atol=3e-2)


def _block_case(keep=0.1, seed=5):
    wl = scaled(WORKLOADS["block"], batch=1, grid_h=16, grid_w=16,
                channels=64, heads=2, keep=keep, seed=seed)
    return wl, make_inputs(wl)


@pytest.mark.parametrize("staged", [False, True])
def test_block_forward_zero_w2_leaves_x1(staged):
    # FT 3.5 block equation: the FFN branch enters the output only through
    # W2, so W2 = 0 gives out = X1 exactly, whatever the rest computes
    wl, inp = _block_case()
    inp = dict(inp, w2=np.zeros_like(inp["w2"]))
    r = O.hsmla_block_forward(inp["x"], inp, staged=staged, **wl.kwargs())
    np.testing.assert_array_equal(r["out"], r["x1"])
    assert np.abs(r["x1"] - inp["x"]).max() > 1e-2  # the attention did act


def test_block_forward_zero_ffn_conv_leaves_x1():
    # a zero depthwise kernel zeroes the conv, GELU(0) = 0, so out = X1
    wl, inp = _block_case()
    inp = dict(inp, dw_ffn=np.zeros_like(inp["dw_ffn"]))
    r = O.hsmla_block_forward(inp["x"], inp, **wl.kwargs())
    np.testing.assert_array_equal(r["out"], r["x1"])


def _phi_cdf(z):
    return 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))


@pytest.mark.parametrize("keep", [0.0, 0.25, 1.0])
def test_block_forward_constant_attention_rows_closed_form(keep):
    """LN with gamma = 0 returns beta on every token.  With LN1 so and no
    depthwise branch acting (dw = 0), Q^ = Q, K^ = K, V^ = V are one row
    r = c1 W_qkv at every token; every head's linear path is then
    relu(q).N relu(k)^T v / relu(q).N relu(k) = v, and any window's softmax
    over identical keys is v while its linear estimate is v as well, so the
    residual vanishes and X1 = X + v W_o for every keep ratio (FT 3.3 and the
    FT 3.5 block equation).  LN2 keeps a non-trivial gamma, so swapping the
    two norms' parameters fails here."""
    wl, inp = _block_case(keep=keep)
    rng = _rng(77)
    C = wl.channels
    c1 = rng.standard_normal(C)
    inp = dict(inp, dw=[np.zeros_like(k) for k in inp["dw"]],
               ln1_g=np.zeros(C), ln1_b=c1,
               ln2_g=1.0 + 0.5 * rng.standard_normal(C), ln2_b=rng.standard_normal(C))
    # keep every head's relu(q).relu(k) away from 0 (a positive q and k)
    w = inp["w_qkv"].copy()
    w[:, :2 * C] = np.abs(w[:, :2 * C]) * np.sign(c1)[:, None]
    inp["w_qkv"] = w
    r = O.hsmla_block_forward(inp["x"], inp, **wl.kwargs())
    v = (c1 @ w)[2 * C:]
    np.testing.assert_allclose(r["x1"], inp["x"] + v @ inp["w_o"], rtol=0, atol=1e-10)


def test_block_forward_constant_ffn_rows_closed_form():
    """With LN2's gamma = 0 and beta = c2, h1 = u = c2 W1 at every token, and
    the zero-padded 3x3 cross-correlation at (y, x) is u times the sum S of
    the taps g[dy][dx] whose neighbour (y + dy - 1, x + dx - 1) lies in the
    grid: 4 taps at a corner, 6 on an edge, all 9 inside.  Then
    out = X1 + GELU(u * S(y, x)) W2 (the FFN-DWConv sandwich of the block).
    LN1 keeps a non-trivial gamma."""
    wl, inp = _block_case(keep=0.25)
    rng = _rng(78)
    C, gh, gw = wl.channels, wl.grid_h, wl.grid_w
    c2 = rng.standard_normal(C)
    inp = dict(inp, ln1_g=1.0 + 0.5 * rng.standard_normal(C),
               ln1_b=rng.standard_normal(C), ln2_g=np.zeros(C), ln2_b=c2)
    r = O.hsmla_block_forward(inp["x"], inp, **wl.kwargs())
    u = c2 @ inp["w1"]
    g = inp["dw_ffn"]  # [4C, 3, 3]
    for (y, x) in [(0, 0), (0, gw - 1), (gh - 1, 0), (gh - 1, gw - 1),
                   (0, 5), (7, 0), (gh - 1, 9), (4, gw - 1), (8, 8), (3, 11)]:
        rows = [dy for dy in range(3) if 0 <= y + dy - 1 < gh]
        cols = [dx for dx in range(3) if 0 <= x + dx - 1 < gw]
        edge_y, edge_x = y in (0, gh - 1), x in (0, gw - 1)
        assert len(rows) * len(cols) == (4 if edge_y and edge_x else
                                         6 if edge_y or edge_x else 9)
        S = sum(g[:, dy, dx] for dy in rows for dx in cols)
        h2 = np.array([z * _phi_cdf(z) for z in u * S])
        n = y * gw + x
        np.testing.assert_allclose(r["out"][0, n] - r["x1"][0, n], h2 @ inp["w2"],
                                   rtol=0, atol=1e-10)


def test_block_forward_zero_input_closed_form():
    """X = 0: LN1 returns beta1 on every token (zero variance), so with no
    depthwise branch acting the attention output is v = (beta1 W_qkv)_V on
    every token (as in the constant-rows case above) and X1 = a = v W_o, one
    row everywhere.  LN2 of that row is a library LayerNorm of a, h1 is
    u = LN2(a) W1 everywhere, and the zero-padded conv makes
    out = a + GELU(u * S(y, x)) W2 with S the in-grid tap sums.  Applying
    LN2 to X instead of X1, or dropping the first residual, fails here."""
    wl, inp = _block_case(keep=0.25)
    rng = _rng(79)
    C, gh, gw = wl.channels, wl.grid_h, wl.grid_w
    c1 = rng.standard_normal(C)
    g2, b2 = 1.0 + 0.5 * rng.standard_normal(C), rng.standard_normal(C)
    inp = dict(inp, x=np.zeros_like(inp["x"]),
               dw=[np.zeros_like(k) for k in inp["dw"]],
               ln1_g=1.0 + 0.5 * rng.standard_normal(C), ln1_b=c1, ln2_g=g2, ln2_b=b2)
    w = inp["w_qkv"].copy()
    w[:, :2 * C] = np.abs(w[:, :2 * C]) * np.sign(c1)[:, None]
    inp["w_qkv"] = w
    r = O.hsmla_block_forward(inp["x"], inp, **wl.kwargs())
    a = (c1 @ w)[2 * C:] @ inp["w_o"]
    np.testing.assert_allclose(r["x1"][0], np.tile(a, (gh * gw, 1)), rtol=0, atol=1e-10)
    z = torch.nn.functional.layer_norm(torch.from_numpy(a)[None], (C,),
                                       torch.from_numpy(g2), torch.from_numpy(b2),
                                       eps=1e-5).numpy()[0]
    u = z @ inp["w1"]
    g = inp["dw_ffn"]
    for (y, x) in [(0, 0), (gh - 1, gw - 1), (0, 6), (9, 0), (5, 7)]:
        rows = [dy for dy in range(3) if 0 <= y + dy - 1 < gh]
        cols = [dx for dx in range(3) if 0 <= x + dx - 1 < gw]
        S = sum(g[:, dy, dx] for dy in rows for dx in cols)
        h2 = np.array([q * _phi_cdf(q) for q in u * S])
        np.testing.assert_allclose(r["out"][0, y * gw + x], a + h2 @ inp["w2"],
                                   rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# threshold routing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_select_threshold_brute_force(seed):
    rng = _rng(300 + seed)
    scores = rng.integers(0, 6, size=(3, 23)) / 5.0
    for tau in (-1.0, 0.0, 0.2, 0.5, 0.6, 1.0, 2.0):
        sel, counts = O.select_threshold(scores, tau)
        for b in range(3):
            want = [t for t in range(23) if scores[b, t] > tau]  # strict
            assert counts[b] == len(want)
            assert sel[b, :counts[b]].tolist() == want
            assert np.all(sel[b, counts[b]:] == -1)


def test_threshold_between_kth_and_next_equals_topk():
    rng = _rng(310)
    scores = rng.random((4, 40))
    for k in (0, 1, 7, 39, 40):
        srt = np.sort(scores, axis=1)[:, ::-1]
        for b in range(4):
            hi = srt[b, k - 1] if k > 0 else 2.0
            lo = srt[b, k] if k < 40 else -1.0
            tau = 0.5 * (hi + lo)
            sel, counts = O.select_threshold(scores[b:b + 1], tau)
            assert counts[0] == k
            assert sel[0, :k].tolist() == O.select_blocks(scores[b:b + 1], k)[0].tolist()


def test_threshold_module_matches_topk_module():
    """A threshold placed between the k-th and (k+1)-th score routes the same
    blocks as top-k, so the module outputs agree exactly."""
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    ref = O.hsmla_forward(inp["x"], inp, **wl.kwargs())
    s = np.sort(ref["scores"].astype(np.float32)[0])[::-1]
    k = wl.keep_blocks
    tau = float(0.5 * (np.float64(s[k - 1]) + np.float64(s[k])))
    thr = O.hsmla_forward(inp["x"], inp, tau=tau, **wl.kwargs())
    assert thr["counts"][0] == k
    np.testing.assert_array_equal(thr["sel"][0, :k], ref["sel"][0])
    np.testing.assert_array_equal(thr["y"], ref["y"])


# ---------------------------------------------------------------------------
# per-head routing
# ---------------------------------------------------------------------------

def test_head_scores_zero_weights_are_sigmoid_of_each_bias():
    rng = _rng(21)
    H, d = 3, 2
    qkvh = rng.standard_normal((1, 4 * 4, 3 * H * d))
    b = np.array([0.0, math.log(3.0), -math.log(3.0)])
    g = O.gate_head_scores(qkvh, np.zeros((H, 3 * d)), b, 4, 4, 2, H)
    np.testing.assert_allclose(g, np.broadcast_to([0.5, 0.75, 0.25], g.shape),
                               rtol=0, atol=1e-15)


def test_head_scores_one_hot_weight_picks_that_head():
    H, d, Bs, gh, gw = 2, 2, 2, 4, 6
    C = H * d
    T = (gh // Bs) * (gw // Bs)
    vals = np.arange(T) * 0.1 - 0.2
    qkvh = np.zeros((1, gh * gw, 3 * C))
    for n in range(gh * gw):
        y, x = divmod(n, gw)
        qkvh[0, n, 2 * C + 1 * d + 0] = vals[(y // Bs) * (gw // Bs) + x // Bs]  # v_0 of head 1
    w = np.zeros((H, 3 * d)); w[1, 2 * d + 0] = 1.0
    g = O.gate_head_scores(qkvh, w, np.zeros(H), gh, gw, Bs, H)
    np.testing.assert_allclose(g[0, :, 0], 0.5, atol=1e-15)
    np.testing.assert_allclose(g[0, :, 1], 1.0 / (1.0 + np.exp(-vals)), atol=1e-15)


def test_head_scores_mean_matches_gate_fixture():
    fx = _load("gate_2x4.json")
    g = O.gate_head_scores(np.array(fx["qkv_hat"]), np.array(fx["gate_w"]),
                           np.array(fx["gate_b"]), grid_h=2, grid_w=4, block=2, heads=2)
    np.testing.assert_allclose(g.mean(axis=-1)[0], fx["expected"]["scores"], atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_select_threshold_per_head_brute_force(seed):
    rng = _rng(40 + seed)
    B, T, H = 2, 9, 3
    g = rng.integers(0, 4, size=(B, T, H)) / 4.0
    tau = 0.5
    sel, cnt = O.select_threshold_per_head(g, tau)
    for b in range(B):
        for h in range(H):
            want = [t for t in range(T) if g[b, t, h] > tau]
            assert cnt[b, h] == len(want)
            assert sel[b, h, :cnt[b, h]].tolist() == want
            assert np.all(sel[b, h, cnt[b, h]:] == -1)


def _small_module_case(seed=3, heads=3):
    wl = scaled(WORKLOADS["tiny"], name="ph", grid_h=8, grid_w=12, channels=32 * heads,
                heads=heads, block=4, window=8, seed=seed)
    return wl, make_inputs(wl)


def test_refine_per_head_with_equal_lists_equals_refine_selected():
    wl, inp = _small_module_case()
    r = O.hsmla_module(inp["x"], inp, **wl.kwargs())
    T = wl.num_blocks
    lst = np.array([[0, 2, 5, -1, -1]])
    same = np.repeat(lst[:, None, :], wl.heads, axis=1)
    a = O.refine_per_head(r["qkv"], r["qkv_hat"], r["o_lin"], same, wl.grid_h, wl.grid_w,
                          wl.heads, wl.block, wl.window)
    b = O.refine_selected(r["qkv"], r["qkv_hat"], r["o_lin"], lst, wl.grid_h, wl.grid_w,
                          wl.heads, wl.block, wl.window)
    assert T > 5
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_refine_per_head_changes_only_the_routed_head():
    """Head 1 routed on blocks {1, 4}, the others on nothing: only head 1's
    channels of those blocks' tokens move, by what the all-head refinement
    of the same blocks gives on head 1."""
    wl, inp = _small_module_case()
    r = O.hsmla_module(inp["x"], inp, **wl.kwargs())
    H, d = wl.heads, wl.head_dim
    lists = np.full((1, H, 2), -1)
    lists[0, 1] = [1, 4]
    got = O.refine_per_head(r["qkv"], r["qkv_hat"], r["o_lin"], lists, wl.grid_h,
                            wl.grid_w, H, wl.block, wl.window)
    full = O.refine_selected(r["qkv"], r["qkv_hat"], r["o_lin"], np.array([[1, 4]]),
                             wl.grid_h, wl.grid_w, H, wl.block, wl.window)
    want = np.array(r["o_lin"], copy=True)
    want[..., d:2 * d] = full[..., d:2 * d]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert not np.allclose(want[..., d:2 * d], r["o_lin"][..., d:2 * d])


def test_per_head_routing_with_equal_heads_equals_threshold_routing():
    """Heads made identical (the projection columns and depthwise kernels of
    every head copied from head 0, the same gate weights and bias) give
    G^(h) = M, so per-head routing must reproduce block routing by M > tau."""
    wl, inp = _small_module_case(seed=5)
    inp = dict(inp)
    C, d = wl.channels, wl.head_dim
    w_qkv = np.array(inp["w_qkv"], copy=True)
    dws = [np.array(w, copy=True) for w in inp["dw"]]
    for s in range(3):
        for h in range(1, wl.heads):
            w_qkv[:, s * C + h * d:s * C + (h + 1) * d] = w_qkv[:, s * C:s * C + d]
            for w in dws:
                w[s * C + h * d:s * C + (h + 1) * d] = w[s * C:s * C + d]
    inp.update(w_qkv=w_qkv, dw=dws,
               gate_w=np.repeat(inp["gate_w"][:1], wl.heads, axis=0),
               gate_b=np.full(wl.heads, 0.1))
    blk = O.hsmla_module(inp["x"], inp, **wl.kwargs())
    tau = float(np.median(blk["scores"]))
    a = O.hsmla_module(inp["x"], inp, tau=tau, **wl.kwargs())
    p = O.hsmla_module(inp["x"], inp, tau=tau, per_head=True, **wl.kwargs())
    for h in range(wl.heads):
        np.testing.assert_array_equal(p["sel"][:, h], a["sel"])
        np.testing.assert_array_equal(p["counts"][:, h], a["counts"])
    assert 0 < a["counts"].sum() < wl.num_blocks * wl.batch
    np.testing.assert_allclose(p["o"], a["o"], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# training-time soft mixture
# ---------------------------------------------------------------------------

def test_soft_mixture_unit_weights_equal_refining_every_block():
    wl, inp = _small_module_case(seed=7, heads=2)
    r = O.hsmla_module(inp["x"], inp, **wl.kwargs())
    T = wl.num_blocks
    allb = np.tile(np.arange(T), (wl.batch, 1))
    hard = O.refine_selected(r["qkv"], r["qkv_hat"], r["o_lin"], allb, wl.grid_h,
                             wl.grid_w, wl.heads, wl.block, wl.window)
    ones = O.refine_selected(r["qkv"], r["qkv_hat"], r["o_lin"], allb, wl.grid_h,
                             wl.grid_w, wl.heads, wl.block, wl.window,
                             weights=np.ones((wl.batch, T)))
    zeros = O.refine_selected(r["qkv"], r["qkv_hat"], r["o_lin"], allb, wl.grid_h,
                              wl.grid_w, wl.heads, wl.block, wl.window,
                              weights=np.zeros((wl.batch, T)))
    np.testing.assert_allclose(ones, hard, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(zeros, r["o_lin"], rtol=0, atol=0)


def test_soft_mixture_moves_each_block_along_its_own_residual():
    """Block t's tokens end at O_lin + w_t (hard - O_lin): the weight scales
    only the residual, block by block (checked against the hard result)."""
    wl, inp = _small_module_case(seed=8, heads=2)
    r = O.hsmla_module(inp["x"], inp, **wl.kwargs())
    T = wl.num_blocks
    allb = np.tile(np.arange(T), (wl.batch, 1))
    w = _rng(3).uniform(0, 1, size=(wl.batch, T))
    hard = O.refine_selected(r["qkv"], r["qkv_hat"], r["o_lin"], allb, wl.grid_h,
                             wl.grid_w, wl.heads, wl.block, wl.window)
    soft = O.refine_selected(r["qkv"], r["qkv_hat"], r["o_lin"], allb, wl.grid_h,
                             wl.grid_w, wl.heads, wl.block, wl.window, weights=w)
    nbc = wl.grid_w // wl.block
    ys, xs = np.divmod(np.arange(wl.tokens), wl.grid_w)
    tblk = (ys // wl.block) * nbc + xs // wl.block
    want = r["o_lin"] + w[:, tblk][..., None] * (hard - r["o_lin"])
    np.testing.assert_allclose(soft, want, rtol=1e-12, atol=1e-12)


def test_soft_module_uses_the_block_scores_as_weights():
    wl, inp = _small_module_case(seed=9, heads=2)
    s = O.hsmla_module(inp["x"], inp, soft=True, **wl.kwargs())
    T = wl.num_blocks
    allb = np.tile(np.arange(T), (wl.batch, 1))
    want = O.refine_selected(s["qkv"], s["qkv_hat"], s["o_lin"], allb, wl.grid_h,
                             wl.grid_w, wl.heads, wl.block, wl.window,
                             weights=s["scores"].astype(np.float32).astype(np.float64))
    np.testing.assert_allclose(s["o"], want, rtol=0, atol=0)
    assert np.all((s["scores"] > 0) & (s["scores"] < 1))
