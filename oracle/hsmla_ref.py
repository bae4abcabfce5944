"""HSMLA forward pass, float64 NumPy reference (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. Nothing here is on the product path.

Citations use the legend of the package docstring: FT is the paper's full
text (paperpeel.com rendering of "HSMLA: Hierarchical Softmax Multi-scale
Linear Attention for Efficient Vision Transformers"), EX is the gist.science
explainer of the same paper (section "Technische Samenvatting").

Layout conventions (shared with the library only as a documented data
format, not as code):

* A token grid of grid_h x grid_w tokens is flattened row-major: token
  n = y * grid_w + x.  Activations are [B, N, C] float64 arrays.
* The projected tensor QKV is [B, N, 3C]; channel s*C + h*d + j holds
  component s (0=Q, 1=K, 2=V) of head h, feature j.
* Blocks are Bs x Bs token tiles numbered row-major over the block grid:
  t = (y // Bs) * (grid_w // Bs) + (x // Bs).
* Weights are [in, out] and used as x @ W.  Depthwise kernels are
  [channels, k, k] and applied as a cross-correlation.

Every floating-point step runs in float64.  With ``staged=True`` the values
the GPU path stores in bfloat16 are rounded to bfloat16 at exactly those
points (see ``round_bf16``); everything else (Z, D, gate scores, all sums)
stays float64.

Parity status per function is given in its docstring.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf  # library primitive (exact GELU)

__all__ = [
    "round_bf16",
    "relu",
    "qkv_projection",
    "dwconv_same",
    "multiscale_branches",
    "kv_state",
    "linear_readout",
    "linear_attention",
    "block_features",
    "gate_scores",
    "gate_head_scores",
    "select_blocks",
    "select_threshold",
    "select_threshold_per_head",
    "refine_per_head",
    "window_bounds",
    "refine_selected",
    "hsmla_module",
    "hsmla_forward",
    "layer_norm",
    "gelu",
    "hsmla_block_forward",
]


# ---------------------------------------------------------------------------
# number format
# ---------------------------------------------------------------------------

_BF16_SIG_BITS = 8  # 1 implicit + 7 stored significand bits
_BF16_MIN_EXP = -133  # spacing of bfloat16 subnormals is 2**-133
_BF16_OVERFLOW = 2.0 ** 128


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps the float32 exponent range with an 8-bit significand.
    The value is rounded directly from float64 (no intermediate float32),
    which is the definition of round-to-nearest-even for that format.
    Returns float64 arrays holding bfloat16-representable values.

    Pinned by: agreement with torch's float32->bfloat16 conversion on values
    that are exact in float32, hand-built tie cases, overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0.0)
    if np.any(fin):
        xv = x[fin]
        _, e = np.frexp(xv)  # xv = m * 2**e, 0.5 <= |m| < 1
        q = np.maximum(e - _BF16_SIG_BITS, _BF16_MIN_EXP)
        r = np.ldexp(np.rint(np.ldexp(xv, -q)), q)  # rint rounds half to even
        r = np.where(np.abs(r) >= _BF16_OVERFLOW, np.copysign(np.inf, r), r)
        out[fin] = r
    return out


def _identity(x):
    return x


# ---------------------------------------------------------------------------
# step 1: projection
# ---------------------------------------------------------------------------

def relu(x):
    """The feature map phi of the linear path: elementwise max(x, 0).

    FT 3.1 (phi of the hatted keys/queries) with the abstract's
    "ReLU-based linear attention".  Pinned by the brute-force linear
    attention test (a different phi breaks it).
    """
    return np.maximum(x, 0.0)


def qkv_projection(x, w_qkv):
    """Q, K, V = LinearProjection(X) for all heads at once (FT 3.1, first
    display equation).  No bias.  x: [B, N, C], w_qkv: [C, 3C].

    Pinned by: a textbook matmul written as explicit sums on a tiny case.
    """
    return np.asarray(x, np.float64) @ np.asarray(w_qkv, np.float64)


# ---------------------------------------------------------------------------
# step 2: multi-scale depthwise branches
# ---------------------------------------------------------------------------

def dwconv_same(t, w, grid_h, grid_w):
    """Depthwise 2-D cross-correlation with zero "same" padding, no bias.

    t: [B, N, Ch] tokens on a grid_h x grid_w grid; w: [Ch, k, k], k odd.
    out[y, x, c] = sum_{dy, dx} w[c, dy, dx] * t[y + dy - r, x + dx - r, c],
    r = (k - 1) // 2, with t = 0 outside the grid.

    The depthwise convolutions are the multi-scale token branches of the
    abstract and of EX section 2 (kernel sizes 3, 5, 7).
    Pinned by: torch.nn.functional.conv2d(groups=Ch) on the CPU, and a delta
    kernel giving the identity.
    """
    t = np.asarray(t, np.float64)
    w = np.asarray(w, np.float64)
    B, N, Ch = t.shape
    k = w.shape[-1]
    assert w.shape == (Ch, k, k) and k % 2 == 1 and N == grid_h * grid_w
    r = (k - 1) // 2
    img = t.reshape(B, grid_h, grid_w, Ch)
    pad = np.zeros((B, grid_h + 2 * r, grid_w + 2 * r, Ch))
    pad[:, r:r + grid_h, r:r + grid_w, :] = img
    out = np.zeros_like(img)
    for dy in range(k):
        for dx in range(k):
            out += w[:, dy, dx] * pad[:, dy:dy + grid_h, dx:dx + grid_w, :]
    return out.reshape(B, N, Ch)


def multiscale_branches(t, kernels, grid_h, grid_w):
    """T_hat = T + sum_s DWConv_{k_s}(T), per channel of Q, K and V.

    The identity ("single-scale") branch plus one depthwise branch per kernel
    size, summed so that each head keeps width d.  The prose defining the
    hatted tensors is missing from FT 3.1; this is the reading taken from
    the abstract ("multi-scale token representations via depthwise
    convolutions") and EX section 2 (tokens "enriched" by depthwise
    convolutions of sizes 3, 5, 7), chosen because it keeps H heads of width
    d and the C x C output projection.

    Pinned by: delta kernels (each branch an identity) give (1 + S) * T.
    The sum-of-branches combination itself is parity unpinned by the pages.
    """
    out = np.array(t, np.float64, copy=True)
    for w in kernels:
        out = out + dwconv_same(t, w, grid_h, grid_w)
    return out


# ---------------------------------------------------------------------------
# step 3: global ReLU linear attention
# ---------------------------------------------------------------------------

def _heads(t, heads):
    B, N, C = t.shape
    return t.reshape(B, N, heads, C // heads)


def kv_state(k_hat, v_hat, heads):
    """Z = sum_j phi(K_hat_j)^T V_hat_j and D = sum_j phi(K_hat_j) per
    (image, head) (FT 3.1, Z/D sums).

    k_hat, v_hat: [B, N, C].  Returns Z [B, H, d, d] (row index = key
    feature, column index = value feature) and D [B, H, d].
    Pinned by: the brute-force O(N^2) linear attention test.
    """
    fk = relu(_heads(np.asarray(k_hat, np.float64), heads))
    vh = _heads(np.asarray(v_hat, np.float64), heads)
    Z = np.einsum("bnhi,bnhj->bhij", fk, vh)
    D = fk.sum(axis=1)
    return Z, D


def _guarded_ratio(num, den):
    """num / den with 0/0 := 0.  With phi = ReLU every term of den is >= 0,
    so den == 0 forces every term of num to zero as well."""
    den_b = den[..., None]
    safe = np.where(den_b > 0.0, den_b, 1.0)
    return np.where(den_b > 0.0, num / safe, 0.0)


def linear_readout(q_hat, Z, D, heads):
    """O_lin_i = phi(Q_hat_i) Z / (phi(Q_hat_i) . D), per head.

    FT 3.3 gives this ratio for a neighbourhood N(i) (lin-local equation);
    the global output is the same ratio with N(i) = all tokens, which is the
    associativity argument of EX section 2.  No epsilon appears in the
    pages, so a zero denominator yields 0 (see _guarded_ratio).
    q_hat: [B, N, C]; returns [B, N, C].
    Pinned by: brute-force O(N^2) form; invariance under a positive scalar on
    Q_hat or K_hat; all-negative queries give exactly 0.
    """
    fq = relu(_heads(np.asarray(q_hat, np.float64), heads))
    num = np.einsum("bnhi,bhij->bnhj", fq, Z)
    den = np.einsum("bnhi,bhi->bnh", fq, D)
    out = _guarded_ratio(num, den)
    B, N, H, d = out.shape
    return out.reshape(B, N, H * d)


def linear_attention(qkv_hat, heads):
    """Global path of the module: returns (O_lin [B,N,C], Z, D)."""
    qkv_hat = np.asarray(qkv_hat, np.float64)
    C = qkv_hat.shape[-1] // 3
    Z, D = kv_state(qkv_hat[..., C:2 * C], qkv_hat[..., 2 * C:], heads)
    return linear_readout(qkv_hat[..., :C], Z, D, heads), Z, D


# ---------------------------------------------------------------------------
# step 4: block gate and selection
# ---------------------------------------------------------------------------

def block_features(qkv_hat, grid_h, grid_w, block, heads):
    """f_t^(h): mean over the Bs*Bs tokens of block t of the concatenation
    [Q_hat^(h); K_hat^(h); V_hat^(h)] (3d values per head).

    Returns [B, T, H, 3d] with the q features first, then k, then v.
    FT 3.2 (head-level score equation, the AvgPool of the block's hatted
    tokens).  The depthwise 3x3 inside that equation, when used, is applied
    by gate_scores before this pooling.
    """
    x = np.asarray(qkv_hat, np.float64)
    B, N, C3 = x.shape
    d = C3 // 3 // heads
    nbr, nbc = grid_h // block, grid_w // block
    img = x.reshape(B, nbr, block, nbc, block, 3, heads, d)
    f = img.mean(axis=(2, 4))  # [B, nbr, nbc, 3, H, d]
    f = np.moveaxis(f, 3, 4)  # [B, nbr, nbc, H, 3, d]
    return f.reshape(B, nbr * nbc, heads, 3 * d)


def gate_scores(qkv_hat, gate_w, gate_b, grid_h, grid_w, block, heads,
                gate_dw=None):
    """M_t = (1/H) sum_h sigmoid(w^(h) . f_t^(h) + b^(h)), shared by all heads.

    FT 3.2: head-level scores G_b^(h) and their mean M_b in [0, 1] (only the
    first equality of the block-level aggregation equation is used; its
    second equality is not consistent with the first).  EX section 2 says
    the aggregated gate is shared.  gate_w: [H, 3d], gate_b: [H].

    gate_dw: None, or [3C, 3, 3] depthwise weights.  When given, the head
    score follows FT 3.2's equation in full: f_t^(h) is the block average of
    DWConv3x3([Q_hat; K_hat; V_hat]), the convolution taken over the whole
    token grid with zero padding at the image border (the reading of
    "DWConv of the block's tokens" in which neighbouring blocks supply the
    halo, as for every other convolution of the module), no bias.  When
    None, the block average of the hatted tokens themselves.
    Returns M: [B, T] float64.
    Pinned by hand-worked fixtures, the w = 0 case (every score equals the
    mean of sigmoid(b)), a delta gate kernel (equal to no kernel), loops
    over the definition on tiny inputs, and a constant field with a ones
    kernel (closed form at border and interior blocks).
    """
    g = gate_head_scores(qkv_hat, gate_w, gate_b, grid_h, grid_w, block, heads,
                         gate_dw=gate_dw)
    return g.mean(axis=-1)


def gate_head_scores(qkv_hat, gate_w, gate_b, grid_h, grid_w, block, heads,
                     gate_dw=None):
    """G_b^(h) = sigmoid(w^(h) . f_b^(h) + b^(h)) for every block and head
    (FT 3.2 head-level score; the features as described in gate_scores).
    Returns [B, T, H] float64; gate_scores is its mean over heads.
    Pinned by: zero weights (G^(h) = sigmoid(b^(h)) head by head), one-hot
    weights on a block-constant feature, and the head mean equal to the
    hand-worked scores fixture.
    """
    if gate_dw is not None:
        qkv_hat = dwconv_same(qkv_hat, gate_dw, grid_h, grid_w)
    f = block_features(qkv_hat, grid_h, grid_w, block, heads)
    w = np.asarray(gate_w, np.float64)
    b = np.asarray(gate_b, np.float64)
    logit = np.einsum("bthf,hf->bth", f, w) + b
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-logit))


def select_blocks(scores, keep_blocks):
    """Indices of the keep_blocks highest scores per image, ascending.

    Ranking is by score, descending; equal scores go to the lower block
    index, which makes the set unique.  The pages route by a threshold tau
    (FT 3.2, the alpha equation); a fixed count is taken here so that the
    number of refined blocks is known before any kernel runs.
    scores: [B, T]; returns int64 [B, keep_blocks].
    Pinned by: exhaustive search over all subsets on tiny inputs, with ties.
    """
    s = np.asarray(scores)
    B, T = s.shape
    k = int(keep_blocks)
    assert 0 <= k <= T
    out = np.zeros((B, k), dtype=np.int64)
    idx = np.arange(T)
    for bi in range(B):
        order = np.lexsort((idx, -s[bi]))  # primary: -score, then index
        out[bi] = np.sort(order[:k])
    return out


def select_threshold(scores, tau):
    """Blocks whose score exceeds tau, per image, ascending (FT 3.2, the
    alpha equation: the routed set is {b : M_b > tau}, a strict inequality).

    scores: [B, T].  Returns (sel [B, T] int64 padded with -1, counts [B]).
    Pinned by: a brute-force membership loop, and agreement with
    select_blocks when tau lies strictly between the k-th and (k+1)-th score.
    """
    s = np.asarray(scores)
    B, T = s.shape
    sel = np.full((B, T), -1, dtype=np.int64)
    counts = np.zeros(B, dtype=np.int64)
    for bi in range(B):
        idx = np.nonzero(s[bi] > tau)[0]
        counts[bi] = idx.size
        sel[bi, :idx.size] = idx
    return sel, counts


# ---------------------------------------------------------------------------
# step 5: local softmax refinement of the selected blocks
# ---------------------------------------------------------------------------

def select_threshold_per_head(head_scores, tau):
    """Per-head routed sets {b : G_b^(h) > tau} (FT 3.2 per-head output
    routing equation), ascending.  head_scores: [B, T, H].  Returns
    (sel [B, H, T] int64 padded with -1, counts [B, H]).
    Pinned by: brute-force membership, and equality with select_threshold
    when every head has the same scores.
    """
    g = np.asarray(head_scores)
    B, T, H = g.shape
    sel, counts = select_threshold(np.moveaxis(g, 2, 1).reshape(B * H, T), tau)
    return sel.reshape(B, H, T), counts.reshape(B, H)


def window_bounds(t, grid_h, grid_w, block, window):
    """Token rows/cols [r_lo, r_hi) x [c_lo, c_hi) of the softmax window of
    block t: a window x window square centred on the block, clipped to the
    grid (no padding keys).  Requires (window - block) even.

    The neighbourhood N(i) of FT 3.3 (local-neighbourhood equation) and the
    w x w window of EX section 2; block-centred so that all queries of a
    block share one window.
    """
    assert (window - block) % 2 == 0 and window >= block
    p = (window - block) // 2
    nbc = grid_w // block
    r0 = (t // nbc) * block
    c0 = (t % nbc) * block
    return (max(0, r0 - p), min(grid_h, r0 + block + p),
            max(0, c0 - p), min(grid_w, c0 + block + p))


def _tokens(r_lo, r_hi, c_lo, c_hi, grid_w):
    ys, xs = np.meshgrid(np.arange(r_lo, r_hi), np.arange(c_lo, c_hi),
                         indexing="ij")
    return (ys * grid_w + xs).reshape(-1)


def refine_selected(qkv, qkv_hat, o_lin, sel, grid_h, grid_w, heads, block,
                    window, rnd=_identity, weights=None):
    """O_i = O_lin_i + O_local_i - O_linloc_i for every token i of every
    selected block, every head; all other tokens keep O_lin_i.

    * O_local_i = softmax_j(q_i . k_j / sqrt(d)) over the window keys, times
      v_j, with the raw (un-hatted) Q, K, V (FT 3.3, local-neighbourhood
      equation).  The scale 1/sqrt(d) is not stated and is the usual one.
    * O_linloc_i = phi(q_hat_i) Z_W / (phi(q_hat_i) . D_W), Z_W and D_W
      being the Z/D sums restricted to the window (FT 3.3, lin-local
      equation), with the same zero-denominator guard as the global path.
    * The sum is the two-path residual of FT 3.3 with R_i = O_local -
      O_linloc on selected tokens and 0 elsewhere (EX section 2 defines R_i).

    Pinned by: keep 0 (identity), keep all with a window covering the grid
    (full softmax attention, torch's reference SDPA on the CPU), and keep
    all with window = block (block-diagonal masked attention built
    independently).  ``rnd`` rounds the result (staged bfloat16 mode).

    ``weights`` [B, T] (optional) scales the residual of block t by
    weights[b, t]: O_i = O_lin_i + w (O_local_i - O_linloc_i), the
    training-time differentiable mixture of FT 3.3 with w = M_b.  Pinned
    by w = 1 (the hard routing), w = 0 (the linear path) and per-block
    weights moving each block along its own residual.
    """
    qkv = np.asarray(qkv, np.float64)
    qkv_hat = np.asarray(qkv_hat, np.float64)
    out = np.array(o_lin, np.float64, copy=True)
    B, N, C3 = qkv.shape
    C = C3 // 3
    d = C // heads
    scale = 1.0 / math.sqrt(d)
    for bi in range(B):
        for t in np.asarray(sel[bi]).tolist():
            if t < 0:  # padding of a thresholded selection
                continue
            nbc = grid_w // block
            r0, c0 = (t // nbc) * block, (t % nbc) * block
            qi = _tokens(r0, r0 + block, c0, c0 + block, grid_w)
            wi = _tokens(*window_bounds(t, grid_h, grid_w, block, window),
                         grid_w)
            nq, nk = qi.size, wi.size
            q = qkv[bi, qi, 0:C].reshape(nq, heads, d)
            k = qkv[bi, wi, C:2 * C].reshape(nk, heads, d)
            v = qkv[bi, wi, 2 * C:].reshape(nk, heads, d)
            s = np.einsum("qhd,khd->hqk", q, k) * scale
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            o_local = np.einsum("hqk,khd->qhd", p, v)

            fq = relu(qkv_hat[bi, qi, 0:C].reshape(nq, heads, d))
            fk = relu(qkv_hat[bi, wi, C:2 * C].reshape(nk, heads, d))
            vh = qkv_hat[bi, wi, 2 * C:].reshape(nk, heads, d)
            Zw = np.einsum("khi,khj->hij", fk, vh)
            Dw = fk.sum(axis=0)
            num = np.einsum("qhi,hij->qhj", fq, Zw)
            den = np.einsum("qhi,hi->qh", fq, Dw)
            o_linloc = _guarded_ratio(num, den)

            base = out[bi, qi].reshape(nq, heads, d)
            if weights is None:
                out[bi, qi] = rnd((base + o_local - o_linloc).reshape(nq, C))
            else:
                w = float(np.asarray(weights)[bi, t])
                out[bi, qi] = rnd((base + w * (o_local - o_linloc)).reshape(nq, C))
    return out


def _head_channels(C, heads, h):
    """Channel indices of head h's q, k and v inside [Q; K; V] (3C wide)."""
    d = C // heads
    return np.concatenate([np.arange(s * C + h * d, s * C + (h + 1) * d)
                           for s in range(3)])


def refine_per_head(qkv, qkv_hat, o_lin, sel_heads, grid_h, grid_w, heads,
                    block, window, rnd=_identity):
    """Per-head routing (FT 3.2 per-head output routing equation): head h of
    the tokens of block b gets the two-path residual when b is in head h's
    list, and keeps the linear output otherwise.  Each head's refinement is
    the single-head case of refine_selected on that head's q, k, v channels.
    sel_heads: [B, H, L] block indices per head, entries < 0 ignored.
    Pinned by: with equal lists for every head it equals refine_selected.
    """
    qkv = np.asarray(qkv, np.float64)
    qkv_hat = np.asarray(qkv_hat, np.float64)
    out = np.array(o_lin, np.float64, copy=True)
    C = out.shape[-1]
    d = C // heads
    for h in range(heads):
        ch = _head_channels(C, heads, h)
        out[..., h * d:(h + 1) * d] = refine_selected(
            qkv[..., ch], qkv_hat[..., ch], out[..., h * d:(h + 1) * d],
            np.asarray(sel_heads)[:, h, :], grid_h, grid_w, 1, block, window,
            rnd=rnd)
    return out


# ---------------------------------------------------------------------------
# composition
# ---------------------------------------------------------------------------

def hsmla_module(x, weights, *, grid_h, grid_w, heads, block, window,
                 keep_blocks, staged=False, sel=None, scores_f32=True,
                 tau=None, per_head=False, soft=False):
    """Steps 1-5 of the module (everything before the output projection).

    Follows the five inference stages FT 3.6 lists: global linear path,
    gating, compaction (the index list), local softmax, and the residual
    write-back.  Returns a dict of every intermediate:
    qkv, qkv_hat, Z, D, o_lin, scores, sel, o.

    ``sel`` injects a selection (used when a GPU run picks a different block
    inside a near-tie band).  ``scores_f32`` ranks the float64 scores after
    rounding them to float32, the precision the GPU ranks in.  With ``tau``
    set, blocks are routed by the threshold M_t > tau instead of the top
    keep_blocks; ``sel`` is then padded with -1 and "counts" is returned.
    With ``per_head`` (and ``tau``) each head routes by its own score
    G_b^(h) > tau: "head_scores" [B, T, H], "sel" [B, H, T] and "counts"
    [B, H] are returned, and an injected ``sel`` has that shape.
    With ``soft`` every block is refined and its residual is scaled by its
    score M_b (FT 3.3 training-time differentiable mixture, forward only;
    the scores enter as float32 when ``scores_f32``).
    """
    rnd = round_bf16 if staged else _identity
    C = x.shape[-1]
    qkv = rnd(qkv_projection(x, weights["w_qkv"]))
    qkv_hat = rnd(multiscale_branches(qkv, weights["dw"], grid_h, grid_w))
    o_lin_raw, Z, D = linear_attention(qkv_hat, heads)
    o_lin = rnd(o_lin_raw)
    scores = gate_scores(qkv_hat, weights["gate_w"], weights["gate_b"],
                         grid_h, grid_w, block, heads,
                         gate_dw=weights.get("gate_dw"))
    counts = None
    head_scores = None
    rank_on = scores.astype(np.float32) if scores_f32 else scores
    thr = (np.float32(tau) if scores_f32 else tau) if tau is not None else None
    if soft:
        T = scores.shape[1]
        sel = np.tile(np.arange(T), (scores.shape[0], 1))
        o = refine_selected(qkv, qkv_hat, o_lin, sel, grid_h, grid_w, heads,
                            block, window, rnd=rnd,
                            weights=rank_on.astype(np.float64))
    elif per_head:
        assert tau is not None or sel is not None
        head_scores = gate_head_scores(qkv_hat, weights["gate_w"], weights["gate_b"],
                                       grid_h, grid_w, block, heads,
                                       gate_dw=weights.get("gate_dw"))
        if sel is None:
            hs = head_scores.astype(np.float32) if scores_f32 else head_scores
            sel, counts = select_threshold_per_head(hs, thr)
        o = refine_per_head(qkv, qkv_hat, o_lin, sel, grid_h, grid_w, heads,
                            block, window, rnd=rnd)
    else:
        if sel is None and tau is not None:
            sel, counts = select_threshold(rank_on, thr)
        elif sel is None:
            sel = select_blocks(rank_on, keep_blocks)
        o = refine_selected(qkv, qkv_hat, o_lin, sel, grid_h, grid_w, heads,
                            block, window, rnd=rnd)
    assert o.shape[-1] == C
    return dict(qkv=qkv, qkv_hat=qkv_hat, Z=Z, D=D, o_lin=o_lin,
                scores=scores, sel=np.asarray(sel), o=o, counts=counts,
                head_scores=head_scores)


def hsmla_forward(x, weights, *, staged=False, **kw):
    """HSMLA(X) = O W_o (the module returns C channels, FT 3.5 block
    equation).  Returns the module intermediates plus "y"."""
    rnd = round_bf16 if staged else _identity
    r = hsmla_module(np.asarray(x, np.float64), weights, staged=staged, **kw)
    r["y"] = rnd(r["o"] @ np.asarray(weights["w_o"], np.float64))
    return r


def layer_norm(x, gamma, beta, eps=1e-5):
    """LayerNorm over channels, biased variance, eps 1e-5 (not stated in the
    pages; the usual definition).  Pinned by torch's layer_norm on CPU."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def gelu(x):
    """Exact GELU, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)).  Pinned by
    torch's gelu (approximate='none') on CPU."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def hsmla_block_forward(x, weights, *, staged=False, **kw):
    """One HSMLA block (FT 3.5 block equation) with its DWConv and FFN steps
    fused into one FFN-DWConv sandwich:

        X1 = X + HSMLA(LN1(X))
        X2 = X1 + W2 GELU(DWConv3x3(W1 LN2(X1)))

    LN gamma/beta come from ``weights``; no biases elsewhere.  In staged mode
    the residual sums are rounded once, after the add, as the GPU stores
    them.  Returns the module intermediates plus xn1, x1, xn2, h1, h2, out.

    Pinned by closed forms of the composition: W2 = 0 or a zero FFN kernel
    leave out = X1; constant LN rows (gamma = 0) give X1 = X + v W_o and
    out = X1 + GELU(u * S) W2 with S the in-grid tap sums; X = 0 pins LN2's
    input as X1 against a library LayerNorm.
    """
    rnd = round_bf16 if staged else _identity
    x = np.asarray(x, np.float64)
    grid_h, grid_w = kw["grid_h"], kw["grid_w"]
    xn1 = rnd(layer_norm(x, weights["ln1_g"], weights["ln1_b"]))
    r = hsmla_module(xn1, weights, staged=staged, **kw)
    x1 = rnd(x + r["o"] @ np.asarray(weights["w_o"], np.float64))
    xn2 = rnd(layer_norm(x1, weights["ln2_g"], weights["ln2_b"]))
    h1 = rnd(xn2 @ np.asarray(weights["w1"], np.float64))
    h2 = rnd(gelu(dwconv_same(h1, weights["dw_ffn"], grid_h, grid_w)))
    out = rnd(x1 + h2 @ np.asarray(weights["w2"], np.float64))
    r.update(xn1=xn1, x1=x1, xn2=xn2, h1=h1, h2=h2, out=out)
    return r
