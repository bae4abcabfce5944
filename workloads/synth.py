"""Workload table and seeded input generators.

Inputs are drawn in float64 with numpy's default_rng(seed) in a fixed order
(X, W_qkv, W_o, depthwise kernels, gate weights, then the block's extra
weights) and rounded once to the run dtype, so the oracle and the GPU see
identical bits.  "N(m, v)" below means mean m, *variance* v.

The spatial structure of X stands in for the paper's benchmark data (which is
not used): a street scene with smooth low-frequency content, a CT slice with
a few elliptical organs on a quiet background, a pathology tile with
clustered foreground, and plain Gaussian noise for the tiny case.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "keep_blocks_for", "make_inputs", "scaled"]


def keep_blocks_for(ratio: float, num_blocks: int) -> int:
    """Number of kept blocks for a keep ratio: ceil(ratio * T), clamped to
    [0, T] (a tiny slack keeps exact products such as 0.25 * 16 at 4)."""
    k = math.ceil(ratio * num_blocks - 1e-9)
    return max(0, min(num_blocks, k))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    grid_h: int
    grid_w: int
    channels: int
    heads: int
    dtype: str  # "f32" or "bf16"
    branches: tuple  # odd depthwise kernel sizes added to the identity
    block: int
    window: int
    keep: float  # fraction of blocks refined per image
    field: str  # "gauss" | "street" | "ct" | "pathology"
    full_block: bool = False  # LN/FFN sandwich around the module
    gate_conv: bool = False  # depthwise 3x3 inside the gate's head score
    seed: int = 0
    keep_override: int | None = None  # explicit block count (edge cases)

    @property
    def tokens(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def head_dim(self) -> int:
        return self.channels // self.heads

    @property
    def num_blocks(self) -> int:
        return (self.grid_h // self.block) * (self.grid_w // self.block)

    @property
    def keep_blocks(self) -> int:
        if self.keep_override is not None:
            return self.keep_override
        return keep_blocks_for(self.keep, self.num_blocks)

    def kwargs(self):
        """Shape keywords shared by the oracle and the library binding."""
        return dict(grid_h=self.grid_h, grid_w=self.grid_w, heads=self.heads,
                    block=self.block, window=self.window,
                    keep_blocks=self.keep_blocks)


def scaled(wl: Workload, **changes) -> Workload:
    """A copy with some fields changed (smaller grids for parity tests, other
    keep ratios for sweeps)."""
    return dataclasses.replace(wl, **changes)


WORKLOADS = {
    # 1x16x16 tokens, C=64 (2 heads of 32), float32, identity + 3x3.
    "tiny": Workload("tiny", 1, 16, 16, 64, 2, "f32", (3,), 4, 8, 0.25,
                     "gauss", seed=1),
    # 4 street scenes of 1024x2048 pixels at stride 16.
    "street": Workload("street", 4, 64, 128, 256, 8, "bf16", (3, 5), 8, 16,
                       0.10, "street", seed=2),
    # 8 CT slices of 512x512 at stride 4.
    "ct": Workload("ct", 8, 128, 128, 128, 4, "bf16", (3, 5), 8, 16, 0.15,
                   "ct", seed=3),
    # 2 pathology tiles of 256x256 tokens.
    "pathology": Workload("pathology", 2, 256, 256, 128, 4, "bf16", (3, 5), 8,
                          24, 0.05, "pathology", seed=4),
    # Full block (LN, module, FFN-DWConv sandwich), 2 x 128x256 tokens.
    "block": Workload("block", 2, 128, 256, 384, 12, "bf16", (3, 5), 8, 16,
                      0.10, "street", full_block=True, seed=5),
}

BLOCK_KEEP_SWEEP = (0.0, 0.05, 0.10, 0.25, 0.50)


# ---------------------------------------------------------------------------
# spatial fields
# ---------------------------------------------------------------------------

def _field_street(rng, B, gh, gw, C):
    """N(0,1) noise plus 4 plane-wave cosines per image with integer
    frequencies of at most 3 cycles per axis and per-channel amplitudes
    N(0, 1/2) (so the smooth part has variance about 1)."""
    ys, xs = np.meshgrid(np.arange(gh) / gh, np.arange(gw) / gw,
                         indexing="ij")
    x = rng.standard_normal((B, gh, gw, C))
    for b in range(B):
        for _ in range(4):
            fy, fx = rng.integers(0, 4, size=2)
            if fy == 0 and fx == 0:
                fx = 1
            phase = rng.uniform(0, 2 * math.pi)
            amp = rng.normal(0.0, math.sqrt(0.5), size=C)
            wave = np.cos(2 * math.pi * (fy * ys + fx * xs) + phase)
            x[b] += wave[:, :, None] * amp[None, None, :]
    return x


def _field_ct(rng, B, gh, gw, C):
    """Background N(0, 0.2); 3-6 rotated ellipses per image (centres in the
    middle 3/4 of the grid, semi-axes 6..24 tokens at a 128 grid, scaled with
    the grid) whose tokens are N(0, 1)."""
    s = min(gh, gw) / 128.0
    ys, xs = np.meshgrid(np.arange(gh), np.arange(gw), indexing="ij")
    x = rng.normal(0.0, math.sqrt(0.2), size=(B, gh, gw, C))
    for b in range(B):
        inside = np.zeros((gh, gw), dtype=bool)
        for _ in range(int(rng.integers(3, 7))):
            cy = rng.uniform(gh / 8, 7 * gh / 8)
            cx = rng.uniform(gw / 8, 7 * gw / 8)
            a = max(1.0, rng.uniform(6, 24) * s)
            bb = max(1.0, rng.uniform(6, 24) * s)
            th = rng.uniform(0, math.pi)
            u = (ys - cy) * math.cos(th) + (xs - cx) * math.sin(th)
            v = -(ys - cy) * math.sin(th) + (xs - cx) * math.cos(th)
            inside |= (u / a) ** 2 + (v / bb) ** 2 <= 1.0
        n_in = int(inside.sum())
        x[b][inside] = rng.standard_normal((n_in, C))
    return x


def _field_pathology(rng, B, gh, gw, C):
    """Foreground mask = 12 Gaussian bumps (sigma 6..20 tokens at a 256 grid,
    scaled with the grid) thresholded at their 80th percentile (about 20%
    coverage); N(0, 1) inside, N(0, 0.1) outside."""
    s = min(gh, gw) / 256.0
    ys, xs = np.meshgrid(np.arange(gh), np.arange(gw), indexing="ij")
    x = np.empty((B, gh, gw, C))
    for b in range(B):
        dens = np.zeros((gh, gw))
        for _ in range(12):
            cy, cx = rng.uniform(0, gh), rng.uniform(0, gw)
            sig = max(1.0, rng.uniform(6, 20) * s)
            dens += np.exp(-((ys - cy) ** 2 + (xs - cx) ** 2) / (2 * sig * sig))
        mask = dens > np.percentile(dens, 80)
        x[b] = rng.normal(0.0, math.sqrt(0.1), size=(gh, gw, C))
        x[b][mask] = rng.standard_normal((int(mask.sum()), C))
    return x


_FIELDS = {
    "gauss": lambda rng, B, gh, gw, C: rng.standard_normal((B, gh, gw, C)),
    "street": _field_street,
    "ct": _field_ct,
    "pathology": _field_pathology,
}


# ---------------------------------------------------------------------------
# rounding to the run dtype (data preparation only)
# ---------------------------------------------------------------------------

def _to_dtype(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    if dtype == "bf16":
        t = t.to(torch.float32).to(torch.bfloat16)
    elif dtype == "f32":
        t = t.to(torch.float32)
    else:
        raise ValueError(dtype)
    return t.to(torch.float64).numpy()


def make_inputs(wl: Workload, seed: int | None = None):
    """Draw X and all weights for a workload.

    Returns float64 arrays whose values are exact in the run dtype (gate
    weights exact in float32):
      x [B, N, C], w_qkv [C, 3C] ~ N(0, 1/C), w_o [C, C] ~ N(0, 1/C),
      dw: list of [3C, k, k] ~ N(0, 1/k^2), gate_w [H, 3d] ~ N(0, 1/(3d)),
      gate_b [H] = 0, and for the full block ln1_g/ln2_g = 1, ln1_b/ln2_b =
      0, w1 [C, 4C] ~ N(0, 1/C), dw_ffn [4C, 3, 3] ~ N(0, 1/9),
      w2 [4C, C] ~ N(0, 1/(4C)); with gate_conv, gate_dw [3C, 3, 3] ~
      N(0, 1/9), drawn from its own generator (seeded by [seed, 1]) so the
      other inputs do not change.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, gh, gw, C, H = wl.batch, wl.grid_h, wl.grid_w, wl.channels, wl.heads
    d = C // H
    dt = wl.dtype
    x = _FIELDS[wl.field](rng, B, gh, gw, C).reshape(B, gh * gw, C)
    w_qkv = rng.normal(0.0, math.sqrt(1.0 / C), size=(C, 3 * C))
    w_o = rng.normal(0.0, math.sqrt(1.0 / C), size=(C, C))
    dw = [rng.normal(0.0, 1.0 / k, size=(3 * C, k, k)) for k in wl.branches]
    gate_w = rng.normal(0.0, math.sqrt(1.0 / (3 * d)), size=(H, 3 * d))
    gate_b = np.zeros(H)
    out = dict(x=_to_dtype(x, dt), w_qkv=_to_dtype(w_qkv, dt),
               w_o=_to_dtype(w_o, dt), dw=[_to_dtype(w, dt) for w in dw],
               gate_w=_to_dtype(gate_w, "f32"), gate_b=_to_dtype(gate_b, "f32"))
    if wl.full_block:
        w1 = rng.normal(0.0, math.sqrt(1.0 / C), size=(C, 4 * C))
        dw_ffn = rng.normal(0.0, 1.0 / 3.0, size=(4 * C, 3, 3))
        w2 = rng.normal(0.0, math.sqrt(1.0 / (4 * C)), size=(4 * C, C))
        out.update(ln1_g=np.ones(C), ln1_b=np.zeros(C), ln2_g=np.ones(C),
                   ln2_b=np.zeros(C), w1=_to_dtype(w1, dt),
                   dw_ffn=_to_dtype(dw_ffn, dt), w2=_to_dtype(w2, dt))
    if wl.gate_conv:
        grng = np.random.default_rng([wl.seed if seed is None else seed, 1])
        out["gate_dw"] = _to_dtype(grng.normal(0.0, 1.0 / 3.0, size=(3 * C, 3, 3)), dt)
    return out
