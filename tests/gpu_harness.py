"""Shared helpers of the GPU parity tests: run the library through its C ABI
on seeded inputs and compare with the CPU oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
from efficient_vision_attention_amd import hsmla as H
from efficient_vision_attention_amd.device import DeviceModel, to_device, to_host
from workloads import Workload

# Tolerances (allclose form |gpu - ref| <= atol + rtol * |ref|).
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}


def announce(msg: str):
    """Name the case before a GPU step, flushed, so a fault names it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def shape_of(wl: Workload, keep_blocks=None, tau=None, per_head=False,
             soft=False) -> dict:
    return dict(batch=wl.batch, grid_h=wl.grid_h, grid_w=wl.grid_w,
                channels=wl.channels, heads=wl.heads, branches=wl.branches,
                block=wl.block, window=wl.window,
                keep_blocks=wl.keep_blocks if keep_blocks is None else keep_blocks,
                dtype=wl.dtype, tau=tau, per_head=per_head, soft=soft)


def assert_close(gpu, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} elements outside "
            f"{atol}+{rtol}|ref|; worst at {idx}: gpu={gpu[idx]!r} ref={ref[idx]!r}")
    return float(err.max()) if err.size else 0.0


def staged(wl: Workload) -> bool:
    return wl.dtype == "bf16"


def rnd_for(wl: Workload):
    return O.round_bf16 if staged(wl) else (lambda a: a)


def oracle_kwargs(wl: Workload, keep_blocks=None):
    kw = wl.kwargs()
    if keep_blocks is not None:
        kw["keep_blocks"] = keep_blocks
    return kw


def selection_band_check(scores_ref, scores_gpu, sel_ref, sel_gpu, k):
    """Accept a differing selection only inside the near-tie band
    |M - M_(k)| <= 2 max|dM| around the k-th score of each image.
    Returns a list of (image, gap, max_dM, n_diff)."""
    report = []
    for b in range(sel_ref.shape[0]):
        a, g = set(sel_ref[b].tolist()), set(sel_gpu[b].tolist())
        dm = float(np.max(np.abs(scores_ref[b] - scores_gpu[b])))
        srt = np.sort(scores_ref[b])[::-1]
        kth = srt[k - 1] if k > 0 else np.inf
        gap = float(srt[k - 1] - srt[k]) if 0 < k < srt.size else np.inf
        diff = a ^ g
        for t in diff:
            assert abs(scores_ref[b][t] - kth) <= 2 * dm + 1e-12, (
                f"image {b}: block {t} differs outside the tie band "
                f"(|M-M_k|={abs(scores_ref[b][t] - kth):.3e}, max dM={dm:.3e})")
        report.append((b, gap, dm, len(diff)))
    return report


def routed_lists(sel, counts):
    """Per-image selections of a threshold run: sel[b][:counts[b]]."""
    return [np.asarray(sel[b][:int(counts[b])]) for b in range(len(counts))]


def padded(lists, width):
    """Per-image index lists -> [B, width] array padded with -1 (the form the
    oracle takes as an injected selection)."""
    out = np.full((len(lists), width), -1, dtype=np.int64)
    for b, l in enumerate(lists):
        out[b, :len(l)] = l
    return out


def threshold_band_check(scores_ref, scores_gpu, tau, ref_lists, gpu_lists):
    """Accept a differing threshold selection only for blocks whose score is
    within 2 max|dM| of tau.  Returns a list of (image, max_dM, n_diff)."""
    report = []
    for b in range(len(ref_lists)):
        dm = float(np.max(np.abs(scores_ref[b] - scores_gpu[b])))
        diff = set(ref_lists[b].tolist()) ^ set(gpu_lists[b].tolist())
        for t in diff:
            assert abs(scores_ref[b][t] - tau) <= 2 * dm + 1e-12, (
                f"image {b}: block {t} routed differently outside the tie band "
                f"(|M-tau|={abs(scores_ref[b][t] - tau):.3e}, max dM={dm:.3e})")
        report.append((b, dm, len(diff)))
    return report


def tau_between(scores, quantile):
    """A float32 threshold halfway between two adjacent distinct float32
    scores near the given quantile of all scores (so no score equals it)."""
    v = np.unique(np.asarray(scores, np.float32).ravel())
    i = min(max(int(quantile * (v.size - 1)), 0), v.size - 2)
    return float(np.float32((np.float64(v[i]) + np.float64(v[i + 1])) / 2))


class Run:
    """Device model + buffers for one workload, with numpy readback.  With
    tau set, the model routes by threshold and the readback holds counts."""

    def __init__(self, wl: Workload, inputs: dict, keep_blocks=None, tau=None,
                 per_head=False, soft=False):
        self.wl = wl
        self.inputs = inputs
        self.model = DeviceModel(shape_of(wl, keep_blocks, tau, per_head, soft), inputs)
        self.desc = self.model.desc
        self.tau = tau
        self.k = ("soft" if soft else self.model.shape["keep_blocks"] if tau is None
                  else f"tau={tau:.6g}{' per head' if per_head else ''}")
        self.x = to_device(inputs["x"], wl.dtype)

    def forward(self):
        m = self.model
        y = m.act()
        ws = m.workspace(H.HSMLA_OP_FORWARD)
        announce(f"hsmla_forward {self.wl.name} B={self.wl.batch} "
                 f"{self.wl.grid_h}x{self.wl.grid_w} C={self.wl.channels} k={self.k}")
        H.hsmla_forward(self.desc, m.weights, self.x, y, ws)
        torch.cuda.synchronize()
        v = m.views(H.HSMLA_OP_FORWARD, ws)
        out = {name: to_host(t) if t.dtype != torch.int32 else t.cpu().numpy()
               for name, t in v.items()}
        out["y"] = to_host(y)
        return out

    def block_forward(self):
        m = self.model
        out_t = m.act()
        ws = m.workspace(H.HSMLA_OP_BLOCK)
        announce(f"hsmla_block_forward {self.wl.name} B={self.wl.batch} "
                 f"{self.wl.grid_h}x{self.wl.grid_w} C={self.wl.channels} k={self.k}")
        H.hsmla_block_forward(self.desc, m.weights, m.ffn, self.x, out_t, ws)
        torch.cuda.synchronize()
        v = m.views(H.HSMLA_OP_BLOCK, ws)
        out = {name: to_host(t) if t.dtype != torch.int32 else t.cpu().numpy()
               for name, t in v.items()}
        out["out"] = to_host(out_t)
        return out
