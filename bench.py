#!/usr/bin/env python3
"""Throughput of the HSMLA block forward on one MI355X.

Workload: 2 images of 128 x 256 tokens, C = 384 (12 heads of 32), bf16,
identity + 3x3 + 5x5 depthwise branches, 8 x 8 blocks, 16 x 16 softmax
windows, keep ratio 10% (52 of 512 blocks per image), wrapped in the LN /
FFN-DWConv block.  One step = one call of hsmla_block_forward over the
batch on one stream (--streams 2: hsmla_block_forward_split, the two
images on two streams), i.e. every kernel of the path, with the weights'
GEMM layouts and folded taps written once by hsmla_prepare (the call
without it is timed beside).  Inputs are seeded synthetic data
(street-scene-like smooth field plus noise) already resident in HBM.
Before the warm-up steps the block runs back to back for 200 ms so the
clocks have left their idle state.

Prints one JSON line: tokens/s; per-kernel durations from HIP events
recorded between the launches of the step, each with the fraction of the
roofline that bounds it (the refinement also against the union of its
windows' bytes); the dominant kernel's roofline; achievable-peak probes (a
1 GiB device copy, a large library GEMM); the street, CT, pathology and
tiny workloads' module forward (tokens/s, per-kernel fractions, and the
oracle on a crop); a keep-ratio sweep with two threshold-routing points,
per-head routing, the training-time mixture forward and the exact-gate /
three-branch variant; and the CPU oracle timed on a bounded crop.

    python bench.py [--steps K] [--warmup W] [--no-sweep] [--no-configs]
                    [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, GB/s
MFMA_BF16_TFLOPS = 2500.0  # dense bf16 matrix peak, TFLOP/s

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--keep", type=float, default=0.10)
    ap.add_argument("--branches", default="3,5",
                    help="depthwise branch sizes added to the identity")
    ap.add_argument("--gate-conv", action="store_true",
                    help="depthwise 3x3 inside the gate's head score")
    ap.add_argument("--streams", type=int, default=1, choices=(1, 2),
                    help="1: one stream (hsmla_block_forward); 2: the block's "
                         "batch split over two streams "
                         "(hsmla_block_forward_split)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--spinup-ms", type=float, default=200.0,
                    help="back-to-back untimed steps before the warm-up")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the street / CT / pathology / tiny module runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power-s", type=float, default=1.0,
                    help="seconds of back-to-back steps over which board power "
                         "and the shader clock are sampled")
    ap.add_argument("--cpu-rows", type=int, default=64,
                    help="token rows of the one-image crop the CPU oracle is "
                         "timed on")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# HIP events through the runtime torch already loaded (same process state)
# ---------------------------------------------------------------------------

class HipEvents:
    def __init__(self):
        import torch
        libdir = os.path.join(os.path.dirname(torch.__file__), "lib")
        path = os.path.join(libdir, "libamdhip64.so")
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def sync(self, e):
        self.hip.hipEventSynchronize(e)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


# ---------------------------------------------------------------------------
# algorithmic work per launch (bytes moved at minimum, flops of the method)
# ---------------------------------------------------------------------------

def window_keys(sel, grid_h, grid_w, block, window):
    """Clipped window size |W| of every selected block."""
    nbc = grid_w // block
    p = (window - block) // 2
    out = []
    for t in np.asarray(sel).reshape(-1).tolist():
        r0, c0 = (t // nbc) * block, (t % nbc) * block
        rows = min(grid_h, r0 + block + p) - max(0, r0 - p)
        cols = min(grid_w, c0 + block + p) - max(0, c0 - p)
        out.append(rows * cols)
    return np.array(out, dtype=np.int64)


def algorithmic_work(name, wl, sel):
    """(bytes, flops) one launch of kernel `name` must move / perform."""
    e = 2 if wl.dtype == "bf16" else 4
    C, P, d = wl.channels, wl.batch * wl.tokens, wl.head_dim
    H, Bs = wl.heads, wl.block
    if name in ("layernorm1", "layernorm2"):
        return 2 * C * e * P, 8 * C * P
    if name == "qkv_gemm":
        return P * 4 * C * e + 3 * C * C * e, 2 * P * C * 3 * C
    if name == "dwconv_qkv":
        k2 = sum(k * k for k in wl.branches) + 1
        return 6 * C * e * P, 2 * 3 * C * P * k2
    if name == "kv_state":
        return 2 * C * e * P, 2 * C * d * P
    if name == "lin_apply":
        return 2 * C * e * P, (2 * C * d + 3 * C) * P
    if name == "gate_scores":
        return 3 * C * e * P, (18 if wl.gate_conv else 1) * 3 * C * P
    if name in ("topk", "threshold"):
        return wl.batch * wl.num_blocks * 8, 0
    if name == "gate_topk":
        # the gate's partial logits (3 per head and block, formed by the S2
        # conv) in, scores and the selection out
        return wl.batch * wl.num_blocks * (3 * H * 4 + 8), 0
    if name == "kv_state_gate_topk":
        # the K/V state with the gate's top-k in its partial-sum launch
        kb, kf = algorithmic_work("kv_state", wl, sel)
        gb, _ = algorithmic_work("gate_topk", wl, sel)
        return kb + gb, kf
    if name == "sparse_softmax":
        W = window_keys(sel, wl.grid_h, wl.grid_w, Bs, wl.window)
        q = Bs * Bs
        by = int(np.sum(e * (4 * q * d + 4 * W * d))) * H
        fl = int(np.sum(4 * q * W * d + 2 * W * d * d + 2 * q * d * d + 2 * W * d)) * H
        return by, fl
    if name in ("out_proj", "out_proj_residual"):
        extra = C * e * P if name.endswith("residual") else 0
        return 2 * C * e * P + extra + C * C * e, 2 * P * C * C
    if name == "ffn1_gemm":
        return P * 5 * C * e + 4 * C * C * e, 2 * P * C * 4 * C
    if name == "ffn_dwconv_gelu":
        return 8 * C * e * P, 2 * 4 * C * P * 9
    if name == "ffn2_gemm_residual":
        return P * 6 * C * e + 4 * C * C * e, 2 * P * 4 * C * C
    if name in ("dw_taps", "ffn_dw_taps", "prep"):
        return 0, 0
    raise KeyError(name)


MFMA_SITES = ("qkv_gemm", "out_proj", "out_proj_residual", "ffn1_gemm",
              "ffn2_gemm_residual", "sparse_softmax")

# float32 FMA issue of the vector ALUs without packed instructions (which the
# build switches off): 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz
VALU_F32_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12


def alu_flops(name, wl):
    """FMA flops the depthwise convolutions execute: the folded tap set
    (kmax^2 taps per output for the module's branches, 9 for the FFN's
    3x3; the GELU's instructions are not counted), or None."""
    P, C = wl.batch * wl.tokens, wl.channels
    if name == "dwconv_qkv":
        kmax = max((1,) + tuple(wl.branches))
        return 2 * 3 * C * P * kmax * kmax
    if name == "ffn_dwconv_gelu":
        return 2 * 4 * C * P * 9
    return None


def union_window_bytes(wl, sel):
    """S5's minimum HBM bytes: every token of the union of the selected
    blocks' clipped windows read once as raw and hatted K and V (4 C
    elements), and every selected token's q, q^ read and o read and written
    (4 C elements), per image; the no-reuse per-window sum is
    algorithmic_work's figure."""
    e = 2 if wl.dtype == "bf16" else 4
    C, Bs, nbc = wl.channels, wl.block, wl.grid_w // wl.block
    p = (wl.window - Bs) // 2
    sel = np.asarray(sel).reshape(wl.batch, -1)
    total = 0
    for b in range(wl.batch):
        cover = np.zeros((wl.grid_h, wl.grid_w), dtype=bool)
        for t in sel[b].tolist():
            if t < 0:
                continue
            r0, c0 = (t // nbc) * Bs, (t % nbc) * Bs
            cover[max(0, r0 - p):r0 + Bs + p, max(0, c0 - p):c0 + Bs + p] = True
        q_tokens = int(np.sum(sel[b] >= 0)) * Bs * Bs
        total += (int(cover.sum()) * 4 * C + q_tokens * 4 * C) * e
    return total


def roofline_entry(name, wl, sel, avg_ms, by=None):
    """Fraction of the roofline that bounds kernel `name`: its algorithmic
    bytes (or `by`) over the HBM peak, or its flops over the bf16 MFMA peak
    when that takes longer (the dense contractions and the refinement)."""
    by0, fl = algorithmic_work(name, wl, sel)
    by = by0 if by is None else by
    t_hbm = by / (HBM_PEAK_GBS * 1e9)
    t_mfma = fl / (MFMA_BF16_TFLOPS * 1e12)
    sec = avg_ms * 1e-3
    if name in MFMA_SITES and t_mfma > t_hbm:
        ach = fl / sec / 1e12
        return dict(bound="mfma", achieved=round(ach, 2), peak=MFMA_BF16_TFLOPS,
                    unit="TFLOP/s", frac=round(ach / MFMA_BF16_TFLOPS, 4),
                    traffic=None)
    fa = alu_flops(name, wl)
    if fa and fa / (VALU_F32_TFLOPS * 1e12) > t_hbm:
        ach = fa / sec / 1e12
        return dict(bound="alu", achieved=round(ach, 2), peak=round(VALU_F32_TFLOPS, 1),
                    unit="TFLOP/s", frac=round(ach / VALU_F32_TFLOPS, 4), traffic=None,
                    hbm_frac=round(by / sec / 1e9 / HBM_PEAK_GBS, 4))
    ach = by / sec / 1e9
    out = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS,
               unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4), traffic=None)
    if fa:
        out["alu_frac"] = round(fa / sec / 1e12 / VALU_F32_TFLOPS, 4)
    if name in MFMA_SITES and fl:
        # matrix-core use at the same duration (flops / time / peak)
        out["mfma_frac"] = round(fl / sec / 1e12 / MFMA_BF16_TFLOPS, 4)
    return out


def measured_traffic(launch):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated), or None when there is none for
    this launch or its kernel sources changed since the counters were taken.
    Summary lines read: 'traffic: launch=<name> bytes=<B> sources=<f1,f2>
    sha256=<hex of the concatenated sources>'."""
    import hashlib
    import glob
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic:"):
                    continue
                kv = dict(tok.split("=", 1) for tok in line.split()[1:])
                if kv.get("launch") != launch:
                    continue
                h = hashlib.sha256()
                try:
                    for src in kv["sources"].split(","):
                        with open(os.path.join(ROOT, src), "rb") as g:
                            h.update(g.read())
                except OSError:
                    return None
                if h.hexdigest() != kv.get("sha256"):
                    return None
                return int(kv["bytes"])
    return None


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded crop of the same workload)
# ---------------------------------------------------------------------------

def _blas_threads():
    try:
        import threadpoolctl
        return max(i["num_threads"] for i in threadpoolctl.threadpool_info())
    except Exception:
        return os.cpu_count()


def cpu_baseline(wl, rows, images=1, runs=3, forward=False):
    """The CPU oracle as it stands, on a crop of `images` images of `rows`
    token rows of the workload: one warm-up, then `runs` timed runs (one if
    a run takes over 60 s), median."""
    import oracle as O  # test infrastructure, timed here as a baseline only
    from workloads import make_inputs, scaled
    crop = scaled(wl, batch=min(images, wl.batch), grid_h=min(rows, wl.grid_h))
    inp = make_inputs(crop)
    fn = O.hsmla_forward if forward else O.hsmla_block_forward
    staged = crop.dtype == "bf16"
    times = []
    for i in range(runs + 1):
        t0 = time.perf_counter()
        fn(inp["x"], inp, staged=staged, **crop.kwargs())
        times.append(time.perf_counter() - t0)
        if times[-1] > 60.0:
            break
    timed = times[1:] or times
    dt = float(np.median(timed))
    what = "module forward" if forward else "block forward"
    return dict(value=round(crop.batch * crop.tokens / dt, 1), unit="tokens/s",
                cores=_blas_threads(), os_cpu_count=os.cpu_count(),
                kind="oracle",
                sample=(f"{crop.batch} image(s) of {crop.grid_h}x{crop.grid_w} tokens "
                        f"({crop.batch * crop.tokens} tokens, keep {crop.keep_blocks} of "
                        f"{crop.num_blocks} blocks per image), float64 "
                        f"{'bf16-staged ' if staged else ''}{what}, median of "
                        f"{len(timed)} run(s) after a warm-up: {dt:.2f} s"))


# ---------------------------------------------------------------------------

def probes(torch):
    """Achievable peaks on this machine: a plain 1 GiB device copy (read + write
    bytes / time) and a large bf16 library GEMM (hipBLASLt through torch)."""
    out = {}
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 10
    out["copy_1GiB_gbs"] = round(2 * src.numel() * 2 / (ms * 1e-3) / 1e9, 1)
    del src, dst
    n = 8192
    x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    w = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        y = x @ w
    torch.cuda.synchronize()
    a.record()
    for _ in range(10):
        y = x @ w
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 10
    out["gemm_bf16_8192_tflops"] = round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    del x, w, y
    torch.cuda.empty_cache()
    return out


class PowerSampler:
    """Board power (hwmon power1_input, W) and the shader clock level
    (pp_dpm_sclk, MHz) sampled every few ms on a host thread while the GPU
    runs; None where the sensors cannot be read."""

    def __init__(self):
        import glob
        self.pw = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
        self.cap = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_cap"))
        self.sclk = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []
        self._stop = False

    def _read(self):
        row = [None, None]
        try:
            row[0] = int(open(self.pw[0]).read()) / 1e6
        except (OSError, IndexError, ValueError):
            pass
        try:
            cur = [l for l in open(self.sclk[0]).read().splitlines() if l.endswith("*")]
            row[1] = int(cur[0].split(":")[1].strip().split("M")[0]) if cur else None
        except (OSError, IndexError, ValueError):
            pass
        return row

    def __enter__(self):
        import threading

        def loop():
            while not self._stop:
                self.samples.append(self._read())
                time.sleep(0.004)
        self._t = threading.Thread(target=loop, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop = True
        self._t.join()

    def summary(self):
        w = [r[0] for r in self.samples if r[0] is not None]
        c = [r[1] for r in self.samples if r[1] is not None]
        cap = None
        try:
            cap = int(open(self.cap[0]).read()) / 1e6
        except (OSError, IndexError, ValueError):
            pass
        if not w and not c:
            return None
        # the second half of the window: the clocks have settled by then
        w, c = w[len(w) // 2:], c[len(c) // 2:]
        return {"board_w_mean": round(float(np.mean(w)), 1) if w else None,
                "cap_w": cap,
                "sclk_mhz_median": float(np.median(c)) if c else None,
                "samples": len(w) or len(c),
                "window": "back-to-back headline steps after the timed ones"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU "
                          "sharding is described, not implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from efficient_vision_attention_amd import hsmla as H
    from efficient_vision_attention_amd.device import DeviceModel, to_device
    from workloads import WORKLOADS, keep_blocks_for, make_inputs, scaled

    torch.cuda.set_device(0)
    probe = probes(torch)
    base = scaled(WORKLOADS["block"], keep=args.keep,
                  branches=tuple(int(k) for k in args.branches.split(",") if k),
                  gate_conv=args.gate_conv)
    inp = make_inputs(base)
    x = to_device(inp["x"], base.dtype)

    def shape(wl, tau=None, per_head=False, soft=False):
        return dict(batch=wl.batch, grid_h=wl.grid_h, grid_w=wl.grid_w,
                    channels=wl.channels, heads=wl.heads, branches=wl.branches,
                    block=wl.block, window=wl.window, keep_blocks=wl.keep_blocks,
                    dtype=wl.dtype, tau=tau, per_head=per_head, soft=soft)

    class Bound:
        """A model with its workspace; `prepared` runs hsmla_prepare once
        and calls with desc.prepared (the weight-only operands are then not
        rewritten by every call)."""

        def __init__(self, model, op, prepared):
            self.m, self.op = model, op
            self.ws = model.workspace(op)
            self.out = model.act()
            self.desc = model.desc
            if prepared:
                H.hsmla_prepare(model.desc, op, model.weights,
                                model.ffn if op == H.HSMLA_OP_BLOCK else None, self.ws)
                self.desc = H.make_desc(**dict(model.shape, prepared=True))

        def block(self, xx):
            H.hsmla_block_forward(self.desc, self.m.weights, self.m.ffn, xx, self.out,
                                  self.ws)

        def block_split(self, xx, two):
            H.hsmla_block_forward_split(self.desc, self.m.weights, self.m.ffn, xx,
                                        self.out, self.ws, two)

        def forward(self, xx):
            H.hsmla_forward(self.desc, self.m.weights, xx, self.out, self.ws)

    def spin_up(fn, ms=200.0):
        """Back-to-back untimed steps for `ms` of wall time, so that the
        clocks have left their idle state before warm-up and timing (the
        steps right after the GPU idled for a while ran about 10% slower)."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()

    def time_steps(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    hev = HipEvents()

    def per_kernel(bound, xx, wl, sel, steps, warmup, block=True, step_ms=None):
        """Average duration of every launch of one step, from HIP events
        recorded on the launch stream between the launches (the steps run
        back to back; the events are read after the last).  Each event
        between two launches adds a gap of about the same length (2-3 us),
        so with step_ms (the same step timed without events) the gaps'
        total, the event-timed step minus step_ms, is taken off the
        launches in equal parts (avg_us_step): the figure the roofline
        fractions use, and the one a kernel trace of the plain step
        reproduces (a proportional scaling instead charged the short
        launches too much of the gaps)."""
        def timed(evs):
            if block:
                return H.hsmla_block_forward_timed(bound.desc, bound.m.weights,
                                                   bound.m.ffn, xx, bound.out,
                                                   bound.ws, evs)
            return H.hsmla_forward_timed(bound.desc, bound.m.weights, xx,
                                         bound.out, bound.ws, evs)
        probe_ev = hev.create(40)
        names = timed(probe_ev)
        L = len(names)
        evsets = [hev.create(L) for _ in range(steps)]
        for _ in range(warmup):
            timed(probe_ev)
        for i in range(steps):
            timed(evsets[i])
        torch.cuda.synchronize()
        per = {}
        for evs in evsets:
            for j in range(L - 1):
                per.setdefault(names[j], []).append(hev.elapsed_ms(evs[j], evs[j + 1]))
        hev.destroy(probe_ev)
        for evs in evsets:
            hev.destroy(evs)
        kernels = {}
        total = sum(float(np.mean(v)) for v in per.values())
        gap = (total - step_ms) / len(per) if step_ms else 0.0
        for n, v in per.items():
            raw = float(np.mean(v))
            avg = max(raw - gap, 0.5 * raw)
            by, fl = algorithmic_work(n, wl, sel)
            k = dict(avg_us=round(raw * 1e3, 2), bytes=int(by), flops=int(fl))
            if step_ms:
                k["avg_us_step"] = round(avg * 1e3, 2)
            if by or fl:
                k["roofline"] = roofline_entry(n, wl, sel, avg)
                if block:  # the committed counters cover the headline block's launches
                    k["roofline"]["traffic"] = measured_traffic(n)
            if n == "sparse_softmax":
                ub = union_window_bytes(wl, sel)
                k["union_bytes"] = int(ub)
                k["roofline_union"] = roofline_entry(n, wl, sel, avg, by=ub)
            kernels[n] = k
        return kernels

    two = H.SplitStreams()
    model = DeviceModel(shape(base), inp)
    head = Bound(model, H.HSMLA_OP_BLOCK, prepared=True)
    plain = Bound(model, H.HSMLA_OP_BLOCK, prepared=False)
    spin_up(lambda: head.block(x), args.spinup_ms)
    if args.streams == 2:
        ms = time_steps(lambda: head.block_split(x, two), args.steps, args.warmup)
        ms_alt = time_steps(lambda: head.block(x), args.steps, args.warmup)
    else:
        ms = time_steps(lambda: head.block(x), args.steps, args.warmup)
        ms_alt = time_steps(lambda: head.block_split(x, two), args.steps, args.warmup)
    ms_plain = time_steps(lambda: plain.block(x), args.steps, args.warmup)
    # board power and clock over a second of back-to-back headline steps
    # (the sensor averages over a window, so a short burst under-reads it),
    # with that window's own step time beside them
    with PowerSampler() as power:
        torch.cuda.synchronize()
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < args.power_s:
            for _ in range(20):
                head.block(x)
            torch.cuda.synchronize()
            n += 20
        steady_ms = (time.perf_counter() - t0) / max(n, 1) * 1e3
    tokens = base.batch * base.tokens
    head.block(x)
    torch.cuda.synchronize()
    spin_up(lambda: head.block(x), 50.0)
    base_views = model.views(H.HSMLA_OP_BLOCK, head.ws)
    sel = base_views["sel"].cpu().numpy()
    base_scores = base_views["scores"].cpu().numpy()
    kernels = per_kernel(head, x, base, sel, args.steps, args.warmup,
                         step_ms=ms if args.streams == 1 else ms_alt)
    prep_us = per_kernel(plain, x, base, sel, 5, 2)["prep"]["avg_us"]
    dominant = max(kernels, key=lambda n: kernels[n]["avg_us"])
    roof = dict(kernels[dominant]["roofline"])
    roof["avg_us"] = kernels[dominant]["avg_us_step"]
    roof["kernel"] = dominant
    roof["traffic"] = measured_traffic(dominant)
    by, fl = algorithmic_work(dominant, base, sel)
    roof["work_per_launch"] = {"bytes": int(by), "flops": int(fl)}
    # the k-th / (k+1)-th score gap per image (the margin of the selection)
    gaps = []
    for b in range(base.batch):
        srt = np.sort(base_scores[b].astype(np.float64))[::-1]
        k = base.keep_blocks
        gaps.append(float(srt[k - 1] - srt[k]) if 0 < k < srt.size else None)

    # the other workloads: the module forward (prepared weights) per config
    configs = []
    crops = {"tiny": (16, 1), "street": (64, 1), "ct": (64, 1), "pathology": (32, 1)}
    for name in () if args.no_configs else ("tiny", "street", "ct", "pathology"):
        wl = WORKLOADS[name]
        winp = make_inputs(wl)
        wx = to_device(winp["x"], wl.dtype)
        bd = Bound(DeviceModel(shape(wl), winp), H.HSMLA_OP_FORWARD, prepared=True)
        spin_up(lambda: bd.forward(wx), 100.0)
        msf = time_steps(lambda: bd.forward(wx), args.steps, args.warmup)
        bd.forward(wx)
        torch.cuda.synchronize()
        wsel = bd.m.views(H.HSMLA_OP_FORWARD, bd.ws)["sel"].cpu().numpy()
        entry = dict(workload=name, batch=wl.batch, grid=[wl.grid_h, wl.grid_w],
                     tokens=wl.batch * wl.tokens, channels=wl.channels,
                     heads=wl.heads, dtype=wl.dtype, block=wl.block,
                     window=wl.window, keep=wl.keep, keep_blocks=wl.keep_blocks,
                     ms_per_forward=round(msf, 4))
        if name == "tiny":
            entry["latency_us"] = round(msf * 1e3, 2)  # launch-bound: latency only
        else:
            entry["tokens_per_s"] = round(wl.batch * wl.tokens / (msf * 1e-3), 1)
            entry["kernels"] = per_kernel(bd, wx, wl, wsel, args.steps, args.warmup,
                                          block=False, step_ms=msf)
        if not args.no_cpu_baseline:
            rows, imgs = crops[name]
            entry["cpu_baseline"] = cpu_baseline(wl, rows, imgs, forward=True)
        configs.append(entry)
        del bd

    sweep = []
    if not args.no_sweep:
        n_sw = max(10, args.steps // 2)
        for r in (0.0, 0.05, 0.10, 0.25, 0.50):
            wl = scaled(base, keep=r)
            m = DeviceModel(shape(wl), inp)
            bb = Bound(m, H.HSMLA_OP_BLOCK, prepared=True)
            spin_up(lambda: bb.block(x), 50.0)
            ms_b = time_steps(lambda: bb.block(x), n_sw, 10)
            bf = Bound(m, H.HSMLA_OP_FORWARD, prepared=True)
            ms_m = time_steps(lambda: bf.forward(x), n_sw, 10)
            bb.block(x)
            torch.cuda.synchronize()
            s_sel = m.views(H.HSMLA_OP_BLOCK, bb.ws)["sel"].cpu().numpy()
            sp = per_kernel(bb, x, wl, s_sel, 5, 2, step_ms=ms_b).get("sparse_softmax")
            sweep.append(dict(keep=r, keep_blocks=keep_blocks_for(r, wl.num_blocks),
                              block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                              block_ms=round(ms_b, 4),
                              module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                              module_ms=round(ms_m, 4),
                              sparse_softmax=sp))
            del m, bb, bf
        # threshold routing (blocks with score > tau), tau placed between two
        # adjacent scores of the run above at the given quantile
        uniq = np.unique(base_scores.astype(np.float32))
        for q in (0.9, 0.7):
            i = min(int(q * (uniq.size - 1)), uniq.size - 2)
            tau = float(np.float32((np.float64(uniq[i]) + np.float64(uniq[i + 1])) / 2))
            m = DeviceModel(shape(base, tau=tau), inp)
            bb = Bound(m, H.HSMLA_OP_BLOCK, prepared=True)
            ms_b = time_steps(lambda: bb.block(x), n_sw, 10)
            routed = int(m.views(H.HSMLA_OP_BLOCK, bb.ws)["counts"].sum().item())
            bf = Bound(m, H.HSMLA_OP_FORWARD, prepared=True)
            ms_m = time_steps(lambda: bf.forward(x), n_sw, 10)
            sweep.append(dict(routing="threshold", tau=tau,
                              routed_fraction=round(routed / (base.batch * base.num_blocks), 4),
                              block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                              block_ms=round(ms_b, 4),
                              module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                              module_ms=round(ms_m, 4)))
            del m, bb, bf

        # per-head routing (each head by its own score), tau between two
        # adjacent head scores of a first per-head run at the 0.7 quantile
        m = DeviceModel(shape(base, tau=0.5, per_head=True), inp)
        bb = Bound(m, H.HSMLA_OP_BLOCK, prepared=True)
        bb.block(x)
        torch.cuda.synchronize()
        hs = m.views(H.HSMLA_OP_BLOCK, bb.ws)["head_scores"].cpu().numpy()
        uniq = np.unique(hs.astype(np.float32))
        i = min(int(0.7 * (uniq.size - 1)), uniq.size - 2)
        tau = float(np.float32((np.float64(uniq[i]) + np.float64(uniq[i + 1])) / 2))
        del m, bb
        m = DeviceModel(shape(base, tau=tau, per_head=True), inp)
        bb = Bound(m, H.HSMLA_OP_BLOCK, prepared=True)
        ms_b = time_steps(lambda: bb.block(x), n_sw, 10)
        routed = int(m.views(H.HSMLA_OP_BLOCK, bb.ws)["counts"].sum().item())
        bf = Bound(m, H.HSMLA_OP_FORWARD, prepared=True)
        ms_m = time_steps(lambda: bf.forward(x), n_sw, 10)
        sweep.append(dict(routing="threshold_per_head", tau=tau,
                          routed_fraction=round(routed / (base.batch * base.num_blocks
                                                          * base.heads), 4),
                          block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                          block_ms=round(ms_b, 4),
                          module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                          module_ms=round(ms_m, 4)))
        del m, bb, bf
        # the training-time mixture forward: every block refined, residual
        # scaled by its score
        m = DeviceModel(shape(base, soft=True), inp)
        bb = Bound(m, H.HSMLA_OP_BLOCK, prepared=True)
        ms_b = time_steps(lambda: bb.block(x), n_sw, 10)
        bf = Bound(m, H.HSMLA_OP_FORWARD, prepared=True)
        ms_m = time_steps(lambda: bf.forward(x), n_sw, 10)
        sweep.append(dict(routing="soft_mixture", routed_fraction=1.0,
                          block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                          block_ms=round(ms_b, 4),
                          module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                          module_ms=round(ms_m, 4)))
        del m, bb, bf
        # the gate's depthwise 3x3 (FT 3.2 head-level score) with the
        # identity + 3x3 + 5x5 + 7x7 branches, top-k at the base keep ratio
        wl = scaled(base, branches=(3, 5, 7), gate_conv=True)
        m = DeviceModel(shape(wl), make_inputs(wl))
        bb = Bound(m, H.HSMLA_OP_BLOCK, prepared=True)
        ms_b = time_steps(lambda: bb.block(x), n_sw, 10)
        bf = Bound(m, H.HSMLA_OP_FORWARD, prepared=True)
        ms_m = time_steps(lambda: bf.forward(x), n_sw, 10)
        sweep.append(dict(variant="gate_dwconv3x3+branches_3_5_7", keep=base.keep,
                          keep_blocks=base.keep_blocks,
                          block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                          block_ms=round(ms_b, 4),
                          module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                          module_ms=round(ms_m, 4)))
        del m, bb, bf

    cpu = None if args.no_cpu_baseline else cpu_baseline(base, args.cpu_rows)

    line = {
        "metric": "HSMLA fwd tokens/s (bf16, 1 MI355X) + % HBM/MFMA roofline vs keep-ratio",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded street-scene-like field; random-init weights)",
        "config": {"workload": "hsmla_block_forward", "batch": base.batch,
                   "grid": [base.grid_h, base.grid_w], "tokens": tokens,
                   "channels": base.channels, "heads": base.heads,
                   "head_dim": base.head_dim, "branches": list(base.branches),
                   "block": base.block, "window": base.window, "keep": base.keep,
                   "keep_blocks": base.keep_blocks, "gate_conv": base.gate_conv,
                   "streams": args.streams, "weights_prepared": True},
        ("one_stream_ms_per_step" if args.streams == 2 else
         "two_stream_ms_per_step"): round(ms_alt, 4),
        "unprepared_ms_per_step": round(ms_plain, 4),
        "spinup_ms": args.spinup_ms,
        "prep_us": prep_us,
        "roofline": roof,
        "kernels": kernels,
        "selection_gap": gaps,
        "probes": probe,
        "power": dict(power.summary() or {}, steady_ms_per_step=round(steady_ms, 4),
                      seconds=args.power_s),
        "configs": configs,
        "sweep": sweep,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
