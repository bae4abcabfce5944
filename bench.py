#!/usr/bin/env python3
"""Throughput of the HSMLA block forward on one MI355X.

Workload: 2 images of 128 x 256 tokens, C = 384 (12 heads of 32), bf16,
identity + 3x3 + 5x5 depthwise branches, 8 x 8 blocks, 16 x 16 softmax
windows, keep ratio 10% (52 of 512 blocks per image), wrapped in the LN /
FFN-DWConv block.  One step = one call of hsmla_block_forward over the batch
on one stream (--streams 2: hsmla_block_forward_split, the two images on two
streams), i.e. every kernel of the path; the other mode is timed beside it.  Inputs are seeded synthetic data
(street-scene-like smooth field plus noise) already resident in HBM.

Prints one JSON line: tokens/s, the per-kernel breakdown from HIP events
recorded between the launches of the step, the roofline of the dominant
kernel, a keep-ratio sweep with two threshold-routing points, per-head
routing, the training-time mixture forward and the exact-gate / three-branch
variant, and the CPU oracle timed on a bounded crop.

    python bench.py [--steps K] [--warmup W] [--no-sweep] [--no-cpu-baseline]
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first copy 1 GiB with a plain device copy (a known "
                         "byte count for calibrating HBM traffic counters)")
    ap.add_argument("--cpu-rows", type=int, default=128,
                    help="token rows of the crop the CPU oracle is timed on")
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


def roofline_entry(name, wl, sel, avg_ms):
    by, fl = algorithmic_work(name, wl, sel)
    t_hbm = by / (HBM_PEAK_GBS * 1e9)
    t_mfma = fl / (MFMA_BF16_TFLOPS * 1e12)
    sec = avg_ms * 1e-3
    if name in ("qkv_gemm", "out_proj", "out_proj_residual", "ffn1_gemm",
                "ffn2_gemm_residual", "sparse_softmax") and t_mfma > t_hbm:
        ach = fl / sec / 1e12
        return dict(bound="mfma", achieved=round(ach, 2), peak=MFMA_BF16_TFLOPS,
                    unit="TFLOP/s", frac=round(ach / MFMA_BF16_TFLOPS, 4),
                    traffic=None)
    ach = by / sec / 1e9
    return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS,
                unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4), traffic=None)


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

def cpu_baseline(wl, rows):
    import oracle as O  # test infrastructure, timed here as a baseline only
    from workloads import make_inputs, scaled
    crop = scaled(wl, grid_h=rows)
    inp = make_inputs(crop)
    t0 = time.perf_counter()
    O.hsmla_block_forward(inp["x"], inp, staged=True, **crop.kwargs())
    dt = time.perf_counter() - t0
    try:
        import threadpoolctl
        cores = max(i["num_threads"] for i in threadpoolctl.threadpool_info())
    except Exception:
        cores = os.cpu_count()
    return dict(value=round(crop.batch * crop.tokens / dt, 1), unit="tokens/s",
                cores=cores,
                kind="oracle",
                sample=(f"{crop.batch} images of {rows}x{wl.grid_w} tokens "
                        f"({crop.batch * crop.tokens} tokens, keep {crop.keep_blocks} of "
                        f"{crop.num_blocks} blocks), float64 bf16-staged block "
                        f"forward, one run of {dt:.1f} s"))


# ---------------------------------------------------------------------------

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
    if args.copy_probe:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
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

    def time_steps(model, fn, steps, warmup):
        ws = model.workspace(H.HSMLA_OP_BLOCK)
        out = model.act()
        for _ in range(warmup):
            fn(model, ws, out)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            fn(model, ws, out)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps, ws

    two = H.SplitStreams()
    split = two if args.streams == 2 else None

    def one_stream_step(m, ws, out):
        H.hsmla_block_forward(m.desc, m.weights, m.ffn, x, out, ws)

    def two_stream_step(m, ws, out):
        H.hsmla_block_forward_split(m.desc, m.weights, m.ffn, x, out, ws, two)

    def block_step(m, ws, out):
        if split is None:
            H.hsmla_block_forward(m.desc, m.weights, m.ffn, x, out, ws)
        else:
            H.hsmla_block_forward_split(m.desc, m.weights, m.ffn, x, out, ws, split)

    def module_step(m, ws, out):
        H.hsmla_forward(m.desc, m.weights, x, out, ws)

    model = DeviceModel(shape(base), inp)
    ms, ws = time_steps(model, block_step, args.steps, args.warmup)
    ms_alt = time_steps(model, one_stream_step if split is not None else
                        two_stream_step, args.steps, args.warmup)[0]
    tokens = base.batch * base.tokens
    base_views = model.views(H.HSMLA_OP_BLOCK, ws)
    sel = base_views["sel"].cpu().numpy()
    base_scores = base_views["scores"].cpu().numpy()

    # per-kernel durations from events recorded between the launches
    hev = HipEvents()
    evs = hev.create(32)
    out = model.act()
    per = {}
    names = None
    for i in range(args.warmup + args.steps):
        names = H.hsmla_block_forward_timed(model.desc, model.weights, model.ffn,
                                            x, out, ws, evs)
        if i < args.warmup:
            continue
        hev.sync(evs[len(names) - 1])
        for j in range(len(names) - 1):
            per.setdefault(names[j], []).append(hev.elapsed_ms(evs[j], evs[j + 1]))
    torch.cuda.synchronize()
    hev.destroy(evs)
    kernels = {}
    for n, v in per.items():
        avg = float(np.mean(v))
        by, fl = algorithmic_work(n, base, sel)
        kernels[n] = dict(avg_us=round(avg * 1e3, 2), bytes=int(by), flops=int(fl),
                          gbs=round(by / (avg * 1e-3) / 1e9, 1) if by else None)
    dominant = max(kernels, key=lambda n: kernels[n]["avg_us"])
    roof = roofline_entry(dominant, base, sel, kernels[dominant]["avg_us"] * 1e-3)
    roof["kernel"] = dominant
    roof["traffic"] = measured_traffic(dominant)
    by, fl = algorithmic_work(dominant, base, sel)
    roof["work_per_launch"] = {"bytes": int(by), "flops": int(fl)}

    sweep = []
    if not args.no_sweep:
        for r in (0.0, 0.05, 0.10, 0.25, 0.50):
            wl = scaled(base, keep=r)
            m = DeviceModel(shape(wl), inp)
            ms_b, _ = time_steps(m, block_step, max(10, args.steps // 2), 10)
            ms_m, _ = time_steps(m, module_step, max(10, args.steps // 2), 10)
            sweep.append(dict(keep=r, keep_blocks=keep_blocks_for(r, wl.num_blocks),
                              block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                              block_ms=round(ms_b, 4),
                              module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                              module_ms=round(ms_m, 4)))
            del m
        # threshold routing (blocks with score > tau), tau placed between two
        # adjacent scores of the run above at the given quantile
        uniq = np.unique(base_scores.astype(np.float32))
        for q in (0.9, 0.7):
            i = min(int(q * (uniq.size - 1)), uniq.size - 2)
            tau = float(np.float32((np.float64(uniq[i]) + np.float64(uniq[i + 1])) / 2))
            m = DeviceModel(shape(base, tau=tau), inp)
            ms_b, ws_t = time_steps(m, block_step, max(10, args.steps // 2), 10)
            routed = int(m.views(H.HSMLA_OP_BLOCK, ws_t)["counts"].sum().item())
            ms_m, _ = time_steps(m, module_step, max(10, args.steps // 2), 10)
            sweep.append(dict(routing="threshold", tau=tau,
                              routed_fraction=round(routed / (base.batch * base.num_blocks), 4),
                              block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                              block_ms=round(ms_b, 4),
                              module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                              module_ms=round(ms_m, 4)))
            del m

        # per-head routing (each head by its own score), tau between two
        # adjacent head scores of a first per-head run at the 0.7 quantile
        m = DeviceModel(shape(base, tau=0.5, per_head=True), inp)
        _, ws_p = time_steps(m, block_step, 1, 0)
        hs = m.views(H.HSMLA_OP_BLOCK, ws_p)["head_scores"].cpu().numpy()
        uniq = np.unique(hs.astype(np.float32))
        i = min(int(0.7 * (uniq.size - 1)), uniq.size - 2)
        tau = float(np.float32((np.float64(uniq[i]) + np.float64(uniq[i + 1])) / 2))
        del m
        m = DeviceModel(shape(base, tau=tau, per_head=True), inp)
        ms_b, ws_t = time_steps(m, block_step, max(10, args.steps // 2), 10)
        routed = int(m.views(H.HSMLA_OP_BLOCK, ws_t)["counts"].sum().item())
        ms_m, _ = time_steps(m, module_step, max(10, args.steps // 2), 10)
        sweep.append(dict(routing="threshold_per_head", tau=tau,
                          routed_fraction=round(routed / (base.batch * base.num_blocks
                                                          * base.heads), 4),
                          block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                          block_ms=round(ms_b, 4),
                          module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                          module_ms=round(ms_m, 4)))
        del m
        # the training-time mixture forward: every block refined, residual
        # scaled by its score
        m = DeviceModel(shape(base, soft=True), inp)
        ms_b, _ = time_steps(m, block_step, max(10, args.steps // 2), 10)
        ms_m, _ = time_steps(m, module_step, max(10, args.steps // 2), 10)
        sweep.append(dict(routing="soft_mixture", routed_fraction=1.0,
                          block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                          block_ms=round(ms_b, 4),
                          module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                          module_ms=round(ms_m, 4)))
        del m
        # the gate's depthwise 3x3 (FT 3.2 head-level score) with the
        # identity + 3x3 + 5x5 + 7x7 branches, top-k at the base keep ratio
        wl = scaled(base, branches=(3, 5, 7), gate_conv=True)
        m = DeviceModel(shape(wl), make_inputs(wl))
        ms_b, _ = time_steps(m, block_step, max(10, args.steps // 2), 10)
        ms_m, _ = time_steps(m, module_step, max(10, args.steps // 2), 10)
        sweep.append(dict(variant="gate_dwconv3x3+branches_3_5_7", keep=base.keep,
                          keep_blocks=base.keep_blocks,
                          block_tokens_per_s=round(tokens / (ms_b * 1e-3), 1),
                          block_ms=round(ms_b, 4),
                          module_tokens_per_s=round(tokens / (ms_m * 1e-3), 1),
                          module_ms=round(ms_m, 4)))
        del m

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
                   "streams": args.streams},
        ("one_stream_ms_per_step" if split is not None else
         "two_stream_ms_per_step"): round(ms_alt, 4),
        "roofline": roof,
        "kernels": kernels,
        "sweep": sweep,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
