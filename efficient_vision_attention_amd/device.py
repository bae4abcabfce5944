"""Host <-> device marshalling for the binding (no computation).

``DeviceModel`` holds the device copies of one set of weights plus the
descriptor, and runs the C entry points on tensors it is given.
"""

from __future__ import annotations

import numpy as np
import torch

from . import hsmla as H

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(a, dtype: str, device="cuda"):
    """float64 numpy array (values exact in `dtype`) -> contiguous tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return t.to(torch.float32).to(TORCH_DTYPE[dtype]).to(device).contiguous()


def to_f32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host(t):
    return t.detach().to("cpu", torch.float64).numpy()


class DeviceModel:
    """Device weights and descriptor for one shape.

    shape: mapping with batch, grid_h, grid_w, channels, heads, branches,
    block, window, keep_blocks, dtype, and optionally tau (threshold
    routing when given), per_head (route each head by its own score) and
    soft (the training-time mixture over every block).  weights: dict of float64 numpy
    arrays (w_qkv, w_o, dw list, gate_w, gate_b, optionally gate_dw, and
    for the block ln1_g,
    ln1_b, ln2_g, ln2_b, w1, dw_ffn, w2), dense weights [in][out]
    (y = x @ W), the library's layout.
    """

    def __init__(self, shape: dict, weights: dict, device="cuda"):
        self.shape = dict(shape)
        self.dtype = shape["dtype"]
        self.device = device
        self.desc = H.make_desc(**self.shape)
        dt = self.dtype
        self.t = {
            "w_qkv": to_device(weights["w_qkv"], dt, device),
            "w_o": to_device(weights["w_o"], dt, device),
            "dw": [to_device(w, dt, device) for w in weights["dw"]],
            "gate_w": to_f32(weights["gate_w"], device),
            "gate_b": to_f32(weights["gate_b"], device),
        }
        self.t["gate_dw"] = (to_device(weights["gate_dw"], dt, device)
                             if weights.get("gate_dw") is not None else None)
        self.weights = H.make_weights(self.t["w_qkv"], self.t["w_o"],
                                      self.t["dw"], self.t["gate_w"],
                                      self.t["gate_b"], self.t["gate_dw"])
        self.ffn = None
        if "w1" in weights:
            for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
                self.t[k] = to_f32(weights[k], device)
            self.t["w1"] = to_device(weights["w1"], dt, device)
            self.t["w2"] = to_device(weights["w2"], dt, device)
            self.t["dw_ffn"] = to_device(weights["dw_ffn"], dt, device)
            self.ffn = H.make_ffn_weights(*(self.t[k] for k in (
                "ln1_g", "ln1_b", "ln2_g", "ln2_b", "w1", "dw_ffn", "w2")))

    # -- buffers ---------------------------------------------------------
    def act(self, channels_mult=1):
        s = self.shape
        return torch.empty((s["batch"], s["grid_h"] * s["grid_w"],
                            channels_mult * s["channels"]),
                           dtype=TORCH_DTYPE[self.dtype], device=self.device)

    def workspace(self, op):
        n = H.hsmla_workspace_bytes(self.desc, op)
        return torch.empty(max(n, 16), dtype=torch.uint8, device=self.device)

    def views(self, op, ws):
        """Typed tensors over the intermediates left in a workspace."""
        s = self.shape
        B, N, C, Hh = s["batch"], s["grid_h"] * s["grid_w"], s["channels"], s["heads"]
        T = (s["grid_h"] // s["block"]) * (s["grid_w"] // s["block"])
        soft = s.get("soft", False)
        thr = s.get("tau") is not None and not soft
        ph = thr and s.get("per_head", False)
        k = 0 if soft else Hh * T if ph else T if thr else s["keep_blocks"]
        off = H.hsmla_workspace_views(self.desc, op, ws)
        adt = TORCH_DTYPE[self.dtype]
        esz = torch.tensor([], dtype=adt).element_size()

        def sl(name, count, dtype, size):
            o = off[name]
            return ws[o:o + count * size].view(dtype)

        out = {
            "qkv": sl("qkv", B * N * 3 * C, adt, esz).view(B, N, 3 * C),
            "qkv_hat": sl("qkv_hat", B * N * 3 * C, adt, esz).view(B, N, 3 * C),
            "o": sl("o", B * N * C, adt, esz).view(B, N, C),
            "kv": sl("kv", B * Hh * 32 * 32, torch.float32, 4).view(B, Hh, 32, 32),
            "ksum": sl("ksum", B * Hh * 32, torch.float32, 4).view(B, Hh, 32),
            "scores": sl("scores", B * T, torch.float32, 4).view(B, T),
            "sel": sl("sel", B * k, torch.int32, 4).view(B, k),
        }
        if ph:
            out["sel"] = out["sel"].view(B, Hh, T)
            out["counts"] = sl("counts", B * Hh, torch.int32, 4).view(B, Hh)
            out["head_scores"] = sl("head_scores", B * T * Hh, torch.float32, 4).view(B, T, Hh)
        elif thr:
            out["counts"] = sl("counts", B, torch.int32, 4)
        if off.get("x1") is not None:
            out["x1"] = sl("x1", B * N * C, adt, esz).view(B, N, C)
        return out
