"""The allocation-free K/V-state entry point against the workspace one.

hsmla_linear_attn_noalloc runs the kernels of hsmla_linear_attn with its
chunk partials in the library's static device array instead of a caller
workspace, so its outputs must equal hsmla_linear_attn's bit for bit; two
calls in a row, the second on a smaller input, check that the array's
leftover contents from the first call do not leak into the second.  Sizes
beyond the array are refused on the host before any launch.
"""

import numpy as np
import pytest
import torch

from efficient_vision_attention_amd import hsmla as H
from efficient_vision_attention_amd.device import DeviceModel, to_device, to_host
from workloads import WORKLOADS, make_inputs, scaled

from gpu_harness import announce, shape_of

pytestmark = pytest.mark.gpu

CASES = [
    # the benchmark's block shape first (largest partials), then smaller ones
    scaled(WORKLOADS["block"], name="na_block", keep=0.1),
    scaled(WORKLOADS["street"], name="na_street", batch=2, grid_h=32, grid_w=64),
    scaled(WORKLOADS["street"], name="na_ragged", batch=3, grid_h=20, grid_w=36,
           channels=96, heads=3, block=4, window=10),
    scaled(WORKLOADS["tiny"], name="na_f32", batch=2, grid_h=12, grid_w=28,
           channels=96, heads=3, block=4, window=10),
]


def _qkv_hat(wl):
    rng = np.random.default_rng(wl.tokens + wl.channels)
    a = rng.standard_normal((wl.batch, wl.tokens, 3 * wl.channels))
    return to_device(a, wl.dtype)  # rounded once to the run dtype


def _run_both(wl):
    m = DeviceModel(shape_of(wl), make_inputs(wl))
    qkvh = _qkv_hat(wl)
    B, Hh = wl.batch, wl.heads
    outs = []
    for noalloc in (False, True):
        o = m.act()
        kv = torch.full((B, Hh, 32, 32), float("nan"), device="cuda")
        ksum = torch.full((B, Hh, 32), float("nan"), device="cuda")
        announce(f"hsmla_linear_attn{'_noalloc' if noalloc else ''} {wl.name} "
                 f"B={B} {wl.grid_h}x{wl.grid_w} C={wl.channels} {wl.dtype}")
        if noalloc:
            H.hsmla_linear_attn_noalloc(m.desc, qkvh, o, kv, ksum)
        else:
            H.hsmla_linear_attn(m.desc, qkvh, o, kv, ksum,
                                m.workspace(H.HSMLA_OP_LINEAR))
        torch.cuda.synchronize()
        outs.append((o, kv, ksum))
    return outs


@pytest.mark.parametrize("pair", [(0, 1), (1, 2), (2, 3)])
def test_noalloc_equals_workspace_entry_two_calls(pair):
    """Two calls in a row, the second on a smaller input: each equals the
    workspace entry point bit for bit."""
    for i in pair:
        (o, kv, ks), (o2, kv2, ks2) = _run_both(CASES[i])
        assert torch.equal(o, o2), CASES[i].name
        assert torch.equal(kv, kv2), CASES[i].name
        assert torch.equal(ks, ks2), CASES[i].name
        assert np.isfinite(to_host(kv2)).all()


def test_noalloc_rejects_sizes_beyond_the_scratch():
    wl = scaled(WORKLOADS["block"], name="na_big", batch=8, grid_h=256, grid_w=256)
    m = DeviceModel(shape_of(wl), make_inputs(scaled(wl, batch=1, grid_h=16,
                                                          grid_w=16)))
    need = H.hsmla_workspace_bytes(m.desc, H.HSMLA_OP_LINEAR)
    assert need > 16 << 20
    t = torch.empty(16, dtype=torch.uint8, device="cuda")  # never read
    with pytest.raises(H.HsmlaError) as e:
        H.hsmla_linear_attn_noalloc(m.desc, t, t, t, t)
    assert e.value.status == H.HSMLA_ERR_SCRATCH
