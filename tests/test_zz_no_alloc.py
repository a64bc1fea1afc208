"""The static-scratch layer entry point (moe_layer_static) against moe_layer
on a caller workspace: identical routing, widths and outputs, on two calls
in a row with the second smaller, on a second workload with shared experts,
and a clear error for a batch beyond the static array."""
import sys

import numpy as np
import pytest
import torch

from dynamic_any_precision_amd import binding as bd
from dynamic_any_precision_amd import workloads as wl

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def _dev(i):
    w = wl.make_workload(wl.config(i), keep_codes=False)
    return w, dict(routed=bd.DeviceBank.from_host(w.routed),
                   shared=bd.DeviceBank.from_host(w.shared) if w.shared is not None else None,
                   x=bd.bf16_tensor(w.x_bf16), w_router=torch.from_numpy(w.w_router).cuda())


def _both(w, dev, T, accumulate=False):
    cfg = w.cfg
    x = dev["x"][:T].contiguous()
    y0 = torch.from_numpy(np.random.default_rng(T).standard_normal((T, cfg.d)).astype(np.float32)).cuda()
    ya = bd.layer(dev["routed"], dev["shared"], x, dev["w_router"], None, cfg.k, cfg.b_lo, cfg.target,
                  y=y0.clone(), accumulate=accumulate)
    yb = bd.layer_static(dev["routed"], dev["shared"], x, dev["w_router"], None, cfg.k, cfg.b_lo, cfg.target,
                         y=y0.clone(), accumulate=accumulate)
    torch.cuda.synchronize()
    for a, b, name in zip(ya, yb, ("y", "idx", "gate", "bits")):
        assert torch.equal(a, b), (T, name)


def test_static_layer_equals_layer_qwen_two_calls():
    w, dev = _dev(2)
    assert bd.lib().moe_layer_static_scratch_bytes() == 64 << 20
    note("layer_static cfg2 T=32 then T=5, T=1")
    _both(w, dev, 32)
    _both(w, dev, 5, accumulate=True)
    _both(w, dev, 1)                   # the one-token plan kernel on the static array
    _both(w, dev, 1, accumulate=True)
    _both(w, dev, 32)


def test_static_layer_equals_layer_deepseek_shared():
    w, dev = _dev(3)
    note("layer_static cfg3 T=16 then T=3, T=1")
    _both(w, dev, 16)
    _both(w, dev, 3)
    _both(w, dev, 1)


def test_static_layer_rejects_batches_beyond_the_array():
    w, dev = _dev(1)
    cfg = w.cfg
    x = bd.bf16_tensor(wl.step_activations(cfg, 0, 20000))
    need = bd.lib().moe_layer_workspace_bytes(bd.ctypes.byref(dev["routed"].struct()), None, 20000, cfg.k)
    assert need > bd.lib().moe_layer_static_scratch_bytes()
    note("layer_static too large")
    with pytest.raises(bd.MoeError) as ei:
        bd.layer_static(dev["routed"], None, x, dev["w_router"], None, cfg.k, cfg.b_lo, cfg.target)
    assert ei.value.status == 5
    # the entry point still works after the rejection
    _both(w, dev, 16)
