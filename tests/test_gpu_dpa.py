"""GPU parity of the residual-aware chunk allocation ("DPA-MoE: A Runtime
Precision Control Framework for MoE Inference", abstract) against the CPU
oracle, through the C ABI.

Bars: per-expert residuals within relative 1e-12 (float64 sums in different
orders); per-pair widths bit-exact when the oracle allocates on the GPU's
own gates and residuals (the allocation is a pure function of them); decode
layers at the resulting widths (1 to 4 planes mixed inside experts) within
the FFN's bars on every row."""
import sys

import numpy as np
import pytest
import torch

from dynamic_any_precision_amd import binding as bd
from dynamic_any_precision_amd import workloads as wl
import oracle as orc

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


_cache = {}


def workload(i, **kw):
    key = (i, tuple(sorted(kw.items())))
    if key not in _cache:
        _cache.clear()
        cfg = wl.config(i, **kw)
        w = wl.make_workload(cfg, keep_codes=False)
        dev = dict(routed=bd.DeviceBank.from_host(w.routed), x=bd.bf16_tensor(w.x_bf16),
                   w_router=torch.from_numpy(w.w_router).cuda(),
                   bias=torch.from_numpy(w.logit_bias).cuda() if w.logit_bias is not None else None)
        _cache[key] = (w, dev, orc.bank_cache(w.routed))
    return _cache[key]


def test_dpa_residuals_tiny_all_experts():
    w, dev, oc = workload(1)
    note("dpa residuals cfg1")
    r = bd.dpa_residuals(dev["routed"]).cpu().numpy()
    assert np.allclose(r, orc.expert_residuals(oc), rtol=1e-12, atol=0)
    assert np.all(r[:, 3] == 0.0)


def test_dpa_residuals_deepseek_sampled_experts():
    # an 11-block down projection (f = 1408)
    w, dev, oc = workload(3)
    note("dpa residuals cfg3 (experts 0, 33, 63)")
    r = bd.dpa_residuals(dev["routed"]).cpu().numpy()
    ex = [0, 33, 63]
    assert np.allclose(r[ex], orc.expert_residuals(oc, experts=ex)[ex], rtol=1e-12, atol=0)


@pytest.mark.parametrize("case", [(1, None), (2, None), (2, 1), (3, None), (4, None)])
def test_dpa_alloc_exact_on_gpu_gates(case):
    i, T = case
    w, dev, oc = workload(i)
    cfg = w.cfg
    x = dev["x"] if T is None else dev["x"][:T].contiguous()
    idx, gate = bd.route(x, dev["w_router"], dev["bias"], cfg.k)
    resid = bd.dpa_residuals(dev["routed"])
    r_np = resid.cpu().numpy()
    g_np, i_np = gate.cpu().numpy().ravel(), idx.cpu().numpy().ravel()
    for b_lo in (1, 2, 3):
        for target in (1.0, 1.5, 2.0, 2.25, 2.5, 3.0, 3.5, 4.0):
            if target < b_lo:
                continue
            note(f"dpa alloc cfg{i} T={x.shape[0]} b_lo={b_lo} target={target}")
            nch = torch.zeros(1, dtype=torch.int32, device="cuda")
            bits = bd.dpa_alloc(gate.reshape(-1), idx.reshape(-1), resid, b_lo, 4, target, n_chunks=nch)
            torch.cuda.synchronize()
            ref, n, budget = orc.dpa_allocate(g_np, i_np, r_np, b_lo, 4, target)
            assert np.array_equal(bits.cpu().numpy().astype(np.int64), ref), (b_lo, target)
            assert int(nch.item()) == n


@pytest.mark.parametrize("target", [1.75, 2.5, 3.0])
def test_dpa_decode_layer_every_row(target):
    # Qwen-shaped decode batch: widths 1..4 mixed inside experts through the
    # unchanged FFN, against the oracle on every row
    w, dev, oc = workload(2)
    cfg = w.cfg
    idx, gate = bd.route(dev["x"], dev["w_router"], None, cfg.k)
    resid = bd.dpa_residuals(dev["routed"])
    bits = bd.dpa_alloc(gate.reshape(-1), idx.reshape(-1), resid, 1, 4, target)
    note(f"dpa decode cfg2 T=32 target={target}")
    y = bd.anyprec_ffn(dev["routed"], None, dev["x"], idx, gate, bits)
    torch.cuda.synchronize()
    idx_np, gate_np, bits_np = idx.cpu().numpy(), gate.cpu().numpy().astype(np.float64), bits.cpu().numpy()
    ref = orc.combine(w.x_bf16, idx_np, gate_np, bits_np, oc)
    got = y.cpu().numpy().astype(np.float64)
    per_row = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    overall = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"[parity] dpa decode target={target}: widths {np.bincount(bits_np, minlength=5)[1:].tolist()}, "
          f"mean {bits_np.mean():.3f}, overall_rel_l2={overall:.3e} max_row_rel_l2={per_row.max():.3e}", flush=True)
    assert overall < 1e-3 and per_row.max() < 5e-3
