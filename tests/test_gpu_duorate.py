"""GPU parity of the DuoRate per-expert allocator ("DuoRate: Two-Rate
Per-Expert Precision Allocation for Mixture-of-Experts Serving", abstract)
against the CPU oracle, through the C ABI.

Bars: the prefill profile bit-exact (both sides add the same exact squares
in pair order); the baked distortion tensor and the per-token distortions
within relative 1e-12 (float64 sums in different orders); the per-expert
widths and the multiplier bit-exact when the oracle's solve runs on the
GPU's own distortions (the solve is a pure function of them), and equal to
the fully independent oracle chain on the tiny layer; decode layers that
read every pair at its expert's width within the FFN's bars."""
import sys

import numpy as np
import pytest
import torch

from dynamic_any_precision_amd import binding as bd
from dynamic_any_precision_amd import workloads as wl
import oracle as orc

pytestmark = pytest.mark.gpu

REL = 1e-12


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


def test_duorate_bake_tiny_all_experts():
    w, dev, oc = workload(1)
    note("duorate bake cfg1")
    delta = bd.duorate_bake(dev["routed"]).cpu().numpy()
    ref = orc.distortion_tensor(oc)
    assert np.allclose(delta, ref, rtol=REL, atol=0)
    assert np.all(delta[:, 3] == 0.0)


def test_duorate_bake_qwen_sampled_experts():
    w, dev, oc = workload(2)
    note("duorate bake cfg2 (experts 0, 37, 127)")
    delta = bd.duorate_bake(dev["routed"]).cpu().numpy()
    ex = [0, 37, 127]
    ref = orc.distortion_tensor(oc, experts=ex)
    assert np.allclose(delta[ex], ref[ex], rtol=REL, atol=0)


def _profile_case(i, T=None):
    w, dev, oc = workload(i)
    cfg = w.cfg
    x, x_np = dev["x"], w.x_bf16
    if T is not None:
        x, x_np = x[:T].contiguous(), x_np[:T]
    idx, _ = bd.route(x, dev["w_router"], dev["bias"], cfg.k)
    a, n = bd.duorate_profile(x, idx, cfg.E)
    torch.cuda.synchronize()
    return w, dev, oc, x_np, idx, a, n


@pytest.mark.parametrize("case", [(1, None), (2, None), (4, None), (4, 777)])
def test_duorate_profile_bit_exact(case):
    i, T = case
    note(f"duorate profile cfg{i} T={T}")
    w, dev, oc, x_np, idx, a, n = _profile_case(i, T)
    ra, rn = orc.prefill_profile(x_np, idx.cpu().numpy(), w.cfg.E)
    assert np.array_equal(n.cpu().numpy(), rn)
    assert np.array_equal(a.cpu().numpy(), ra)


def test_duorate_profile_skips_out_of_range_and_empty():
    w, dev, oc = workload(1)
    cfg = w.cfg
    idx, _ = bd.route(dev["x"], dev["w_router"], None, cfg.k)
    bad = idx.clone()
    bad[2, 0] = cfg.E + 5
    bad[7, 1] = -1
    note("duorate profile out-of-range entries")
    a, n = bd.duorate_profile(dev["x"], bad, cfg.E)
    torch.cuda.synchronize()
    keep = bad.cpu().numpy().copy()
    ra = np.zeros((cfg.E, cfg.d))
    rn = np.zeros(cfg.E, dtype=np.int64)
    x = wl.bf16_bits_to_f32(w.x_bf16).astype(np.float64)
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = keep[t, j]
            if 0 <= e < cfg.E:
                ra[e] += x[t] * x[t]
                rn[e] += 1
    assert np.array_equal(n.cpu().numpy(), rn) and np.array_equal(a.cpu().numpy(), ra)
    a0, n0 = bd.duorate_profile(dev["x"][:0], idx[:0], cfg.E)
    torch.cuda.synchronize()
    assert not a0.cpu().numpy().any() and not n0.cpu().numpy().any()


@pytest.mark.parametrize("b_lo", [1, 2])
def test_duorate_solve_exact_on_gpu_distortion_prefill(b_lo):
    # the Qwen-shaped prefill (T=4096, Zipf load) profiles the workload; the
    # solve's widths and multiplier must equal the oracle's solve run on the
    # GPU's distortions, at every target
    w, dev, oc, x_np, idx, a, n = _profile_case(4)
    cfg = w.cfg
    delta = bd.duorate_bake(dev["routed"])
    a_np, n_np, d_np = a.cpu().numpy(), n.cpu().numpy().astype(np.int64), delta.cpu().numpy()
    for target in (1.0, 1.5, 2.0, 2.3, 2.5, 2.9, 3.0, 3.5, 4.0):
        if target < b_lo:
            continue
        note(f"duorate solve cfg4 b_lo={b_lo} target={target}")
        wts, D, lam = bd.duorate_solve(delta, a, n, b_lo, cfg.b_max, target)
        torch.cuda.synchronize()
        D_np = D.cpu().numpy()
        assert np.allclose(D_np, orc.expert_distortion(d_np, a_np, n_np), rtol=REL, atol=0)
        ref_w, ref_lam = orc.duorate_widths(D_np, n_np, b_lo, cfg.b_max, target)
        assert np.array_equal(wts.cpu().numpy().astype(np.int64), ref_w), target
        assert float(lam.item()) == ref_lam, (target, float(lam.item()), ref_lam)
        rate = float(np.dot(n_np, ref_w)) / n_np.sum()
        assert rate <= target + 1e-12
        print(f"[duorate] b_lo={b_lo} target={target}: decode rate {rate:.4f}, lambda {ref_lam:.6g}, "
              f"widths {np.bincount(ref_w, minlength=5)[1:].tolist()}", flush=True)


def test_duorate_tiny_fully_independent_chain():
    # bake, profile, distortion and solve all computed by the oracle from the
    # stored bank and the oracle's own routing, against the GPU chain
    w, dev, oc, x_np, idx, a, n = _profile_case(1)
    cfg = w.cfg
    oidx, _, gap, _ = orc.route(x_np, w.w_router, None, cfg.k)
    assert np.array_equal(idx.cpu().numpy()[gap >= 1e-5], oidx[gap >= 1e-5])
    delta = bd.duorate_bake(dev["routed"])
    ra, rn = orc.prefill_profile(x_np, oidx, cfg.E)
    rD = orc.expert_distortion(orc.distortion_tensor(oc), ra, rn)
    for b_lo in (1, 2):
        for target in (1.5, 2.0, 2.5, 3.0, 3.5):
            if target < b_lo:
                continue
            note(f"duorate chain cfg1 b_lo={b_lo} target={target}")
            wts, D, lam = bd.duorate_solve(delta, a, n, b_lo, cfg.b_max, target)
            torch.cuda.synchronize()
            ref_w, ref_lam = orc.duorate_widths(rD, rn, b_lo, cfg.b_max, target)
            assert np.array_equal(wts.cpu().numpy().astype(np.int64), ref_w), (target, wts, ref_w)
            assert abs(float(lam.item()) - ref_lam) <= 1e-12 * max(1.0, ref_lam)


def test_bits_from_expert_widths_exact():
    rng = np.random.default_rng(3)
    E, P = 64, 3001
    idx = rng.integers(0, E, size=P).astype(np.int32)
    idx[[5, 77, 3000]] = [E, -1, E + 100]
    wts = rng.integers(1, 5, size=E).astype(np.uint8)
    note("bits from expert widths")
    bits = bd.bits_from_expert_widths(torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda())
    torch.cuda.synchronize()
    ref = np.where((idx >= 0) & (idx < E), wts[np.clip(idx, 0, E - 1)], 0)
    assert np.array_equal(bits.cpu().numpy(), ref)


@pytest.mark.parametrize("target", [2.3, 2.9])
def test_duorate_decode_layer_every_row(target):
    # widths solved on a Qwen-shaped prefill profile, then a T=32 decode batch
    # of the same layer read at those per-expert widths through the unchanged
    # FFN, against the oracle on every row
    w, dev, oc, x_np, idx, a, n = _profile_case(4)
    cfg = w.cfg
    delta = bd.duorate_bake(dev["routed"])
    wts, _, _ = bd.duorate_solve(delta, a, n, 1, cfg.b_max, target)
    xs_np = wl.step_activations(cfg, 900, 32)
    xs = bd.bf16_tensor(xs_np)
    didx, dgate = bd.route(xs, dev["w_router"], dev["bias"], cfg.k)
    bits = bd.bits_from_expert_widths(didx, wts)
    note(f"duorate decode cfg4 layer T=32 target={target}")
    y = bd.anyprec_ffn(dev["routed"], None, xs, didx, dgate, bits)
    torch.cuda.synchronize()
    idx_np, gate_np, bits_np = didx.cpu().numpy(), dgate.cpu().numpy().astype(np.float64), bits.cpu().numpy()
    assert np.array_equal(bits_np, orc.pair_bits_from_expert_widths(idx_np, wts.cpu().numpy()))
    ref = orc.combine(xs_np, idx_np, gate_np, bits_np, oc)
    got = y.cpu().numpy().astype(np.float64)
    per_row = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    overall = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"[parity] duorate decode target={target}: widths read {sorted(set(bits_np.tolist()))}, "
          f"overall_rel_l2={overall:.3e} max_row_rel_l2={per_row.max():.3e}", flush=True)
    assert overall < 1e-3 and per_row.max() < 5e-3
