"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: routing indices, per-pair bits and dequantised weights bit-exact (top-k
ties flagged where the oracle's logit gap is below 1e-5); layer outputs within
relative L2 1e-3 (bf16 activations, fp32 accumulation)."""
import sys

import numpy as np
import pytest
import torch

from dynamic_any_precision_amd import binding as bd
from dynamic_any_precision_amd import workloads as wl
import oracle as orc

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
TIE_GAP = 1e-5


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


_cache = {}


def workload(i, **kw):
    key = (i, tuple(sorted(kw.items())))
    if key not in _cache:
        cfg = wl.config(i, **kw)
        w = wl.make_workload(cfg)
        dev = dict(
            routed=bd.DeviceBank.from_host(w.routed),
            shared=bd.DeviceBank.from_host(w.shared) if w.shared is not None else None,
            x=bd.bf16_tensor(w.x_bf16),
            w_router=torch.from_numpy(w.w_router).cuda(),
            bias=torch.from_numpy(w.logit_bias).cuda() if w.logit_bias is not None else None,
        )
        _cache[key] = (w, dev, orc.bank_cache(w.routed), orc.bank_cache(w.shared) if w.shared is not None else None)
    return _cache[key]


# ---------------------------------------------------------------------------
# dequantisation: bit-exact


@pytest.mark.parametrize("cfg_id", [1, 2, 3])
def test_dequant_bit_exact(cfg_id):
    w, dev, oc, _ = workload(cfg_id)
    bank = dev["routed"]
    experts = range(bank.n_experts) if cfg_id == 1 else (0, 37 % bank.n_experts, bank.n_experts - 1)
    for e in experts:
        for m in (0, 1):
            for b in range(1, 5):
                note(f"dequant cfg{cfg_id} e{e} m{m} b{b}")
                got = bd.dequant(bank, e, m, b).cpu().numpy()
                ref = oc.weights(e, b)[m].astype(np.float32)
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (e, m, b)


def test_dequant_shared_bank_bit_exact():
    w, dev, _, sc = workload(3)
    for e in range(2):
        for m in (0, 1):
            note(f"dequant shared e{e} m{m}")
            got = bd.dequant(dev["shared"], e, m, 4).cpu().numpy()
            assert np.array_equal(got, sc.weights(e, 4)[m].astype(np.float32))


# ---------------------------------------------------------------------------
# router


def _check_route(w, dev, renorm=False):
    cfg = w.cfg
    idx, gate = bd.route(dev["x"], dev["w_router"], dev["bias"], cfg.k, renorm)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    gate = gate.cpu().numpy()
    oidx, ogate, gap, _ = orc.route(w.x_bf16, w.w_router, w.logit_bias, cfg.k, renorm)
    flagged = gap < TIE_GAP
    ok = ~flagged
    assert np.array_equal(idx[ok], oidx[ok]), np.nonzero((idx != oidx).any(1) & ok)
    # gates: fp32 rounding of the oracle's fp64 value, up to a few ulps of
    # summation-order difference in the softmax denominator
    assert np.allclose(gate[ok], ogate[ok], rtol=4e-7, atol=1e-30)
    return idx, gate, flagged


@pytest.mark.parametrize("cfg_id", [1, 2, 3])
def test_route_matches_oracle(cfg_id):
    w, dev, _, _ = workload(cfg_id)
    note(f"route cfg{cfg_id}")
    _check_route(w, dev)


def test_route_renorm_and_bias_prefill():
    w, dev, _, _ = workload(4)
    note("route cfg4 (T=4096, Zipf bias)")
    _check_route(w, dev)
    w1, dev1, _, _ = workload(1)
    note("route cfg1 renorm")
    idx, gate, _ = _check_route(w1, dev1, renorm=True)
    assert np.allclose(gate.sum(1), 1.0, atol=1e-6)


@pytest.mark.parametrize("T", [1, 5, 9, 33, 77])
def test_route_ragged_token_counts(T):
    # token counts that leave partial 8-token tiles, from a decode step's own activations
    w, dev, _, _ = workload(2)
    x_np = wl.step_activations(w.cfg, 300 + T, T)
    x = bd.bf16_tensor(x_np)
    note(f"route cfg2 T={T}")
    idx, gate = bd.route(x, dev["w_router"], None, w.cfg.k)
    torch.cuda.synchronize()
    oidx, ogate, gap, _ = orc.route(x_np, w.w_router, None, w.cfg.k)
    ok = gap >= TIE_GAP
    assert np.array_equal(idx.cpu().numpy()[ok], oidx[ok])


@pytest.mark.parametrize("T", [256, 300, 1000])
def test_route_matrix_core_logits_ragged(T):
    # 256 tokens and more take the logits on the fp64 matrix cores (16-token
    # tiles; 300 and 1000 leave a ragged last tile)
    w, dev, _, _ = workload(4)
    x = dev["x"][:T].contiguous()
    note(f"route cfg4 T={T}")
    idx, gate = bd.route(x, dev["w_router"], dev["bias"], w.cfg.k)
    torch.cuda.synchronize()
    oidx, ogate, gap, _ = orc.route(w.x_bf16[:T], w.w_router, w.logit_bias, w.cfg.k)
    ok = gap >= TIE_GAP
    assert np.array_equal(idx.cpu().numpy()[ok], oidx[ok])
    assert np.allclose(gate.cpu().numpy()[ok], ogate[ok], rtol=4e-7, atol=1e-30)


def test_route_exact_ties_go_to_lower_index():
    # duplicate router rows give exactly equal logits
    w, dev, _, _ = workload(1)
    W = w.w_router.copy()
    W[5] = W[2]
    W[7] = W[2]
    Wd = torch.from_numpy(W).cuda()
    note("route exact ties")
    idx, gate = bd.route(dev["x"], Wd, None, 3)
    torch.cuda.synchronize()
    oidx, _, _, _ = orc.route(w.x_bf16, W, None, 3)
    assert np.array_equal(idx.cpu().numpy(), oidx)


def test_route_workspace_reusable():
    w, dev, _, _ = workload(1)
    ws = bd.route_workspace(w.cfg.T, w.cfg.E)
    note("route reuse workspace")
    a = bd.route(dev["x"], dev["w_router"], None, w.cfg.k, workspace=ws)
    b = bd.route(dev["x"], dev["w_router"], None, w.cfg.k, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------------------
# allocation: bit-exact against the oracle run on the GPU's own gates


def _check_alloc(gates_np, b_lo, b_max, target):
    g = torch.from_numpy(np.ascontiguousarray(gates_np, dtype=np.float32)).cuda()
    tau = torch.empty(1, dtype=torch.float32, device="cuda")
    nhi = torch.empty(1, dtype=torch.int32, device="cuda")
    bits = bd.alloc_bits(g, b_lo, b_max, target, tau=tau, n_hi=nhi)
    torch.cuda.synchronize()
    obits, n, ns = orc.allocate_bits(gates_np.astype(np.float64), b_lo, b_max, target)
    assert np.array_equal(bits.cpu().numpy().astype(np.int64), obits)
    assert int(nhi.item()) == n
    if 0 < ns < gates_np.size:
        t = float(tau.item())
        assert int(np.sum(gates_np > t)) == n
    return n, ns


@pytest.mark.parametrize("cfg_id", [1, 2, 3])
def test_alloc_on_routed_gates(cfg_id):
    w, dev, _, _ = workload(cfg_id)
    cfg = w.cfg
    _, gate = bd.route(dev["x"], dev["w_router"], dev["bias"], cfg.k)
    gates = gate.cpu().numpy().ravel()
    for b_lo in ((1, 2) if cfg_id == 3 else (2,)):
        for target in (2.0, 2.25, 2.5, 3.0, 3.75, 4.0):
            if target < b_lo:
                continue
            note(f"alloc cfg{cfg_id} b_lo={b_lo} target={target}")
            n, ns = _check_alloc(gates, b_lo, 4, target)
            avg = (n * 4 + (gates.size - n) * b_lo) / gates.size
            assert abs(avg - target) <= (4 - b_lo) / gates.size + 1e-9 or n < ns


@pytest.mark.parametrize("P", [1, 2, 63, 64, 65, 2047, 2048, 2049, 5000, 32768, 40000])
def test_alloc_sizes_and_ties(P):
    rng = np.random.default_rng(P)
    for kind in ("uniform", "ties", "allsame", "zeros"):
        if kind == "uniform":
            g = rng.random(P).astype(np.float32)
        elif kind == "ties":
            g = (rng.integers(0, 7, P) / 8).astype(np.float32)
        elif kind == "allsame":
            g = np.full(P, 0.125, dtype=np.float32)
        else:
            g = np.zeros(P, dtype=np.float32)
            g[: P // 3] = rng.random(P // 3)
        for target in (2.0, 2.5, 3.0, 3.3, 4.0):
            note(f"alloc P={P} {kind} target={target}")
            _check_alloc(g, 2, 4, target)


# ---------------------------------------------------------------------------
# calibration-threshold mode: tau from the bisection over a calibration set,
# then fixed widths on later batches


@pytest.mark.parametrize("kind", ["routed", "ties"])
def test_calibrated_threshold_and_fixed_widths(kind):
    if kind == "routed":
        # calibration gates of 16 decode batches of the Qwen shape, widths of 4 more
        w, dev, _, _ = workload(2)
        cfg = w.cfg
        wr = dev["w_router"]
        gates = []
        for s in range(20):
            x = bd.bf16_tensor(wl.step_activations(cfg, 500 + s, 32))
            gates.append(bd.route(x, wr, None, cfg.k)[1].reshape(-1))
        cal, held = torch.cat(gates[:16]), torch.cat(gates[16:])
    else:
        rng = np.random.default_rng(31)
        cal = torch.from_numpy((rng.integers(0, 9, 5000) / 16).astype(np.float32)).cuda()
        held = torch.from_numpy((rng.integers(0, 9, 3000) / 16).astype(np.float32)).cuda()
    cal_np = cal.cpu().numpy().astype(np.float64)
    held_np = held.cpu().numpy().astype(np.float64)
    for target in (2.0, 2.5, 3.0, 3.3, 4.0):
        note(f"calibrated threshold {kind} target={target}")
        tau = torch.empty(1, dtype=torch.float32, device="cuda")
        bd.alloc_bits(cal, 2, 4, target, tau=tau)
        torch.cuda.synchronize()
        tau_ref = orc.calibrate_threshold(cal_np, 2, 4, target)
        assert float(tau.item()) == tau_ref, (target, tau.item(), tau_ref)
        bits = bd.bits_from_threshold(held, float(tau.item()), 2, 4)
        torch.cuda.synchronize()
        ref = orc.bits_from_threshold(held_np, tau_ref, 2, 4)
        assert np.array_equal(bits.cpu().numpy().astype(np.int64), ref)


def test_threshold_controller_follows_a_changing_target():
    # a target that changes from step to step (a latency budget following the
    # system load): tau is re-bisected on the device over the stored
    # calibration gates when the target changes, and every step's widths
    # equal the oracle's fixed-threshold widths for that target
    w, dev, _, _ = workload(2)
    cfg = w.cfg
    wr = dev["w_router"]
    cal = torch.cat([bd.route(bd.bf16_tensor(wl.step_activations(cfg, 700 + s, 32)), wr, None, cfg.k)[1].reshape(-1)
                     for s in range(16)])
    cal_np = cal.cpu().numpy().astype(np.float64)
    ctl = bd.ThresholdController(cal, 2, 4)
    targets = [3.0, 3.0, 2.5, 2.5, 2.5, 3.5, 2.0, 4.0, 3.25, 3.25, 2.75, 3.0]
    avgs = []
    for step, target in enumerate(targets):
        x = bd.bf16_tensor(wl.step_activations(cfg, 800 + step, 32))
        _, gate = bd.route(x, wr, None, cfg.k)
        note(f"controller step {step} target {target}")
        bits = ctl.widths(gate, target)
        torch.cuda.synchronize()
        tau_ref = orc.calibrate_threshold(cal_np, 2, 4, target)
        assert float(ctl.tau.item()) == tau_ref, (step, target)
        ref = orc.bits_from_threshold(gate.cpu().numpy().astype(np.float64), tau_ref, 2, 4)
        got = bits.cpu().numpy().astype(np.int64)
        assert np.array_equal(got, ref), (step, target)
        avgs.append(float(got.mean()))
    print("[controller] per-step targets " + " ".join(f"{t:g}" for t in targets), flush=True)
    print("[controller] per-step averages " + " ".join(f"{a:.3f}" for a in avgs), flush=True)


def test_fixed_widths_at_the_threshold_value():
    # scores equal to tau stay low; -inf makes every pair high; empty input
    g = torch.tensor([0.25, 0.5, 0.5, 0.75, 0.0, 1.0], dtype=torch.float32, device="cuda")
    note("fixed widths at tau")
    assert bd.bits_from_threshold(g, 0.5, 1, 4).cpu().tolist() == [1, 1, 1, 4, 1, 4]
    assert bd.bits_from_threshold(g, float("-inf"), 2, 3).cpu().tolist() == [3] * 6
    assert bd.bits_from_threshold(g[:0], 0.5, 2, 4).numel() == 0


# ---------------------------------------------------------------------------
# permutation: stable order by (expert, bits desc, pair id)


@pytest.mark.parametrize("cfg_id", [1, 2, 4])
def test_permute_stable_order(cfg_id):
    w, dev, _, _ = workload(cfg_id)
    cfg = w.cfg
    idx, gate = bd.route(dev["x"], dev["w_router"], dev["bias"], cfg.k)
    bits = bd.alloc_bits(gate.reshape(-1), cfg.b_lo, 4, cfg.target)
    ws = bd.ffn_workspace(dev["routed"], None, cfg.T, cfg.k)
    note(f"permute cfg{cfg_id}")
    sp, eoff, emax = bd.permute(idx, bits, cfg.E, 4, ws)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy().ravel()
    bits_np = bits.cpu().numpy().astype(np.int64)
    pid = np.arange(idx_np.size)
    order = np.lexsort((pid, -bits_np, idx_np))
    assert np.array_equal(sp.cpu().numpy(), order)
    counts = np.bincount(idx_np, minlength=cfg.E)
    assert np.array_equal(eoff.cpu().numpy(), np.concatenate([[0], np.cumsum(counts)]))
    mb = np.zeros(cfg.E, dtype=np.int64)
    np.maximum.at(mb, idx_np, bits_np)
    assert np.array_equal(emax.cpu().numpy(), mb)


def _messy_routing(T, k, E, B, seed):
    """Top-k lists with repeated experts, out-of-range experts and widths
    outside [1, B] mixed in."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    bits = rng.integers(1, B + 1, size=(T, k)).astype(np.uint8)
    u = rng.random((T, k))
    for t, j in zip(*np.nonzero(u < 0.03)):
        if j > 0:
            idx[t, j] = idx[t, rng.integers(0, j)]  # repeat an earlier expert
    idx[u > 0.99] = E + 3
    idx[(u > 0.98) & (u <= 0.985)] = -1
    bits[(u > 0.97) & (u <= 0.975)] = 0
    bits[(u > 0.96) & (u <= 0.965)] = B + 1
    return idx, bits


def _expected_plan(idx, bits, E, B):
    T, k = idx.shape
    keep = np.zeros((T, k), dtype=bool)
    for t in range(T):
        seen = set()
        for j in range(k):
            e, b = int(idx[t, j]), int(bits[t, j])
            if 0 <= e < E and 1 <= b <= B:
                if e not in seen:
                    keep[t, j] = True
                seen.add(e)
    e_f, b_f, k_f = idx.ravel().astype(np.int64), bits.ravel().astype(np.int64), keep.ravel()
    pid = np.nonzero(k_f)[0]
    order = pid[np.lexsort((pid, -b_f[pid], e_f[pid]))]
    sp = np.full(T * k, -1, dtype=np.int64)
    sp[:order.size] = order
    counts = np.bincount(e_f[pid], minlength=E)
    mb = np.zeros(E, dtype=np.int64)
    np.maximum.at(mb, e_f[pid], b_f[pid])
    return sp, np.concatenate([[0], np.cumsum(counts)]), mb


@pytest.mark.parametrize("T,k,E", [(100, 2, 8), (37, 8, 128), (300, 6, 64), (5000, 6, 64), (20000, 8, 128)])
def test_permute_drops_invalid_and_repeated(T, k, E):
    # both plan variants: one block with the words in LDS (small batches) and
    # the three-launch plan (large batches)
    idx, bits = _messy_routing(T, k, E, 4, seed=T)
    ws = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")
    note(f"permute messy T={T} k={k} E={E}")
    sp, eoff, emax = bd.permute(torch.from_numpy(idx).cuda(), torch.from_numpy(bits).cuda(), E, 4, ws)
    torch.cuda.synchronize()
    sp_ref, eoff_ref, mb_ref = _expected_plan(idx, bits, E, 4)
    assert np.array_equal(sp.cpu().numpy(), sp_ref)
    assert np.array_equal(eoff.cpu().numpy(), eoff_ref)
    assert np.array_equal(emax.cpu().numpy(), mb_ref)


# ---------------------------------------------------------------------------
# expert FFN


def _ffn_case(i, bits_np=None, tokens=None, target=None, accumulate=False, T=None, over=None, **kw):
    w, dev, oc, sc = workload(i, **kw, **(over or {}))
    cfg = w.cfg
    x = dev["x"]
    x_np = w.x_bf16
    if T is not None:
        x = x[:T].contiguous()
        x_np = x_np[:T]
    TT = x.shape[0]
    idx, gate = bd.route(x, dev["w_router"], dev["bias"], cfg.k)
    if bits_np is None:
        bits = bd.alloc_bits(gate.reshape(-1), cfg.b_lo, 4, cfg.target if target is None else target)
    else:
        bits = torch.from_numpy(np.ascontiguousarray(bits_np, dtype=np.uint8)).cuda()
    y0 = None
    if accumulate:
        y0 = torch.from_numpy(np.random.default_rng(9).standard_normal((TT, cfg.d)).astype(np.float32)).cuda()
        y = y0.clone()
    else:
        y = None
    y = bd.anyprec_ffn(dev["routed"], dev["shared"], x, idx, gate, bits, y=y, accumulate=accumulate)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    gate_np = gate.cpu().numpy().astype(np.float64)
    b_np = bits.cpu().numpy().astype(np.int64)
    ref = orc.combine(x_np, idx_np, gate_np, b_np, oc, sc, cfg.n_shared, tokens)
    got = y.cpu().numpy().astype(np.float64)
    if accumulate:
        ref = ref + y0.cpu().numpy().astype(np.float64)
    rows = range(TT) if tokens is None else tokens
    rows = list(rows)
    err = rel_l2(got[rows], ref[rows])
    return err, b_np


def test_ffn_tiny_full():
    note("ffn cfg1 target 3.0")
    err, b = _ffn_case(1)
    assert set(np.unique(b)) <= {2, 4}
    assert err < REL_L2, err


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_ffn_tiny_arbitrary_bit_mix(seed):
    # widths 1..4 mixed inside one expert exercise every plane-unit pattern
    w, _, _, _ = workload(1)
    rng = np.random.default_rng(seed)
    b = rng.integers(1, 5, size=w.cfg.P)
    note(f"ffn cfg1 random bits seed={seed}")
    err, _ = _ffn_case(1, bits_np=b)
    assert err < REL_L2, err


@pytest.mark.parametrize("width", [1, 2, 3, 4])
def test_ffn_tiny_uniform_width(width):
    w, _, _, _ = workload(1)
    note(f"ffn cfg1 uniform width {width}")
    err, _ = _ffn_case(1, bits_np=np.full(w.cfg.P, width))
    assert err < REL_L2, err


def test_ffn_tiny_accumulate_and_ragged():
    note("ffn cfg1 accumulate")
    err, _ = _ffn_case(1, accumulate=True)
    assert err < REL_L2, err
    for T in (1, 3, 7):
        note(f"ffn cfg1 T={T}")
        err, _ = _ffn_case(1, T=T)
        assert err < REL_L2, (T, err)


def test_ffn_qwen_decode_group64():
    # two quant groups per k-block on the decode path with many items
    note("ffn cfg2 T=32 g=64")
    err, _ = _ffn_case(2, over=dict(g=64))
    assert err < REL_L2, err


# Small batches: one or a few pairs per expert, each chunk a single width
# (T=1) or a few; the DeepSeek shape adds shared experts with an 11-k-block
# down projection; group size 64 takes two-group k-blocks.
@pytest.mark.parametrize("case", [(2, 1, {}), (2, 2, {}), (2, 4, {}), (2, 1, dict(g=64)), (3, 1, {}),
                                  (3, 3, dict(b_lo=1))])
def test_ffn_small_batches(case):
    i, T, over = case
    note(f"ffn small batch cfg{i} T={T} {over}")
    err, _ = _ffn_case(i, T=T, over=over)
    assert err < REL_L2, err


@pytest.mark.parametrize("seed", [0, 1])
def test_ffn_small_batch_arbitrary_bit_mix(seed):
    w, _, _, _ = workload(2)
    rng = np.random.default_rng(20 + seed)
    b = rng.integers(1, 5, size=4 * w.cfg.k)
    note(f"ffn small batch cfg2 T=4 random bits seed={seed}")
    err, _ = _ffn_case(2, bits_np=b, T=4)
    assert err < REL_L2, err


# 32 or more pairs per expert on average switch the layer to chunks of 64
# pairs (four 16-token blocks per workgroup): ragged chunk tails, empty
# blocks, both group sizes, mixed widths and shared experts


@pytest.mark.parametrize("g,T", [(64, 128), (64, 150), (128, 300)])
def test_ffn_wide_chunks_full(g, T):
    note(f"ffn cfg1 wide g={g} T={T}")
    err, _ = _ffn_case(1, over=dict(g=g, T=T))
    assert err < REL_L2, err


@pytest.mark.parametrize("seed", [0, 1])
def test_ffn_wide_chunks_arbitrary_bit_mix(seed):
    w, _, _, _ = workload(1, g=128, T=300)
    rng = np.random.default_rng(10 + seed)
    b = rng.integers(1, 5, size=w.cfg.P)
    note(f"ffn cfg1 wide random bits seed={seed}")
    err, _ = _ffn_case(1, bits_np=b, over=dict(g=128, T=300))
    assert err < REL_L2, err


def test_ffn_wide_chunks_accumulate():
    note("ffn cfg1 wide accumulate")
    err, _ = _ffn_case(1, accumulate=True, over=dict(g=64, T=200))
    assert err < REL_L2, err


def test_ffn_wide_chunks_large_plan():
    # 9000 pairs: the plan runs as three launches over the chip
    note("ffn cfg1 wide T=4500")
    err, _ = _ffn_case(1, tokens=list(range(0, 4500, 97)) + [4499], over=dict(g=128, T=4500))
    assert err < REL_L2, err


def test_ffn_wide_chunks_deepseek_shared():
    note("ffn cfg3 wide T=384")
    err, _ = _ffn_case(3, tokens=[0, 1, 100, 383], over=dict(T=384))
    assert err < REL_L2, err


def _check_rmsnorm(h, x, eps):
    ref = orc.rmsnorm_bf16(h.cpu().numpy(), eps)
    assert np.array_equal(x.float().cpu().numpy().astype(np.float64), ref)


def test_ffn_drops_invalid_pairs():
    # an out-of-range expert index contributes nothing and breaks nothing
    w, dev, oc, _ = workload(1)
    cfg = w.cfg
    idx, gate = bd.route(dev["x"], dev["w_router"], None, cfg.k)
    bits = bd.alloc_bits(gate.reshape(-1), 2, 4, 3.0)
    idx_bad = idx.clone()
    idx_bad[3, 1] = 99
    note("ffn invalid pair dropped")
    y = bd.anyprec_ffn(dev["routed"], None, dev["x"], idx_bad, gate, bits)
    torch.cuda.synchronize()
    g = gate.cpu().numpy().astype(np.float64)
    g[3, 1] = 0.0
    ii = idx.cpu().numpy()
    ref = orc.combine(w.x_bf16, ii, g, bits.cpu().numpy(), oc)
    assert rel_l2(y.cpu().numpy(), ref) < REL_L2


def test_ffn_one_token_drops_invalid_and_repeated():
    # One token runs its own plan kernel (each pair a chunk of its own); it
    # keeps the general plan's dropping rules: an expert out of range, a width
    # out of range, a repeat of an earlier pair's expert (of a repeat, the
    # first pair with a valid width is kept).
    w, dev, oc, _ = workload(2)
    cfg = w.cfg
    x = dev["x"][:1].contiguous()
    idx, gate = bd.route(x, dev["w_router"], dev["bias"], cfg.k)
    bits = bd.alloc_bits(gate.reshape(-1), cfg.b_lo, 4, cfg.target)
    idx_bad, bits_bad = idx.clone(), bits.clone()
    idx_bad[0, 2] = idx[0, 1]   # repeats pair 1: dropped
    idx_bad[0, 3] = idx[0, 4]   # pair 3 and pair 4 share an expert ...
    bits_bad[3] = 9             # ... pair 3's width is out of range: dropped, pair 4 kept
    idx_bad[0, 5] = 500         # expert out of range: dropped
    bits_bad[6] = 0             # width out of range: dropped
    note("ffn one token, invalid and repeated pairs")
    y = bd.anyprec_ffn(dev["routed"], None, x, idx_bad, gate, bits_bad)
    torch.cuda.synchronize()
    g = gate.cpu().numpy().astype(np.float64)
    g[0, [2, 3, 5, 6]] = 0.0
    ref = orc.combine(w.x_bf16[:1], idx.cpu().numpy(), g, bits.cpu().numpy().astype(np.int64), oc)
    err = rel_l2(y.cpu().numpy(), ref)
    assert err < REL_L2, err
    # accumulate onto y, one token, shared experts (DeepSeek shape, B_lo 1)
    note("ffn one token accumulate cfg3 b_lo=1")
    err, _ = _ffn_case(3, T=1, accumulate=True, over=dict(b_lo=1))
    assert err < REL_L2, err


@pytest.mark.parametrize("rows,d", [(64, 2048), (3, 100), (5, 1), (1, 4096)])
def test_rmsnorm_to_bf16_exact(rows, d):
    # rows of very different magnitudes, a zero row, ragged widths
    rng = np.random.default_rng(rows * 1000 + d)
    h = (rng.standard_normal((rows, d)) * 10.0 ** rng.integers(-4, 5, (rows, 1))).astype(np.float32)
    if rows > 2:
        h[1] = 0.0
    note(f"rmsnorm_to_bf16 rows={rows} d={d}")
    ht = torch.from_numpy(h).cuda()
    for eps in (1e-6, 0.5):
        x = bd.rmsnorm_to_bf16(ht, eps=eps)
        torch.cuda.synchronize()
        _check_rmsnorm(ht, x, eps)


def test_residual_to_bf16_exact():
    rng = np.random.default_rng(4)
    h = (rng.standard_normal(10001) * 3).astype(np.float32)
    note("residual_to_bf16")
    x = bd.residual_to_bf16(torch.from_numpy(h).cuda())
    torch.cuda.synchronize()
    ref = orc.round_bf16(h.astype(np.float64))
    got = x.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 2048 * 3 + 48, 1 << 26])
def test_stream_read_folds_every_word_once(nbytes):
    # the measurement helper reads every 16-byte word exactly once: the XOR
    # of its per-wave folds equals the XOR of all 32-bit words of the buffer
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(bd.STREAM_SINK, dtype=torch.int32, device="cuda")
    note(f"stream_read {nbytes} B")
    bd.stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


# ---------------------------------------------------------------------------
# the whole layer in one call: identical to route + alloc + FFN in sequence


@pytest.mark.parametrize("case", [(1, {}), (1, dict(T=100)), (1, dict(T=200)), (1, dict(T=300)), (2, dict(T=1)),
                                  (2, dict(T=4)), (2, dict(T=64)),
                                  (3, dict(T=1)), (2, {}),
                                  (2, dict(T=128)), (3, {}), (3, dict(b_lo=1)), (4, dict(T=512))])
def test_layer_call_equals_three_calls(case):
    i, over = case
    w, dev, _, _ = workload(i, **over)
    cfg = w.cfg
    x = dev["x"]
    note(f"layer cfg{i} {over}")
    idx, gate = bd.route(x, dev["w_router"], dev["bias"], cfg.k)
    bits = bd.alloc_bits(gate.reshape(-1), cfg.b_lo, 4, cfg.target)
    y_ref = bd.anyprec_ffn(dev["routed"], dev["shared"], x, idx, gate, bits)
    y, idx2, gate2, bits2 = bd.layer(dev["routed"], dev["shared"], x, dev["w_router"], dev["bias"], cfg.k,
                                     cfg.b_lo, cfg.target)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx)
    assert torch.equal(gate2, gate)
    assert torch.equal(bits2, bits)
    assert torch.equal(y, y_ref)
