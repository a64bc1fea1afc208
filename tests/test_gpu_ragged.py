"""GPU parity of ragged banks (per-expert maximum width B_e in {2, 3, 4};
MatMoE review, Core Contribution) against the CPU oracle, through the C ABI:
dequantised weights bit-exact at every width (reads wider than B_e clamp to
B_e), and layers on every row within the FFN's bars, on the decode and the
wide (prefill-sized) paths."""
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
        w = wl.make_ragged_workload(wl.config(i, ragged=True, **kw), keep_codes=False)
        dev = dict(routed=bd.DeviceBank.from_host(w.routed), x=bd.bf16_tensor(w.x_bf16),
                   w_router=torch.from_numpy(w.w_router).cuda())
        _cache[key] = (w, dev, orc.ragged_bank_cache(w.routed))
    return _cache[key]


@pytest.mark.parametrize("cfg_id", [1, 2])
def test_ragged_dequant_bit_exact(cfg_id):
    w, dev, oc = workload(cfg_id)
    bank = dev["routed"]
    widths = np.diff(w.routed.plane_prefix)
    experts = range(bank.n_experts) if cfg_id == 1 else [int(np.argmax(widths == b)) for b in (2, 3, 4)]
    for e in experts:
        for m in (0, 1):
            for b in range(1, 5):
                note(f"ragged dequant cfg{cfg_id} e{e} (B_e {widths[e]}) m{m} b{b}")
                got = bd.dequant(bank, e, m, b).cpu().numpy()
                ref = oc.weights(e, b)[m].astype(np.float32)
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (e, m, b)


@pytest.mark.parametrize("case", [(1, None, 3.0), (1, None, 4.0), (2, None, 3.0), (2, None, 4.0), (2, 1, 3.0),
                                  (1, 300, 3.0)])
def test_ragged_layer_every_row(case):
    i, T, target = case
    w, dev, oc = workload(i) if T is None else workload(i, T=T)
    cfg = w.cfg
    note(f"ragged layer cfg{i} T={cfg.T if T is None else T} target={target}")
    y, idx, gate, bits = bd.layer(dev["routed"], None, dev["x"], dev["w_router"], None, cfg.k, cfg.b_lo, target)
    torch.cuda.synchronize()
    idx_np, gate_np, bits_np = idx.cpu().numpy(), gate.cpu().numpy().astype(np.float64), bits.cpu().numpy()
    obits, _, _ = orc.allocate_bits(gate_np.ravel(), cfg.b_lo, cfg.b_max, target)
    assert np.array_equal(bits_np.astype(np.int64), obits)
    ref = orc.combine(w.x_bf16, idx_np, gate_np, bits_np, oc)
    got = y.cpu().numpy().astype(np.float64)
    per_row = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    overall = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    widths = np.diff(w.routed.plane_prefix)
    read = np.minimum(bits_np, widths[idx_np.ravel()])
    print(f"[parity] ragged cfg{i} T={got.shape[0]} target={target}: widths read "
          f"{np.bincount(read, minlength=5)[1:].tolist()}, overall_rel_l2={overall:.3e} "
          f"max_row_rel_l2={per_row.max():.3e}", flush=True)
    assert overall < 1e-3 and per_row.max() < 5e-3


def test_ragged_permute_reports_read_widths():
    w, dev, oc = workload(1)
    cfg = w.cfg
    idx, gate = bd.route(dev["x"], dev["w_router"], None, cfg.k)
    bits = torch.full((cfg.P,), 4, dtype=torch.uint8, device="cuda")
    ws = bd.ffn_workspace(dev["routed"], None, cfg.T, cfg.k)
    note("ragged permute")
    # the standalone permutation sees no bank: widths as given
    _, _, emax = bd.permute(idx, bits, cfg.E, 4, ws)
    torch.cuda.synchronize()
    assert set(emax.cpu().numpy().tolist()) <= {0, 4}


def test_ragged_bank_rejected_by_bakes():
    w, dev, oc = workload(1)
    with pytest.raises(bd.MoeError) as ei:
        bd.duorate_bake(dev["routed"])
    assert ei.value.status == 6
