"""Full-size GPU parity: the layer as the benchmark runs it (one moe_layer
call), on the full-size workloads, against the CPU oracle on every output
row (decode), on 512+ rows and whole expert groups (prefill), and on every
layer of the 48-layer stack (teacher-forced).

Bars: routing indices and per-pair widths bit-exact (top-k ties flagged
where the oracle's logit gap is below 1e-5; widths from the oracle's
allocation on the GPU's own gates); all checked output rows together within
relative L2 1e-3, and every single row within 5e-3.  Each case prints its
largest row error.

The per-row bar follows from the arithmetic.  The SwiGLU output h is rounded
to bf16 on both sides, from fp32 sums on the GPU and fp64 sums in the
oracle; where the two land on different sides of a bf16 rounding boundary
the element differs by one bf16 step (2^-8 relative), which moves its row
by about 2^-8 |h_j| / ||h|| (1.4e-4 for a typical element of 768, near 1e-3
for the largest of a row).  A handful of such steps in one row stays below
5e-3, while a pair read at a wrong width moves its row by 1e-1 or more."""
import multiprocessing as mp
import sys

import numpy as np
import pytest
import torch

from dynamic_any_precision_amd import binding as bd
from dynamic_any_precision_amd import workloads as wl
import oracle as orc
import oracle_pool

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
ROW_REL_L2 = 5e-3
TIE_GAP = 1e-5


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def row_rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)


def check_rows(name, got, ref):
    """Per-row and overall relative L2 against the oracle; prints both."""
    per_row = row_rel_l2(got, ref)
    overall = float(np.linalg.norm(np.asarray(got, np.float64) - ref) / np.linalg.norm(ref))
    print(f"[parity] {name}: rows={per_row.size} overall_rel_l2={overall:.3e} "
          f"max_row_rel_l2={per_row.max():.3e} median_row_rel_l2={np.median(per_row):.3e}", flush=True)
    assert overall < REL_L2, (name, overall)
    assert per_row.max() < ROW_REL_L2, (name, int(per_row.argmax()), float(per_row.max()))
    return per_row


def check_routing(name, x_np, w_router, bias, k, idx, gate, renorm=False):
    """Indices exact on unflagged tokens; gates to fp32 rounding."""
    oidx, ogate, gap, _ = orc.route(x_np, w_router, bias, k, renorm)
    ok = gap >= TIE_GAP
    assert np.array_equal(idx[ok], oidx[ok]), (name, np.nonzero((idx != oidx).any(1) & ok))
    assert np.allclose(gate[ok], ogate[ok], rtol=4e-7, atol=1e-30), name
    return int((~ok).sum())


def check_widths(name, gate, bits, b_lo, b_max, target):
    obits, n, ns = orc.allocate_bits(gate.astype(np.float64).ravel(), b_lo, b_max, target)
    assert np.array_equal(np.asarray(bits).astype(np.int64).ravel(), obits), name
    return n, ns


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


_cache = {}


def workload(i, **kw):
    """Host workload, its device copy and the oracle's dequantisation cache;
    one configuration is kept at a time (each cache holds GBs)."""
    key = (i, tuple(sorted(kw.items())))
    if key not in _cache:
        _cache.clear()
        cfg = wl.config(i, **kw)
        w = wl.make_workload(cfg, keep_codes=False)
        dev = dict(
            routed=bd.DeviceBank.from_host(w.routed),
            shared=bd.DeviceBank.from_host(w.shared) if w.shared is not None else None,
            x=bd.bf16_tensor(w.x_bf16),
            w_router=torch.from_numpy(w.w_router).cuda(),
            bias=torch.from_numpy(w.logit_bias).cuda() if w.logit_bias is not None else None,
        )
        _cache[key] = (w, dev, orc.bank_cache(w.routed), orc.bank_cache(w.shared) if w.shared is not None else None)
    return _cache[key]


def _layer_case(i, T=None, target=None, b_lo=None):
    """One moe_layer call on the device copy of workload i (first T tokens)."""
    w, dev, oc, sc = workload(i)
    cfg = w.cfg
    x, x_np = dev["x"], w.x_bf16
    if T is not None:
        x, x_np = x[:T].contiguous(), x_np[:T]
    target = cfg.target if target is None else target
    b_lo = cfg.b_lo if b_lo is None else b_lo
    y, idx, gate, bits = bd.layer(dev["routed"], dev["shared"], x, dev["w_router"], dev["bias"], cfg.k, b_lo,
                                  target)
    torch.cuda.synchronize()
    return (w, oc, sc, x_np, y.cpu().numpy().astype(np.float64), idx.cpu().numpy(), gate.cpu().numpy(),
            bits.cpu().numpy())


# ---------------------------------------------------------------------------
# decode: every row


@pytest.mark.parametrize("target", [2.0, 2.5, 3.0, 4.0])
def test_qwen_decode_every_row(target):
    note(f"full-size cfg2 T=32 target={target} (moe_layer)")
    w, oc, _, x_np, y, idx, gate, bits = _layer_case(2, target=target)
    cfg = w.cfg
    check_routing("cfg2 T=32", x_np, w.w_router, None, cfg.k, idx, gate)
    check_widths("cfg2 T=32", gate, bits, cfg.b_lo, cfg.b_max, target)
    ref = orc.combine(x_np, idx, gate.astype(np.float64), bits, oc)
    check_rows(f"cfg2 T=32 target={target}", y, ref)


@pytest.mark.parametrize("target", [2.0, 2.5, 3.0, 4.0])
def test_qwen_decode_batch1_every_target(target):
    note(f"full-size cfg2 T=1 target={target} (moe_layer)")
    w, oc, _, x_np, y, idx, gate, bits = _layer_case(2, T=1, target=target)
    cfg = w.cfg
    check_routing("cfg2 T=1", x_np, w.w_router, None, cfg.k, idx, gate)
    check_widths("cfg2 T=1", gate, bits, cfg.b_lo, cfg.b_max, target)
    ref = orc.combine(x_np, idx, gate.astype(np.float64), bits, oc)
    check_rows(f"cfg2 T=1 target={target}", y, ref)


@pytest.mark.parametrize("b_lo", [1, 2])
def test_deepseek_every_row(b_lo):
    note(f"full-size cfg3 T=16 b_lo={b_lo} (moe_layer, two shared experts)")
    w, oc, sc, x_np, y, idx, gate, bits = _layer_case(3, b_lo=b_lo)
    cfg = w.cfg
    check_routing("cfg3", x_np, w.w_router, None, cfg.k, idx, gate)
    check_widths("cfg3", gate, bits, b_lo, cfg.b_max, cfg.target)
    assert set(np.unique(bits)) <= {b_lo, 4}
    ref = orc.combine(x_np, idx, gate.astype(np.float64), bits, oc, sc, cfg.n_shared)
    check_rows(f"cfg3 T=16 b_lo={b_lo}", y, ref)


# ---------------------------------------------------------------------------
# prefill: 512+ rows, and the smallest and largest expert groups whole


def test_qwen_prefill_rows():
    note("full-size cfg4 T=4096 (moe_layer)")
    w, oc, _, x_np, y, idx, gate, bits = _layer_case(4)
    cfg = w.cfg
    flagged = check_routing("cfg4", x_np, w.w_router, w.logit_bias, cfg.k, idx, gate)
    check_widths("cfg4", gate, bits, cfg.b_lo, cfg.b_max, cfg.target)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    live = np.nonzero(counts)[0]
    e_small = int(live[np.argmin(counts[live])])
    rng = np.random.default_rng(44)
    rows = set(rng.choice(cfg.T, size=512, replace=False).tolist())
    rows |= set(np.nonzero((idx == e_small).any(1))[0].tolist())
    rows |= {0, cfg.T - 1}
    rows = sorted(rows)
    print(f"[parity] cfg4 expert load: max {counts.max()} min {counts[live].min()} "
          f"(expert {e_small}), flagged ties {flagged}", flush=True)
    ref = orc.combine(x_np[rows], idx[rows], gate[rows].astype(np.float64), bits.reshape(cfg.T, cfg.k)[rows], oc)
    check_rows(f"cfg4 T=4096 {len(rows)} rows", y[rows], ref)


@pytest.mark.parametrize("which", ["largest", "smallest"])
def test_qwen_prefill_whole_expert_group(which):
    # Only one expert's pairs are kept (the others get an out-of-range index
    # and are dropped), so its chunks are exactly those of the full batch and
    # every one of its pairs is compared.
    w, dev, oc, _ = workload(4)
    cfg = w.cfg
    idx, gate = bd.route(dev["x"], dev["w_router"], dev["bias"], cfg.k)
    bits = bd.alloc_bits(gate.reshape(-1), cfg.b_lo, cfg.b_max, cfg.target)
    counts = torch.bincount(idx.reshape(-1).long(), minlength=cfg.E).cpu().numpy()
    live = np.nonzero(counts)[0]
    e = int(live[np.argmax(counts[live])] if which == "largest" else live[np.argmin(counts[live])])
    idx_e = torch.where(idx == e, idx, torch.full_like(idx, cfg.E + 1))
    note(f"full-size cfg4 T=4096 {which} group: expert {e}, {counts[e]} pairs")
    y = bd.anyprec_ffn(dev["routed"], None, dev["x"], idx_e, gate, bits)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    gate_np = gate.cpu().numpy().astype(np.float64)
    bits_np = bits.cpu().numpy().reshape(cfg.T, cfg.k)
    toks, js = np.nonzero(idx_np == e)
    ref = orc.combine(w.x_bf16[toks], idx_np[toks, js][:, None], gate_np[toks, js][:, None],
                      bits_np[toks, js][:, None], oc)
    got = y.cpu().numpy().astype(np.float64)
    check_rows(f"cfg4 {which} group (expert {e}, widths {sorted(set(bits_np[toks, js].tolist()))})",
               got[toks], ref)
    others = np.setdiff1d(np.arange(cfg.T), toks)
    assert np.all(got[others] == 0.0)


# ---------------------------------------------------------------------------
# the 48-layer stack, teacher-forced on every layer


N_LAYERS = 48
RMS_EPS = 1e-6


def test_stack48_every_layer_teacher_forced():
    # The stack as the benchmark steps it: h = x0; per layer x = bf16(rmsnorm(h)),
    # h += moe_layer(x).  Every layer's input is checked bit for bit, its
    # routing and widths exactly, and three of its output rows against the
    # oracle run on the GPU's own layer input (teacher forcing), at targets
    # 2.0, 3.0 and 4.0.
    cfg = wl.config(5)
    T, d = cfg.T, cfg.d
    targets = (2.0, 3.0, 4.0)
    banks, routers = [], []
    for l in range(N_LAYERS):
        wr, bank = wl.make_stack_layer(cfg, l)
        routers.append((wr, torch.from_numpy(wr).cuda()))
        banks.append(bd.DeviceBank.from_host(bank))
        del bank
    note(f"stack48: {N_LAYERS} layers resident")
    h0 = wl.bf16_bits_to_f32(wl.step_activations(cfg, 0, T))
    ws = bd.layer_workspace(banks[0], None, T, cfg.k)
    tasks = {l: {} for l in range(N_LAYERS)}
    rows_of = {}
    got_of = {}
    flagged = 0
    for target in targets:
        note(f"stack48 target={target}")
        h = torch.from_numpy(h0.copy()).cuda()
        x = bd.rmsnorm_to_bf16(h, eps=RMS_EPS)
        for l in range(N_LAYERS):
            h_prev = h.clone()
            y, idx, gate, bits = bd.layer(banks[l], None, x, routers[l][1], None, cfg.k, cfg.b_lo, target, y=h,
                                          accumulate=True, workspace=ws)
            torch.cuda.synchronize()
            x_np = x.view(torch.int16).cpu().numpy().view(np.uint16)
            idx_np, gate_np, bits_np = idx.cpu().numpy(), gate.cpu().numpy(), bits.cpu().numpy()
            flagged += check_routing(f"stack layer {l}", x_np, routers[l][0], None, cfg.k, idx_np, gate_np)
            check_widths(f"stack layer {l}", gate_np, bits_np, cfg.b_lo, cfg.b_max, target)
            rows = sorted({l % T, (7 * l + 13) % T, T - 1 - (l % 5)})
            rows_of[(l, target)] = rows
            got_of[(l, target)] = (h.cpu().numpy().astype(np.float64)[rows]
                                   - h_prev.cpu().numpy().astype(np.float64)[rows])
            tasks[l][target] = (x_np[rows], idx_np[rows], gate_np[rows], bits_np.reshape(T, cfg.k)[rows])
            x = bd.rmsnorm_to_bf16(h, eps=RMS_EPS)
            torch.cuda.synchronize()
            ref_x = orc.rmsnorm_bf16(h.cpu().numpy(), RMS_EPS)
            assert np.array_equal(x.float().cpu().numpy().astype(np.float64), ref_x), l
        assert np.all(np.isfinite(h.cpu().numpy()))
    del banks
    torch.cuda.empty_cache()
    note(f"stack48: oracle on {N_LAYERS} layers in {oracle_pool.pool_size()} worker processes")
    ctx = mp.get_context("spawn")
    refs = {}
    with ctx.Pool(oracle_pool.pool_size()) as pool:
        for l, out in pool.imap_unordered(oracle_pool.stack_layer, sorted(tasks.items())):
            refs[l] = out
            note(f"stack48: oracle layer {l} done ({len(refs)}/{N_LAYERS})")
    for target in targets:
        errs = []
        for l in range(N_LAYERS):
            per_row = row_rel_l2(got_of[(l, target)], refs[l][target])
            errs.append(per_row.max())
            assert per_row.max() < ROW_REL_L2, (l, target, per_row)
        overall = np.concatenate([got_of[(l, target)] - refs[l][target] for l in range(N_LAYERS)])
        norm = np.concatenate([refs[l][target] for l in range(N_LAYERS)])
        assert np.linalg.norm(overall) / np.linalg.norm(norm) < REL_L2, target
        print(f"[parity] stack48 target={target}: max row rel-L2 over 48 layers {max(errs):.3e}, "
              f"final layer {errs[-1]:.3e}", flush=True)
    print(f"[parity] stack48 flagged router ties {flagged}", flush=True)
