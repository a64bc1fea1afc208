"""Benchmark of the dynamic any-precision MoE layer on one MI355X.

Workload: one Qwen3-30B-A3B-shaped MoE layer in decode (hidden 2048, expert
intermediate 768, 128 experts, top-8, SwiGLU, 4 bitplanes, group 128),
synthetic seeded inputs.  A step is one pass of the whole layer over a batch:
router (logits, softmax, top-k), bit allocation (threshold bisection to the
target average), and the any-precision expert FFN with the gate-weighted
combine.  Inputs are resident in HBM before timing; four copies of the
expert bank (1.36 GB) are rotated and eight activation batches cycled so the
256 MB last-level cache can not serve the weights.

The headline step is one moe_layer call (the whole layer; at decode sizes
its allocation and plan run as one single-block kernel, with the top-k too
for T <= 16) on T=32 tokens at target 3.0 bits, replayed from HIP graphs
that each hold one cycle of the 8 activation batches; a sweep over T in
{1, 32} and targets {2.0, 2.5, 3.0, 4.0} follows.
The roofline object is for the FFN stage's dominant kernel, gate/up +
SwiGLU, timed with HIP events recorded on the FFN's stream around that
kernel's launch (moe_set_kernel_events), against its algorithmic bytes per
launch; the down kernel and the whole FFN call are reported beside it.  Its
"traffic" is the counter-measured HBM bytes per launch of that kernel
recorded under profiles/ (FETCH_SIZE and WRITE_SIZE, calibrated on a plain
copy), used only while the kernel sources still hash to the value recorded
there.

With --prefill the same layer runs one T=4096 prefill batch with a
Zipf(1.1)-skewed expert load (the grouped matrix-core path: chunks of 64
pairs); that line's roofline is matrix-core bound: the gate/up kernel's
algorithmic flops (4 d f per routed pair) over its event-timed duration,
in TFLOP/s against the bf16 dense peak, the down kernel and the whole
routed SwiGLU FFN (6 d f flops per routed pair) beside it.

With --calibrated the widths come from a gate threshold calibrated once
(MatMoE's calibration-threshold mode): the bisection runs over the gates of
64 calibration batches, and each step then runs the router, the fixed-
threshold widths and the FFN; the line reports the spread of the per-step
average width over 64 held-out batches for targets 2.5, 3.0 and 3.5.

With --stack the step is a decode step through 48 such layers (T=64, each
layer with its own router and expert bank, 16.3 GB resident): per layer
the RMS-normalised bf16 cast of the fp32 residual as the layer's input,
then one moe_layer call that adds its output into the residual; the
targets 2.0 .. 4.0 in steps of 0.25 are swept.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep] [--no-cpu] [--prefill | --stack | --calibrated]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
N_COPIES = 4
N_XBATCH = 8


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_ffn_bytes(idx, bits, cfg, accumulate=False):
    """Bytes the FFN stage must move: the first b_e planes and the (scale,
    zero) of every active expert (b_e = widest pair of the expert), the
    shared experts at full width, the activations in, the output, and the
    bf16 intermediate round trip."""
    k = kernel_bytes(idx, bits, cfg, accumulate)
    return k["total"], k["bits_read"], k["bits_alloc"], k["n_active"]


def kernel_bytes(idx, bits, cfg, accumulate=False, expert_widths=None):
    """Algorithmic bytes of the FFN stage and of its two streaming kernels:
    gate/up (W13 planes and (scale, zero) of the active experts, the shared
    experts' W13, the activations in, the SwiGLU output written) and down
    (W2 likewise, the SwiGLU output read, the layer output written).  With
    per-expert stored widths (a ragged bank) a pair reads min(b, B_e)."""
    d, f, g = cfg.d, cfg.f, cfg.g
    idx = np.asarray(idx).ravel()
    bits = np.asarray(bits).ravel().astype(np.int64)
    if expert_widths is not None:
        bits = np.minimum(bits, np.asarray(expert_widths)[idx])
    be = np.zeros(cfg.E, dtype=np.int64)
    np.maximum.at(be, idx, bits)
    act = be > 0
    T = idx.size // cfg.k
    ns, fs = getattr(cfg, "n_shared", 0), getattr(cfg, "f_shared", 0)
    planes13 = int(np.sum(be[act])) * 2 * d * f // 8 + ns * cfg.b_max * 2 * d * fs // 8
    planes2 = int(np.sum(be[act])) * d * f // 8 + ns * cfg.b_max * d * fs // 8
    sz13 = int(np.sum(act)) * 2 * d * f // g * 8 + ns * 2 * d * fs // g * 8
    sz2 = int(np.sum(act)) * d * f // g * 8 + ns * d * fs // g * 8
    x_in = T * d * 2
    y_out = T * d * 4 * (2 if accumulate else 1)
    h = (idx.size * f + ns * T * fs) * 2
    w13 = planes13 + sz13 + x_in + h
    w2 = planes2 + sz2 + h + y_out
    return dict(total=w13 + w2, w13=w13, w2=w2, bits_read=float(np.mean(be[act])), bits_alloc=float(np.mean(bits)),
                n_active=int(np.sum(act)))


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_decode_qwen_T32_b3.0_hbm_bytes.md")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_prefill_qwen_T4096_counters.md")
FFN_SOURCES = ("ffn.hip", "permute.hip", "common.hpp", "kernels.hpp")


def ffn_source_hash():
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        with open(os.path.join(ROOT, "dynamic_any_precision_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(T, target, path=None, T_rec=32):
    """Counter-measured bytes per launch of the gate/up kernel for the
    recorded workload (decode T=32 or prefill T=4096, 3.0 bits), or None when
    that record is missing or older than the kernels."""
    path = TRAFFIC_FILE if path is None else path
    if T != T_rec or target != 3.0 or not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(("|", "#", "`")):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != ffn_source_hash() or "traffic_bytes_per_launch" not in rec:
        return None
    return float(rec["traffic_bytes_per_launch"])


def read_ceiling(torch, bd, gib=2, reps=10):
    """Achievable HBM read rate: the library's pure streaming read of a
    buffer far larger than the 256 MB last-level cache, HIP-event timed."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(bd.STREAM_SINK, dtype=torch.int32, device="cuda")
    for _ in range(3):
        bd.stream_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        bd.stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = buf.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    return gbs


def router_bytes(cfg, T):
    return cfg.E * cfg.d * 4 + T * cfg.d * 2 + T * cfg.k * 9


class Layer:
    """Device state for one workload: bank copies, x batches, buffers, graphs.

    The per-pair widths of a step come from `policy`: "threshold" (the
    gate-threshold bisection of the batch: one moe_layer call, or route +
    alloc + FFN when timed with events), "calibrated" (a fixed threshold
    tau), "duorate" (per-expert widths `expert_bits`) or "dpa" (residual-
    aware chunk allocation over the residuals `resid`)."""

    def __init__(self, cfg, w, torch, bd, T):
        self.cfg, self.torch, self.bd, self.T = cfg, torch, bd, T
        self.bias = torch.from_numpy(w.logit_bias).to("cuda") if w.logit_bias is not None else None
        dev = "cuda"
        base = bd.DeviceBank.from_host(w.routed)
        self.banks = [base] + [base.clone() for _ in range(N_COPIES - 1)]
        self.shared = None
        if w.shared is not None:
            sb = bd.DeviceBank.from_host(w.shared)
            self.shared = [sb] + [sb.clone() for _ in range(N_COPIES - 1)]
        from dynamic_any_precision_amd import workloads as wl
        self.xs = [bd.bf16_tensor(wl.step_activations(cfg, s, T)) for s in range(N_XBATCH)]
        self.wr = torch.from_numpy(w.w_router).to(dev)
        self.rws = bd.route_workspace(T, cfg.E)
        sh0 = self.shared[0] if self.shared else None
        self.fws = bd.ffn_workspace(base, sh0, T, cfg.k)
        self.lws = bd.layer_workspace(base, sh0, T, cfg.k)
        self.idx = [torch.empty(T, cfg.k, dtype=torch.int32, device=dev) for _ in range(N_XBATCH)]
        self.gate = [torch.empty(T, cfg.k, dtype=torch.float32, device=dev) for _ in range(N_XBATCH)]
        self.bits = [torch.empty(T * cfg.k, dtype=torch.uint8, device=dev) for _ in range(N_XBATCH)]
        self.y = torch.empty(T, cfg.d, dtype=torch.float32, device=dev)
        self.graphs = {}
        self.policy = "threshold"
        self.tau = None          # calibrated: fixed gate threshold (host float)
        self.expert_bits = None  # duorate: [E] uint8 device
        self.resid = None        # dpa: [E][B] float64 device
        self.dws = None          # dpa workspace
        pp = getattr(w.routed, "plane_prefix", None)
        self.expert_widths = None if pp is None else np.diff(np.asarray(pp))   # ragged bank: B_e

    def widths(self, s, target):
        bd, cfg = self.bd, self.cfg
        if self.policy == "calibrated":
            bd.bits_from_threshold(self.gate[s].view(-1), self.tau, cfg.b_lo, cfg.b_max, bits=self.bits[s])
        elif self.policy == "duorate":
            bd.bits_from_expert_widths(self.idx[s].view(-1), self.expert_bits, bits=self.bits[s])
        elif self.policy == "dpa":
            bd.dpa_alloc(self.gate[s].view(-1), self.idx[s].view(-1), self.resid, cfg.b_lo, cfg.b_max, target,
                         bits=self.bits[s], workspace=self.dws)
        else:
            bd.alloc_bits(self.gate[s].view(-1), cfg.b_lo, cfg.b_max, target, bits=self.bits[s])

    def step(self, i, target, ev=None, kev=None):
        """One layer step: moe_layer (one call), or with ev the calls route,
        widths, FFN with HIP events ev around the FFN call and kev (four
        events) around its gate/up and down kernels."""
        bd, cfg = self.bd, self.cfg
        s = i % N_XBATCH
        bank = self.banks[i % N_COPIES]
        shared = self.shared[i % N_COPIES] if self.shared else None
        if self.policy == "threshold" and ev is None and kev is None:
            bd.layer(bank, shared, self.xs[s], self.wr, self.bias, cfg.k, cfg.b_lo, target, y=self.y,
                     idx=self.idx[s], gate=self.gate[s], bits=self.bits[s], workspace=self.lws)
            return
        bd.route(self.xs[s], self.wr, self.bias, cfg.k, workspace=self.rws, idx=self.idx[s], gate=self.gate[s])
        self.widths(s, target)
        if ev is not None:
            ev[0].record()
        if kev is not None:
            bd.set_kernel_events(kev)
        bd.anyprec_ffn(bank, shared, self.xs[s], self.idx[s], self.gate[s], self.bits[s], y=self.y,
                       workspace=self.fws)
        if kev is not None:
            bd.set_kernel_events(None)
        if ev is not None:
            ev[1].record()

    def capture(self, target, nsteps=N_XBATCH):
        """HIP graph of steps 0 .. nsteps-1 of a cycle (nsteps <= N_XBATCH)."""
        torch = self.torch
        key = (float(target), nsteps, self.policy)
        if key in self.graphs:
            return self.graphs[key]
        gs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(N_XBATCH):       # warm the kernels outside capture
                self.step(i, target)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nsteps):
                self.step(i, target)
        gs.append(g)
        torch.cuda.synchronize()
        self.graphs[key] = gs
        return gs

    def timed_graph(self, target, steps, warmup):
        torch = self.torch
        # one graph per cycle of N_XBATCH steps, plus one for the remainder:
        # exactly `steps` steps are timed
        full = self.capture(target)[0]
        rem = self.capture(target, steps % N_XBATCH)[0] if steps % N_XBATCH else None
        for i in range(max(1, -(-warmup // N_XBATCH))):
            full.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps // N_XBATCH):
            full.replay()
        if rem is not None:
            rem.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def timed_events(self, target, steps):
        """Eager steps on the current stream: first HIP events around each FFN
        call, then, in steps of their own (the marks split the call), events
        around its gate/up and down kernels, recorded by the library on the
        call's stream."""
        torch = self.torch

        def evs(n, k):
            out = []
            for _ in range(n):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
                for x in e:
                    x.record()            # creates the HIP event behind each
                out.append(e)
            return out
        warm, call, kern = evs(N_XBATCH, 2), evs(steps, 2), evs(steps, 4)
        torch.cuda.synchronize()
        for i in range(N_XBATCH):
            self.step(i, target, warm[i])
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(i, target, call[i])
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(i, target, None, kern[i])
        torch.cuda.synchronize()
        ffn_ms = [e[0].elapsed_time(e[1]) for e in call]
        w13_ms = [e[0].elapsed_time(e[1]) for e in kern]
        w2_ms = [e[2].elapsed_time(e[3]) for e in kern]
        kb = []
        for i in range(steps):
            s = i % N_XBATCH
            kb.append(kernel_bytes(self.idx[s].cpu().numpy(), self.bits[s].cpu().numpy(), self.cfg,
                                   expert_widths=self.expert_widths))
        cfg = self.cfg
        flops = 6.0 * cfg.d * cfg.f * self.T * cfg.k  # routed SwiGLU FFN: gate, up, down

        def mean(key):
            return float(np.mean([k[key] for k in kb]))
        return dict(ffn_ms=float(np.mean(ffn_ms)), ffn_ms_p10=float(np.percentile(ffn_ms, 10)), ffn_flops=flops,
                    ffn_ms_p50=float(np.percentile(ffn_ms, 50)), ffn_ms_p90=float(np.percentile(ffn_ms, 90)),
                    w13_ms=float(np.mean(w13_ms)), w2_ms=float(np.mean(w2_ms)),
                    ffn_bytes=mean("total"), w13_bytes=mean("w13"), w2_bytes=mean("w2"), bits_read=mean("bits_read"),
                    bits_alloc=mean("bits_alloc"), n_active=mean("n_active"))


def kernel_roofline(ev, traffic=None):
    """Roofline of the dominant kernel (gate/up): its algorithmic bytes per
    launch over its event-timed duration, against the 8 TB/s HBM peak; the
    down kernel and the whole FFN call beside it."""
    a13 = ev["w13_bytes"] / (ev["w13_ms"] * 1e-3) / 1e9
    a2 = ev["w2_bytes"] / (ev["w2_ms"] * 1e-3) / 1e9
    ac = ev["ffn_bytes"] / (ev["ffn_ms"] * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": a13, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": a13 / HBM_PEAK_GBS,
            "traffic": traffic, "kernel": "gate/up + SwiGLU streaming kernel (k_ffn<W13>; k_ffn_small<W13> for batches of a few tokens), the FFN stage's dominant kernel",
            "bytes_per_launch": ev["w13_bytes"], "us_per_launch": ev["w13_ms"] * 1e3,
            "down_kernel": {"achieved": a2, "frac": a2 / HBM_PEAK_GBS, "bytes_per_launch": ev["w2_bytes"],
                            "us_per_launch": ev["w2_ms"] * 1e3},
            "ffn_call": {"achieved": ac, "frac": ac / HBM_PEAK_GBS, "bytes_per_launch": ev["ffn_bytes"],
                         "us_per_launch": ev["ffn_ms"] * 1e3,
                         "kernels": "plan, activation gather, gate/up + SwiGLU, down, combine"}}


def cpu_baseline(cfg, w, budget_s=10.0):
    """The oracle, untouched, on a bounded sample: whole routing and
    allocation of one T-token batch plus the expert FFN (routed and shared)
    of its first tokens, each token on a fresh dequantisation cache.  Timed
    with NumPy's BLAS on every core this process may use, then on one core."""
    import oracle as orc
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))

    def run(limit):
        done = 0
        t0 = time.perf_counter()
        with threadpool_limits(limits=limit):
            tok = 0
            while time.perf_counter() - t0 < budget_s and tok < cfg.T:
                rc = (orc.ragged_bank_cache(w.routed) if hasattr(w.routed, "plane_prefix")
                      else orc.bank_cache(w.routed))   # dequantisation is part of the work
                sc = orc.bank_cache(w.shared) if w.shared is not None else None
                orc.layer(w.x_bf16, w.w_router, w.logit_bias, cfg.k, cfg.b_lo, cfg.b_max, cfg.target, rc, sc,
                          cfg.n_shared, tokens=[tok])
                tok += 1
                done += 1
        return done, time.perf_counter() - t0
    n_all, t_all = run(cores)
    n_one, t_one = run(1)
    what = (f"token(s) of the T={cfg.T} batch: full routing and allocation of the batch plus those tokens' "
            f"{cfg.k} routed expert FFNs" + (f" and {cfg.n_shared} shared" if cfg.n_shared else "") +
            " (dequantised from the stored planes), float64 NumPy")
    return dict(value=n_all / t_all, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{n_all} {what}, {t_all:.1f} s on {cores} cores",
                single_core={"value": n_one / t_one, "unit": "tokens/s", "cores": 1,
                             "sample": f"{n_one} {what}, {t_one:.1f} s on 1 core"})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 200; 20 with --prefill)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 20; 3 with --prefill)")
    ap.add_argument("--prefill", action="store_true",
                    help="the T=4096 Zipf-skewed prefill batch instead of the decode headline")
    ap.add_argument("--stack", action="store_true",
                    help="a decode step through the 48-layer stack (T=64) instead of the single-layer headline")
    ap.add_argument("--calibrated", action="store_true",
                    help="calibration-threshold mode: a gate threshold fixed from calibration batches")
    ap.add_argument("--deepseek", action="store_true",
                    help="the DeepSeekMoE-16B-shaped decode layer (T=16, two shared experts, B_lo 2 and 1)")
    ap.add_argument("--duorate", action="store_true",
                    help="DuoRate per-expert widths solved on a prefill profile, then decode steps at those widths")
    ap.add_argument("--dpa", action="store_true",
                    help="DPA-MoE residual-aware chunk allocation over widths 1-4 on every decode step")
    ap.add_argument("--ragged", action="store_true",
                    help="the decode headline on a ragged bank: per-expert maximum widths B_e in {2, 3, 4}")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--target", type=float, default=3.0)
    ap.add_argument("--tokens", type=int, default=32)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device-to-device copy of MIB MiB (a reference dispatch of known "
                         "size for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 20 if args.prefill else 48 if args.stack else 200
    if args.warmup is None:
        args.warmup = 3 if args.prefill else 8 if args.stack else 20
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer runs on a single MI355X and has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from dynamic_any_precision_amd import binding as bd
    from dynamic_any_precision_amd import workloads as wl
    bd.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.copy_calibration} MiB device copies")
        del src, dst

    if args.prefill:
        return prefill(args, torch, bd, wl)
    if args.stack:
        return stack(args, torch, bd, wl)
    if args.calibrated:
        return calibrated(args, torch, bd, wl)
    if args.deepseek:
        return deepseek(args, torch, bd, wl)
    if args.duorate or args.dpa:
        return per_expert_modes(args, torch, bd, wl)
    cfg = wl.config(2, T=args.tokens, target=args.target, ragged=args.ragged)
    log("generating the Qwen3-30B-A3B-shaped layer (seeded)" + (", ragged bank" if args.ragged else ""))
    t0 = time.perf_counter()
    w = wl.make_ragged_workload(cfg, keep_codes=False) if args.ragged else wl.make_workload(cfg, keep_codes=False)
    log(f"generated in {time.perf_counter() - t0:.1f} s; stored {w.routed.stored_bytes() / 1e6:.1f} MB per copy")

    layers = {}

    def layer_for(T):
        if T not in layers:
            layers[T] = Layer(cfg, w, torch, bd, T)
        return layers[T]

    T = args.tokens
    L = layer_for(T)
    log(f"timing T={T} target={args.target}: {args.warmup} warmup + {args.steps} graph-replayed steps")
    t_step = L.timed_graph(args.target, args.steps, args.warmup)
    log(f"step {t_step * 1e3:.4f} ms; event-timing the FFN stage")
    ev = L.timed_events(args.target, args.steps)
    step_bytes = ev["ffn_bytes"] + router_bytes(cfg, T)
    log(f"gate/up {ev['w13_ms'] * 1e3:.1f} us ({ev['w13_bytes'] / ev['w13_ms'] / 1e6:.0f} GB/s), down "
        f"{ev['w2_ms'] * 1e3:.1f} us, FFN call {ev['ffn_ms'] * 1e3:.1f} us")

    sweep = []
    if not args.no_sweep:
        for TT in (1, 32):
            LT = layer_for(TT)
            for tgt in (2.0, 2.5, 3.0, 4.0):
                n = max(20, args.steps // 4)
                ts = LT.timed_graph(tgt, n, 5)
                e2 = LT.timed_events(tgt, n)
                gbs = e2["ffn_bytes"] / (e2["ffn_ms"] * 1e-3) / 1e9
                g13 = e2["w13_bytes"] / (e2["w13_ms"] * 1e-3) / 1e9
                sweep.append(dict(T=TT, target=tgt, tokens_per_s=TT / ts, ms_per_step=ts * 1e3,
                                  ffn_ms=e2["ffn_ms"], ffn_gbs=gbs, ffn_frac=gbs / HBM_PEAK_GBS,
                                  w13_us=e2["w13_ms"] * 1e3, w13_gbs=g13, w13_frac=g13 / HBM_PEAK_GBS,
                                  w2_us=e2["w2_ms"] * 1e3, bits_read=e2["bits_read"], bits_alloc=e2["bits_alloc"],
                                  n_active=e2["n_active"], ffn_bytes=e2["ffn_bytes"]))
                log(f"sweep T={TT} target={tgt}: {TT / ts:.0f} tok/s, FFN {e2['ffn_ms'] * 1e3:.1f} us, "
                    f"{gbs:.0f} GB/s; gate/up {e2['w13_ms'] * 1e3:.1f} us {g13:.0f} GB/s; bits read "
                    f"{e2['bits_read']:.2f}")

    ceiling = read_ceiling(torch, bd)
    log(f"streaming-read ceiling {ceiling:.0f} GB/s")

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg, w)

    out = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s vs avg bits read (Qwen3-30B shape)",
        "value": T / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-30B-A3B-shaped single MoE layer, decode" +
                               (", ragged bank (per-expert maximum width 2/3/4)" if args.ragged else ""),
                   "tokens": T, "hidden": cfg.d,
                   "expert_intermediate": cfg.f, "experts": cfg.E, "top_k": cfg.k, "bitplanes": cfg.b_max,
                   "group": cfg.g, "b_lo": cfg.b_lo, "target_avg_bits": args.target,
                   "weight_copies_rotated": N_COPIES, "activation_batches": N_XBATCH},
        "step_gbs": step_bytes / t_step / 1e9,
        "stored_bytes_per_copy": w.routed.stored_bytes(),
        "bits_read": ev["bits_read"],
        "bits_alloc": ev["bits_alloc"],
        "n_active_experts": ev["n_active"],
        "ffn_ms": {"mean": ev["ffn_ms"], "p10": ev["ffn_ms_p10"], "p50": ev["ffn_ms_p50"], "p90": ev["ffn_ms_p90"]},
        "roofline": dict(kernel_roofline(ev, recorded_traffic(T, args.target)), read_ceiling=ceiling,
                         frac_of_read_ceiling=ev["w13_bytes"] / (ev["w13_ms"] * 1e-3) / 1e9 / ceiling),
        "cpu_baseline": cpu,
        "sweep": sweep,
    }
    print(json.dumps(out), flush=True)


def prefill(args, torch, bd, wl):
    cfg = wl.config(4, target=args.target)
    T = cfg.T
    log(f"generating the Qwen3-30B-A3B-shaped layer, prefill T={T} with Zipf-skewed load (seeded)")
    w = wl.make_workload(cfg, keep_codes=False)
    L = Layer(cfg, w, torch, bd, T)
    log(f"timing T={T} target={args.target}: {args.warmup} warmup + {args.steps} graph-replayed steps")
    t_step = L.timed_graph(args.target, args.steps, args.warmup)
    ev = L.timed_events(args.target, args.steps)
    tflops = ev["ffn_flops"] / (ev["ffn_ms"] * 1e-3) / 1e12
    f13 = ev["ffn_flops"] * 2.0 / 3.0   # gate and up: 4 d f of the 6 d f per pair
    t13 = f13 / (ev["w13_ms"] * 1e-3) / 1e12
    t2 = (ev["ffn_flops"] - f13) / (ev["w2_ms"] * 1e-3) / 1e12
    log(f"gate/up {ev['w13_ms'] * 1e3:.1f} us ({t13:.0f} TFLOP/s), down {ev['w2_ms'] * 1e3:.1f} us, "
        f"FFN call {ev['ffn_ms'] * 1e3:.1f} us ({tflops:.0f} TFLOP/s)")
    ceiling = read_ceiling(torch, bd)
    out = {
        "metric": "MoE-layer tokens/s, prefill (Qwen3-30B shape)",
        "value": T / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-30B-A3B-shaped single MoE layer, prefill, Zipf(1.1) expert load", "tokens": T,
                   "hidden": cfg.d, "expert_intermediate": cfg.f, "experts": cfg.E, "top_k": cfg.k,
                   "bitplanes": cfg.b_max, "group": cfg.g, "b_lo": cfg.b_lo, "target_avg_bits": args.target,
                   "weight_copies_rotated": N_COPIES, "activation_batches": N_XBATCH},
        "bits_read": ev["bits_read"],
        "bits_alloc": ev["bits_alloc"],
        "n_active_experts": ev["n_active"],
        "ffn_ms": {"mean": ev["ffn_ms"], "p10": ev["ffn_ms_p10"], "p50": ev["ffn_ms_p50"], "p90": ev["ffn_ms_p90"]},
        "roofline": {"bound": "mfma", "achieved": t13, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": t13 / BF16_PEAK_TFLOPS,
                     "traffic": recorded_traffic(T, args.target, PREFILL_TRAFFIC_FILE, 4096),
                     "kernel": "gate/up + SwiGLU on 64-pair chunks (k_wide<W13>), the FFN stage's dominant kernel",
                     "flops_per_launch": f13, "us_per_launch": ev["w13_ms"] * 1e3,
                     "down_kernel": {"achieved": t2, "frac": t2 / BF16_PEAK_TFLOPS,
                                     "flops_per_launch": ev["ffn_flops"] - f13, "us_per_launch": ev["w2_ms"] * 1e3},
                     "ffn_call": {"achieved": tflops, "frac": tflops / BF16_PEAK_TFLOPS,
                                  "flops_per_launch": ev["ffn_flops"], "us_per_launch": ev["ffn_ms"] * 1e3,
                                  "kernels": "plan, gather, gate/up + SwiGLU, group sums, down, combine",
                                  "hbm_gbs": ev["ffn_bytes"] / (ev["ffn_ms"] * 1e-3) / 1e9},
                     "hbm_read_ceiling_gbs": ceiling},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def deepseek(args, torch, bd, wl):
    """The DeepSeekMoE-16B-shaped decode layer: T=16, 64 routed experts of
    intermediate 1408, top-6, two always-on shared experts read at 4 bits,
    target 2.5 bits, B_lo 2 (the headline) and 1."""
    rows, head = [], None
    for b_lo in (2, 1):
        cfg = wl.config(3, b_lo=b_lo, target=2.5 if args.target == 3.0 else args.target)
        T = cfg.T
        log(f"generating the DeepSeekMoE-16B-shaped layer (seeded), B_lo {b_lo}")
        w = wl.make_workload(cfg, keep_codes=False)
        L = Layer(cfg, w, torch, bd, T)
        ts = L.timed_graph(cfg.target, args.steps, args.warmup)
        ev = L.timed_events(cfg.target, args.steps)
        g13 = ev["w13_bytes"] / (ev["w13_ms"] * 1e-3) / 1e9
        row = dict(b_lo=b_lo, target=cfg.target, tokens_per_s=T / ts, ms_per_step=ts * 1e3,
                   ffn_us=ev["ffn_ms"] * 1e3, w13_us=ev["w13_ms"] * 1e3, w13_gbs=g13, w13_frac=g13 / HBM_PEAK_GBS,
                   w2_us=ev["w2_ms"] * 1e3, bits_read=ev["bits_read"], bits_alloc=ev["bits_alloc"],
                   n_active=ev["n_active"], ffn_bytes=ev["ffn_bytes"])
        rows.append(row)
        log(f"deepseek B_lo={b_lo}: {T / ts:.0f} tok/s, FFN {ev['ffn_ms'] * 1e3:.1f} us, gate/up "
            f"{ev['w13_ms'] * 1e3:.1f} us ({g13:.0f} GB/s), bits read {ev['bits_read']:.2f}")
        if head is None:
            head = (cfg, w, ts, ev)
        del L
        torch.cuda.empty_cache()
    cfg, w, ts, ev = head
    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg, w)
    out = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s vs avg bits read (DeepSeekMoE-16B shape)",
        "value": cfg.T / ts, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ts * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "DeepSeekMoE-16B-shaped single MoE layer, decode, two shared experts",
                   "tokens": cfg.T, "hidden": cfg.d, "expert_intermediate": cfg.f, "experts": cfg.E,
                   "top_k": cfg.k, "shared_experts": cfg.n_shared, "bitplanes": cfg.b_max, "group": cfg.g,
                   "b_lo": cfg.b_lo, "target_avg_bits": cfg.target, "weight_copies_rotated": N_COPIES,
                   "activation_batches": N_XBATCH},
        "bits_read": ev["bits_read"], "bits_alloc": ev["bits_alloc"], "n_active_experts": ev["n_active"],
        "roofline": kernel_roofline(ev),
        "cpu_baseline": cpu,
        "sweep": rows,
    }
    print(json.dumps(out), flush=True)


def per_expert_modes(args, torch, bd, wl):
    """The Qwen3-30B-A3B-shaped decode layer (T=32) with widths from DuoRate's
    per-expert solve (--duorate: the distortion tensor baked from the bank,
    a 4096-token prefill of fresh activations profiled through the router,
    widths 1..4 per expert, decode steps reading each pair at its expert's
    width) or from DPA-MoE's residual-aware chunk allocation on every step
    (--dpa: widths 1..4 per pair)."""
    mode = "duorate" if args.duorate else "dpa"
    cfg = wl.config(2, T=args.tokens, b_lo=1, target=args.target)
    T = cfg.T
    log(f"generating the Qwen3-30B-A3B-shaped layer (seeded); {mode} widths")
    w = wl.make_workload(cfg, keep_codes=False)
    L = Layer(cfg, w, torch, bd, T)
    L.policy = mode
    extra = {}
    if mode == "duorate":
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        delta = bd.duorate_bake(L.banks[0])
        torch.cuda.synchronize()
        t_bake = time.perf_counter() - t0
        xp = bd.bf16_tensor(wl.step_activations(cfg, 50_000, 4096))
        idx_p, _ = bd.route(xp, L.wr, None, cfg.k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a, n = bd.duorate_profile(xp, idx_p, cfg.E)
        torch.cuda.synchronize()
        t_prof = time.perf_counter() - t0
        n_np = n.cpu().numpy().astype(np.int64)
        extra = {"bake_ms": t_bake * 1e3, "profile_ms": t_prof * 1e3, "prefill_tokens": 4096}
    else:
        L.resid = bd.dpa_residuals(L.banks[0])
        L.dws = torch.empty(max(256, int(bd.lib().moe_dpa_alloc_workspace_bytes(T * cfg.k, cfg.b_lo, cfg.b_max))),
                            dtype=torch.uint8, device="cuda")
    stored_bpw = cfg.b_max + 64.0 / cfg.g   # the uniform stored tier plus fp32 (scale, zero) per group
    rows, head = [], None
    targets = sorted({1.75, 2.0, 2.3, 2.5, 2.9, 3.0, 3.5, args.target})
    for tgt in targets:
        if mode == "duorate":
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            wts, D, lam = bd.duorate_solve(delta, a, n, cfg.b_lo, cfg.b_max, tgt)
            torch.cuda.synchronize()
            t_solve = time.perf_counter() - t0
            L.expert_bits = wts
            wn = wts.cpu().numpy().astype(np.int64)
            prof_rate = float(np.dot(n_np, wn)) / max(1, int(n_np.sum()))
        ts = L.timed_graph(tgt, args.steps, args.warmup)
        ev = L.timed_events(tgt, args.steps)
        g13 = ev["w13_bytes"] / (ev["w13_ms"] * 1e-3) / 1e9
        row = dict(target=tgt, tokens_per_s=T / ts, ms_per_step=ts * 1e3, ffn_us=ev["ffn_ms"] * 1e3,
                   w13_us=ev["w13_ms"] * 1e3, w13_gbs=g13, w13_frac=g13 / HBM_PEAK_GBS, w2_us=ev["w2_ms"] * 1e3,
                   bits_read=ev["bits_read"], bits_alloc=ev["bits_alloc"], n_active=ev["n_active"],
                   stored_bpw=stored_bpw, read_bpw=ev["bits_read"] + 64.0 / cfg.g)
        if mode == "duorate":
            row.update(solve_ms=t_solve * 1e3, lam=float(lam.item()), profile_rate=prof_rate,
                       expert_widths=np.bincount(wn, minlength=cfg.b_max + 1)[1:].tolist())
        rows.append(row)
        log(f"{mode} target={tgt}: {T / ts:.0f} tok/s, gate/up {ev['w13_ms'] * 1e3:.1f} us ({g13:.0f} GB/s), "
            f"bits read {ev['bits_read']:.2f}, allocated {ev['bits_alloc']:.2f}")
        if tgt == args.target:
            head = (ts, ev, row)
    ts, ev, row = head
    name = "DuoRate per-expert widths" if mode == "duorate" else "DPA-MoE residual-aware chunk allocation"
    out = {
        "metric": f"MoE-layer tokens/s, {name} (Qwen3-30B shape)",
        "value": T / ts, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ts * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"Qwen3-30B-A3B-shaped single MoE layer, decode, {name}", "tokens": T,
                   "hidden": cfg.d, "expert_intermediate": cfg.f, "experts": cfg.E, "top_k": cfg.k,
                   "bitplanes": cfg.b_max, "group": cfg.g, "widths": [cfg.b_lo, cfg.b_max],
                   "target_rate_bits": args.target, "weight_copies_rotated": N_COPIES,
                   "activation_batches": N_XBATCH},
        "bits_read": ev["bits_read"], "bits_alloc": ev["bits_alloc"], "stored_bpw": stored_bpw,
        "read_bpw": row["read_bpw"],
        "roofline": kernel_roofline(ev),
        "cpu_baseline": None,
        "sweep": rows,
        **extra,
    }
    print(json.dumps(out), flush=True)


N_CAL = 64  # calibration batches (and as many held-out batches)


def calibrated(args, torch, bd, wl):
    cfg = wl.config(2, T=args.tokens, target=args.target)
    T = cfg.T
    log(f"generating the Qwen3-30B-A3B-shaped layer (seeded); calibration-threshold mode, T={T}")
    w = wl.make_workload(cfg, keep_codes=False)
    L = Layer(cfg, w, torch, bd, T)

    def gates_of(first):
        out = []
        for s in range(N_CAL):
            x = bd.bf16_tensor(wl.step_activations(cfg, first + s, T))
            out.append(bd.route(x, L.wr, L.bias, cfg.k)[1].reshape(-1))
        return torch.cat(out)

    cal, held = gates_of(10_000), gates_of(20_000)   # distinct from the timed batches (steps 0..7)
    tau_t = torch.empty(1, dtype=torch.float32, device="cuda")
    rows, head = [], None
    for tgt in sorted({2.5, 3.0, 3.5, args.target}):
        bd.alloc_bits(cal, cfg.b_lo, cfg.b_max, tgt, tau=tau_t)   # the bisection, once, on the calibration set
        tau = float(tau_t.item())
        hb = bd.bits_from_threshold(held, tau, cfg.b_lo, cfg.b_max).view(N_CAL, T * cfg.k).float().mean(1).cpu().numpy()
        L.tau = tau
        L.policy = "calibrated"
        ts = L.timed_graph(tgt, args.steps, args.warmup)
        ev = L.timed_events(tgt, args.steps)
        row = dict(target=tgt, tau=tau, tokens_per_s=T / ts, ms_per_step=ts * 1e3, ffn_ms=ev["ffn_ms"],
                   ffn_gbs=ev["ffn_bytes"] / (ev["ffn_ms"] * 1e-3) / 1e9, bits_read=ev["bits_read"],
                   held_out_bits={"mean": float(hb.mean()), "std": float(hb.std()), "min": float(hb.min()),
                                  "max": float(hb.max())})
        rows.append(row)
        log(f"calibrated target={tgt}: tau {tau:.6g}, {T / ts:.0f} tok/s, FFN {ev['ffn_ms'] * 1e3:.1f} us; held-out "
            f"per-step bits {hb.mean():.3f} +- {hb.std():.3f} (min {hb.min():.3f}, max {hb.max():.3f})")
        if tgt == args.target:
            head = (ts, ev, row)
    ts, ev, row = head
    out = {
        "metric": "MoE-layer tokens/s, calibration-threshold mode (Qwen3-30B shape)",
        "value": T / ts,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ts * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-30B-A3B-shaped single MoE layer, decode, calibrated gate threshold",
                   "tokens": T, "hidden": cfg.d, "expert_intermediate": cfg.f, "experts": cfg.E, "top_k": cfg.k,
                   "bitplanes": cfg.b_max, "group": cfg.g, "b_lo": cfg.b_lo, "target_avg_bits": args.target,
                   "calibration_batches": N_CAL, "held_out_batches": N_CAL,
                   "weight_copies_rotated": N_COPIES, "activation_batches": N_XBATCH},
        "tau": row["tau"],
        "held_out_bits": row["held_out_bits"],
        "bits_read": ev["bits_read"],
        "bits_alloc": ev["bits_alloc"],
        "roofline": kernel_roofline(ev),
        "cpu_baseline": None,
        "sweep": rows,
    }
    print(json.dumps(out), flush=True)


N_LAYERS = 48
RMS_EPS = 1e-6


class Stack:
    """The 48-layer stack on the device: per layer a router and an expert
    bank; a fp32 residual h and its bf16 cast x; per layer the routing and
    widths of the last step; HIP graphs of whole steps."""

    def __init__(self, cfg, torch, bd, wl):
        self.cfg, self.torch, self.bd = cfg, torch, bd
        T, dev = cfg.T, "cuda"
        self.layers = []
        t0 = time.perf_counter()
        for l in range(N_LAYERS):
            wr, bank = wl.make_stack_layer(cfg, l)
            self.layers.append((torch.from_numpy(wr).to(dev), bd.DeviceBank.from_host(bank)))
            del wr, bank
            if l % 8 == 7:
                log(f"stack: {l + 1} layers resident ({time.perf_counter() - t0:.0f} s)")
        self.h0 = [torch.from_numpy(wl.bf16_bits_to_f32(wl.step_activations(cfg, s, T))).to(dev)
                   for s in range(N_XBATCH)]
        self.h = torch.empty(T, cfg.d, dtype=torch.float32, device=dev)
        self.x = torch.empty(T, cfg.d, dtype=torch.bfloat16, device=dev)
        self.lws = bd.layer_workspace(self.layers[0][1], None, T, cfg.k)
        self.idx = [torch.empty(T, cfg.k, dtype=torch.int32, device=dev) for _ in range(N_LAYERS)]
        self.gate = [torch.empty(T, cfg.k, dtype=torch.float32, device=dev) for _ in range(N_LAYERS)]
        self.bits = [torch.empty(T * cfg.k, dtype=torch.uint8, device=dev) for _ in range(N_LAYERS)]
        self.graphs = {}

    def step(self, i, target):
        """Decode step on activation batch i mod 8: h = x0, then per layer
        h += layer(bf16(rmsnorm(h)))."""
        bd, cfg = self.bd, self.cfg
        self.h.copy_(self.h0[i % N_XBATCH])
        bd.rmsnorm_to_bf16(self.h, self.x, eps=RMS_EPS)
        for l, (wr, bank) in enumerate(self.layers):
            bd.layer(bank, None, self.x, wr, None, cfg.k, cfg.b_lo, target, y=self.h, accumulate=True,
                     idx=self.idx[l], gate=self.gate[l], bits=self.bits[l], workspace=self.lws)
            bd.rmsnorm_to_bf16(self.h, self.x, eps=RMS_EPS)

    def timed(self, target, steps, warmup):
        """Steps replayed from a graph of one cycle of the 8 activation
        batches (plus one of the remainder); seconds per step."""
        torch = self.torch
        key = float(target)
        if key not in self.graphs:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self.step(0, target)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            gs = []
            for n in (N_XBATCH, steps % N_XBATCH):
                if n == 0:
                    gs.append(None)
                    continue
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(n):
                        self.step(i, target)
                gs.append(g)
            torch.cuda.synchronize()
            self.graphs[key] = gs
        full, rem = self.graphs[key]
        for _ in range(max(1, -(-warmup // N_XBATCH))):
            full.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps // N_XBATCH):
            full.replay()
        if rem is not None:
            rem.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def step_bytes(self, target):
        """Algorithmic bytes of one step (batch 0), from its routing and widths."""
        self.step(0, target)
        self.torch.cuda.synchronize()
        tot, bread, balloc, nact = 0.0, [], [], []
        for l in range(N_LAYERS):
            b, br, ba, na = algorithmic_ffn_bytes(self.idx[l].cpu().numpy(), self.bits[l].cpu().numpy(), self.cfg,
                                                  accumulate=True)
            tot += b + router_bytes(self.cfg, self.cfg.T)
            bread.append(br); balloc.append(ba); nact.append(na)
        return tot, float(np.mean(bread)), float(np.mean(balloc)), float(np.mean(nact))


def stack(args, torch, bd, wl):
    cfg = wl.config(5, target=args.target)
    T = cfg.T
    log(f"generating the 48-layer Qwen3-30B-A3B-shaped stack, T={T} (seeded)")
    S = Stack(cfg, torch, bd, wl)
    targets = [args.target] if args.no_sweep else [2.0 + 0.25 * i for i in range(9)]
    if args.target not in targets:
        targets.insert(0, args.target)
    sweep, head = [], None
    for tgt in targets:
        ts = S.timed(tgt, args.steps, args.warmup)
        nbytes, br, ba, na = S.step_bytes(tgt)
        row = dict(target=tgt, tokens_per_s=T / ts, ms_per_step=ts * 1e3, step_gbs=nbytes / ts / 1e9,
                   step_bytes=nbytes, bits_read=br, bits_alloc=ba, n_active=na)
        sweep.append(row)
        log(f"stack target={tgt}: {T / ts:.0f} tok/s, {ts * 1e3:.3f} ms per step, {nbytes / ts / 1e9:.0f} GB/s, "
            f"bits read {br:.2f}, bits allocated {ba:.2f}")
        if tgt == args.target:
            head = (ts, row)
    ceiling = read_ceiling(torch, bd)
    ts, row = head
    out = {
        "metric": "48-layer stack decode tokens/s + achieved HBM GB/s vs avg bits read (Qwen3-30B shape)",
        "value": T / ts,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ts * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "48 Qwen3-30B-A3B-shaped MoE layers, decode, residual carried", "tokens": T,
                   "layers": N_LAYERS, "hidden": cfg.d, "expert_intermediate": cfg.f, "experts": cfg.E,
                   "top_k": cfg.k, "bitplanes": cfg.b_max, "group": cfg.g, "b_lo": cfg.b_lo,
                   "target_avg_bits": args.target, "activation_batches": N_XBATCH},
        "bits_read": row["bits_read"],
        "bits_alloc": row["bits_alloc"],
        "n_active_experts": row["n_active"],
        "roofline": {"bound": "hbm", "achieved": row["step_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": row["step_gbs"] / HBM_PEAK_GBS, "traffic": None, "read_ceiling": ceiling,
                     "frac_of_read_ceiling": row["step_gbs"] / ceiling,
                     "kernel": "whole step: 48 x (RMS-normalised cast + moe_layer)", "bytes_per_step": row["step_bytes"]},
        "cpu_baseline": None,
        "sweep": sweep,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
