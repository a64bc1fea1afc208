"""Oracle work for the full-size GPU parity tests, run in worker processes.

The 48-layer stack case needs the oracle's per-pair FFN over many experts
of every layer; a pool of spawned workers (NumPy only, no GPU) shares that
work.
Each worker rebuilds its inputs from the seeded generators and calls the
oracle unchanged."""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pool_size() -> int:
    """Workers for the oracle pool: the CPUs this process may use, at most 8
    (each worker holds one layer's dequantised experts, a few GB)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(8, n))


def stack_layer(task):
    """Teacher-forced oracle for one layer of the 48-layer stack.

    task = (layer, {target: (x_rows, idx_rows, gate_rows, bits_rows)}):
    the GPU's own layer input, routing, gates and widths on a few rows.
    Returns {target: y_rows} from the oracle's combine."""
    from dynamic_any_precision_amd import workloads as wl
    import oracle as orc
    layer, cases = task
    cfg = wl.config(5)
    _, bank = wl.make_stack_layer(cfg, layer)
    oc = orc.bank_cache(bank)
    out = {}
    for target, (x, idx, gate, bits) in cases.items():
        out[target] = orc.combine(x, idx, gate.astype(np.float64), bits, oc)
    return layer, out

