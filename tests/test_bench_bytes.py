"""Host checks of bench.py's algorithmic byte count (the numerator of the
roofline it reports), against counts worked out by hand."""
import numpy as np

import bench
from dynamic_any_precision_amd import workloads as wl


def test_batch1_bytes_by_hand():
    # Qwen3-30B-A3B shape: one token, experts 0..7, expert 0 at 4 bits and
    # the rest at 2.  Per expert and plane the three matrices hold
    # 3 * 2048 * 768 / 8 = 589 824 bytes; (scale, zero) of one expert
    # 3 * 2048 * 768 / 128 groups * 8 bytes = 294 912 bytes.
    cfg = wl.config(2, T=1)
    idx = np.arange(8, dtype=np.int32).reshape(1, 8)
    bits = np.array([4, 2, 2, 2, 2, 2, 2, 2], dtype=np.uint8)
    total, bread, balloc, nact = bench.algorithmic_ffn_bytes(idx, bits, cfg)
    planes = (4 + 7 * 2) * 589_824
    sz = 8 * 294_912
    io = 2048 * 2 + 2048 * 4 + 8 * 768 * 2 * 2   # x in, y out, h written and read
    assert total == planes + sz + io == 13_012_992
    assert bread == 18 / 8 and balloc == 18 / 8 and nact == 8


def test_shared_expert_reads_its_widest_pair_once():
    # two tokens on the same expert 5 at 1 and 3 bits: the expert's planes
    # are read once at 3 bits; accumulate reads y as well as writing it
    cfg = wl.config(1, T=2)                 # d 256, f 128, g 64, E 8, k 2
    idx = np.array([[5, 0], [5, 1]], dtype=np.int32)
    bits = np.array([1, 2, 3, 2], dtype=np.uint8)
    total, bread, balloc, nact = bench.algorithmic_ffn_bytes(idx, bits, cfg, accumulate=True)
    per_plane = 3 * 256 * 128 // 8           # 12 288
    per_sz = 3 * 256 * 128 // 64 * 8         # 12 288
    planes = (3 + 2 + 2) * per_plane         # experts 5, 0, 1
    io = 2 * 256 * 2 + 2 * 256 * 4 * 2 + 4 * 128 * 2 * 2
    assert total == planes + 3 * per_sz + io
    assert nact == 3 and bread == 7 / 3 and balloc == 2.0


def test_recorded_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    # the counter record is used only for its own workload and while the
    # kernel sources hash to the recorded value
    rec = tmp_path / "rec.md"
    rec.write_text(f"# x\n\nsource_sha256: {bench.ffn_source_hash()}\ntraffic_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.recorded_traffic(32, 3.0) == 12345.0
    assert bench.recorded_traffic(1, 3.0) is None
    assert bench.recorded_traffic(32, 2.5) is None
    rec.write_text("source_sha256: 0000000000000000\ntraffic_bytes_per_launch: 12345\n")
    assert bench.recorded_traffic(32, 3.0) is None
    # the prefill record: its own file and token count
    pre = tmp_path / "pre.md"
    pre.write_text(f"source_sha256: {bench.ffn_source_hash()}\ntraffic_bytes_per_launch: 777\n")
    assert bench.recorded_traffic(4096, 3.0, str(pre), 4096) == 777.0
    assert bench.recorded_traffic(32, 3.0, str(pre), 4096) is None


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr
