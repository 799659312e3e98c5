"""bench.py's host logic, on the CPU: the single-GPU refusal, the algorithmic byte counts of
decode attention, and the rule that ties the reported HBM traffic to the kernel source the
counters were taken on."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from workloads import custom
from workloads.gen import Request

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_decode_bytes_by_hand():
    """K and V rows of every position for all key/value heads, 2 B of query and 4 B of output
    per query-head element, and the mapping entries the positions resolve through."""
    reqs = [Request(40, 1), Request(17, 1), Request(0, 0)]
    w = custom("bytes", 3, reqs, block_size=16, num_blocks=64, runs=("count", 2, 2),
               num_kv_heads=2, head_dim=128)
    ctx = np.array([rq.end for rq in reqs], np.int64)
    kv = (40 + 17) * 2 * 128 * 2 * 2
    qo = 3 * 8 * 128 * (2 + 4)
    # paged: one 4-byte table entry per block in use (3 blocks + 2 blocks)
    assert bench.decode_bytes(w, ctx, 8, "paged") == kv + qo + 4 * (3 + 2)
    # ranges: 12 bytes per run descriptor in use plus a 4-byte count per request
    runs = int(w.num_ranges.sum())
    assert bench.decode_bytes(w, ctx, 8, "ranges") == kv + qo + 12 * runs + 4 * 3


def test_counter_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    """The committed counter figure is reported only while the kernel source is the one the
    counters were taken on."""
    src = tmp_path / "kernel.hip"
    src.write_text("// one version of the kernel\nint x = 1;\n")
    counters = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    monkeypatch.setattr(bench, "COUNTERS", str(counters))
    assert bench.counter_traffic() is None  # no counter file
    counters.write_text(json.dumps({"kernel_source_sha256": bench.kernel_source_hash(),
                                    "traffic_bytes_per_launch": 1234}))
    assert bench.counter_traffic() == 1234
    # comments, trailing blanks and empty lines do not change the compiled kernel
    src.write_text("/* a comment\n   over lines */\n// another\nint x = 1;   // same code\n\n")
    assert bench.counter_traffic() == 1234
    src.write_text("// the kernel changed since\nint x = 2;\n")
    assert bench.counter_traffic() is None
    counters.write_text("not json")
    assert bench.counter_traffic() is None


def test_committed_counters_match_the_current_source():
    """The counter summary under profiles/ was taken on today's write-path source."""
    with open(bench.COUNTERS) as f:
        c = json.load(f)
    assert c["kernel_source_sha256"] == bench.kernel_source_hash()
    assert c["traffic_bytes_per_launch"] >= c["algorithmic_bytes_per_launch"]
