"""Host-side parts of bench.py, without a GPU: the one-GPU refusal, the parsing
of the committed counter summaries, and the CPU baseline leg."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _fields(path):
    out = {}
    for line in open(os.path.join(ROOT, path)):
        if ":" in line:
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


@pytest.mark.parametrize("key", sorted(bench.TRAFFIC_FILES))
def test_counter_summaries_are_consistent(key):
    """Every counter summary the bench reads holds a source hash, the scaled
    fetch and write bytes, their sum, and the algorithmic bytes it is compared with."""
    f = _fields(bench.TRAFFIC_FILES[key])
    assert len(f["source_sha256"]) == 64
    fetch, write = [int(x.split()[-1]) for x in f["scaled bytes per launch"].split(",")]
    assert fetch + write == int(f["traffic_bytes_per_launch"])
    algo = int(next(v for k, v in f.items() if k.startswith("algorithmic bytes per launch")))
    # counter traffic at least the algorithmic bytes, within a few times of them
    assert 0.99 * algo <= fetch + write <= 3 * algo


def test_cpu_baseline_runs_the_oracle():
    from paged_kv_decode_slot_amd import workloads as W

    r = bench.cpu_baseline(W.config_case(1), 0.0)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0 and r["cores"] >= 1
