"""The benchmark's accounting, on the CPU.

- Algorithmic bytes and FLOPs per stage against figures worked out by hand
  from the workload shapes: one attention layer reads every K and V row of
  every sequence's context and tree once and reads Q / writes O once, 35.7 /
  346 / 223 / 547 MB for the vicuna7b / 13b / 33b / zephyr7b shapes; the
  heads read both weight matrices of every head once, 1.183 / 1.901 / 2.058 /
  1.478 GB, for 2·B·K·(H² + H·V) = 1.18 / 7.60 / 2.06 / 11.83 GFLOP.
- The counter-record guard: a record of HBM counters stands only for the
  kernel source it was taken from (sha256); any other source gives no traffic
  figure.
- One GPU: --gpus above 1 exits with a message before touching a GPU.
"""
import hashlib
import json
import os
import subprocess
import sys

import pytest

import bench
from medusa_tree_verification_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SHAPES = ["vicuna7b-shaped", "vicuna13b-shaped", "vicuna33b-shaped", "zephyr7b-shaped"]
ATTN_MB = [35.65, 346.0, 223.3, 547.4]
HEAD_WEIGHT_GB = [1.183, 1.901, 2.058, 1.478]
HEAD_GFLOP = [1.18, 7.60, 2.06, 11.83]


@pytest.mark.parametrize("i", range(4))
def test_stage_accounting(i):
    w = synth.WORKLOADS[SHAPES[i]]
    assert bench.attention_bytes(w) / 1e6 == pytest.approx(ATTN_MB[i], rel=2e-3)
    hb = bench.heads_bytes(w) / 1e9
    # the weights dominate; activations and fp32 logits add well under 1%
    assert HEAD_WEIGHT_GB[i] <= hb + 5e-4 and hb <= HEAD_WEIGHT_GB[i] * 1.01
    assert bench.heads_flops(w) / 1e9 == pytest.approx(HEAD_GFLOP[i], rel=5e-3)


def _record(tmp, wl, source_text, traffic):
    os.makedirs(os.path.join(tmp, "profiles"))
    os.makedirs(os.path.join(tmp, "medusa_tree_verification_amd", "csrc"))
    with open(os.path.join(tmp, "medusa_tree_verification_amd", "csrc", "attention.hip"), "w") as f:
        f.write("current source\n")
    rec = {"workload": wl,
           "sources": {"attention.hip": hashlib.sha256(source_text.encode()).hexdigest()},
           "traffic_bytes_per_launch": {"tree_attention": traffic}}
    with open(os.path.join(tmp, "profiles", f"hbm_counters_{wl}.txt"), "w") as f:
        f.write("header\nrecord: " + json.dumps(rec) + "\n")


def test_counter_record_stands_only_for_its_source(tmp_path, monkeypatch):
    w = synth.WORKLOADS["vicuna7b-shaped"]
    same = tmp_path / "same"
    _record(str(same), w.name, "current source\n", 123)
    monkeypatch.setattr(bench, "ROOT", str(same))
    assert bench.counter_traffic(w, "tree_attention", "attention.hip") == 123
    other = tmp_path / "other"
    _record(str(other), w.name, "an older source\n", 123)
    monkeypatch.setattr(bench, "ROOT", str(other))
    assert bench.counter_traffic(w, "tree_attention", "attention.hip") is None
    monkeypatch.setattr(bench, "ROOT", str(tmp_path / "missing"))
    assert bench.counter_traffic(w, "tree_attention", "attention.hip") is None


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
