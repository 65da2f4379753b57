"""Host-side checks of the benchmark's bookkeeping (no GPU): the algorithmic
byte counts behind the roofline figure, the counter records it reports as
traffic, and its refusals."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import phx_inputs  # noqa: E402


def test_pi05_algorithmic_bytes():
    # per Euler step: 18 layers of W_qkv [1024 x 2560], W_o [2048 x 1024], W_gu [1024 x 8192] and
    # W_down [4096 x 1024] in bf16, the 32-wide in- and out-projections, 768 prefix rows of one
    # 256-wide key and value head per layer, and 37 modulation rows of 2 x 1024 fp32
    cfg = phx_inputs.workload("pi05_expert_bf16")
    ab = bench.algorithmic_bytes(cfg)
    w_layer = (1024 * 2560 + 2048 * 1024 + 1024 * 8192 + 4096 * 1024) * 2
    w_step = 18 * w_layer + 2 * 32 * 1024 * 2
    kv_step = 18 * 768 * 256 * 2 * 2
    mod_step = 37 * 2 * 1024 * 4
    assert ab["weights_per_step"] == w_step
    assert ab["kv_per_step"] == kv_step
    assert ab["per_decision"] == 10 * (w_step + kv_step + mod_step) == 6374440960


def test_w8_algorithmic_bytes():
    # the 8-bit tier: one byte per code of the layer projections plus a float scale per output column
    cfg = phx_inputs.workload("pi05_expert_w8a16")
    ab = bench.algorithmic_bytes(cfg)
    w_layer = (1024 * 2560 + 2048 * 1024 + 1024 * 8192 + 4096 * 1024) + 4 * (2560 + 1024 + 8192 + 1024)
    assert ab["weights_per_step"] == 18 * w_layer + 2 * 32 * 1024 * 2
    assert ab["per_decision"] == 3269386240


@pytest.mark.parametrize("name", sorted(bench.TRAFFIC_FILES))
def test_traffic_records_are_whole(name):
    with open(bench.TRAFFIC_FILES[name]) as fh:
        t = json.load(fh)
    assert t["bytes_per_launch"] == t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    assert t["bytes_per_launch"] > t["algorithmic_bytes_per_launch"] > 0
    assert len(t["kernel_hash"]) == 16 and len(t["commands"]) == 2
    # reported only for the sources the counters were taken on
    assert bench.measured_traffic(t["kernel_hash"], name) == t["bytes_per_launch"]
    assert bench.measured_traffic("0" * 16, name) is None


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr + r.stdout
