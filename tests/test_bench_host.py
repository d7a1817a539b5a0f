"""Host-side logic of bench.py (no GPU): the single-GPU refusal, the decode's
algorithmic bytes per token, and the rule that counted HBM traffic is only
reported for the kernel source it was taken on."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_a_token():
    # per layer: all of K1 (r x d_ff bf16), per selected neuron its K2 row
    # (d_model - r bf16) and V row (d_model bf16), the fp32 input and output
    counts = np.full(bench.LAYERS, 737)
    per_layer = 1152 * 9216 * 2 + 737 * ((2304 - 1152) + 2304) * 2 + 2 * 2304 * 4
    assert bench.algorithmic_bytes(counts) == 26 * per_layer
    # only the total count matters, not how it is spread over the layers
    uneven = counts.copy()
    uneven[0] += 5
    uneven[1] -= 5
    assert bench.algorithmic_bytes(uneven) == bench.algorithmic_bytes(counts)
    assert abs(bench.algorithmic_bytes(counts) / 1e6 - 685.00) < 0.01


def test_traffic_only_for_the_current_kernel_source(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "decode_traffic.json")) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "source_hash", lambda: rec["source_hash"])
    assert bench.load_traffic() == rec["hbm_bytes_per_launch"]
    # the record's total is its two counters, each scaled by the copy kernel's reading
    fetch = rec["fetch_kib_per_launch_raw"] * 1024 * rec["copy_fetch_scale"]
    write = rec["write_kib_per_launch_raw"] * 1024 * rec["copy_write_scale"]
    # (the stored scales are rounded to three decimals)
    assert abs(fetch + write - rec["hbm_bytes_per_launch"]) <= 1e-4 * rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.load_traffic() is None
