"""bench.py's host logic on the CPU: the metric's byte count, the counter
file lookup and the one-GPU rule (no GPU is touched)."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gqa_mqa_kv_amd import workloads  # noqa: E402


def test_algorithmic_bytes_follow_the_footprint_formula():
    """K + V of the valid tokens (2 x tokens x H_kv x d x bytes per element,
    the KV footprint formula per layer) plus q and out: 268,697,600 B for the
    Llama-3-8B-shaped layer, 134,348,800 B for the MQA sweep run."""
    w = workloads.WORKLOADS["llama3-8b-layer"]
    sl = workloads.seq_lens_for(w)
    assert bench.algorithmic_bytes(w, sl, 2) == 268_697_600
    assert bench.algorithmic_bytes(workloads.WORKLOADS["grouping-sweep-mqa"],
                                   workloads.seq_lens_for(workloads.WORKLOADS["grouping-sweep-mqa"]), 2) == 134_348_800
    # fp32 output: out counted at 4 bytes per element
    assert bench.algorithmic_bytes(w, sl, 4) == 268_697_600 + 16 * 32 * 128 * 2
    # pages: plus one 4-byte table entry per page in use (16 x 4096 / 16 pages)
    assert bench.algorithmic_bytes(w, sl, 2, page=16) == 268_697_600 + 4 * 16 * 256
    # one-byte cache elements: K and V halve, q and out do not
    assert bench.algorithmic_bytes(w, sl, 2, kv_elem_bytes=1) == 268_435_456 // 2 + 262_144


def test_counter_files_are_keyed_by_workload_and_layout():
    assert bench.traffic_profile("llama3-8b-layer").endswith("gqa_decode_mfma_llama3_8b_layer_counters.txt")
    assert bench.traffic_profile("llama3-8b-layer/paged16/fp8").endswith(
        "gqa_decode_mfma_llama3_8b_layer_paged16_fp8_counters.txt")
    assert bench.read_traffic("no-such-workload", 1) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_samples_layers_of_a_layer_batched_workload():
    """A layer-batched workload's baseline times the oracle on whole layers
    (0, 1, ...) until the budget is spent and scales the mean to all layers;
    a tiny budget samples exactly one layer."""
    w = workloads.Workload("stack-tiny", 3, 8, 2, 64, 20, 60, torch.bfloat16, 5, layers=4, packed=True)
    x = workloads.generate(w, "cpu")
    r = bench.cpu_baseline(w, budget_s=0.0, x=x)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0 and r["cores"] >= 1
    assert r["sample"].startswith("1 of 4 layers of stack-tiny")
    nbytes = bench.algorithmic_bytes(w, x["seq_lens"], 2)
    assert abs(nbytes / (r["us_per_step"] * 1e-6) / 1e9 - r["value"]) <= 1e-3 * r["value"] + 1e-3
    r = bench.cpu_baseline(w, budget_s=60.0, x=x)
    assert r["sample"].startswith("4 of 4 layers")
