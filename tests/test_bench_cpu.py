"""CPU checks of bench.py: its accounting, its one-GPU contract and the
host-side pieces of its passes (no GPU needed)."""
import json
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workload  # noqa: E402


def test_llama_accounting():
    w = workload.WORKLOADS["llama3_8b_bf16_causal"]
    # 4 b h n^2 d_k / 2 and Q + K + V + O in bf16 plus fp32 LSE
    assert bench.algorithmic_flops(w) == 4 * 32 * 8192 ** 2 * 128 / 2 == 5.49755813888e11
    assert bench.min_hbm_bytes(w) == 269484032
    assert bench.backward_flops(w) == 2.5 * bench.algorithmic_flops(w)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_scrub_read_runs_on_a_plain_tensor():
    scrub = torch.ones(1 << 12, dtype=torch.float32)
    acc = torch.zeros((), dtype=torch.float32)
    bench.scrub_read(scrub, acc)
    assert acc.item() == float(1 << 12)


def test_traffic_record_names_the_kernel_sources():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["kernel_sources"] == list(bench.KERNEL_SOURCES)
    assert len(t["kernel_source_hash"]) == len(bench.kernel_source_hash())
    assert t["hbm_bytes_per_launch"] == t["hbm_read_bytes_per_launch"] + t["hbm_write_bytes_per_launch"]
