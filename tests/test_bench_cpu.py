"""CPU checks of bench.py: its accounting, its one-GPU contract and the
host-side pieces of its passes (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
import workload  # noqa: E402


def test_llama_accounting():
    w = workload.WORKLOADS["llama3_8b_bf16_causal"]
    # 4 b h n^2 d_k / 2 and Q + K + V + O in bf16 plus fp32 LSE
    assert bench.algorithmic_flops(w) == 4 * 32 * 8192 ** 2 * 128 / 2 == 5.49755813888e11
    assert bench.min_hbm_bytes(w) == 269484032
    assert bench.backward_flops(w) == 2.5 * bench.algorithmic_flops(w)


@pytest.mark.parametrize("name", sorted(workload.WORKLOADS))
def test_roofline_denominators_match_an_independent_count(name):
    """bench.py keeps its own FLOP and byte counts (it may not import the
    oracle outside its CPU-baseline leg). Both are pinned here for every
    workload: the bytes against the sizes of the tensors the generator makes
    plus the O and LSE tensors bench.py allocates for them, the FLOPs against
    the two products of one head counted on a tiny case and scaled, and both
    against the oracle's own accounting."""
    w = workload.WORKLOADS[name]
    rows = 16
    inp = workload.make_inputs(1, 1, rows, w.d_k, w.dtype, seed=0)
    o = torch.empty(1, 1, rows, w.d_k, dtype=workload.torch_dtype(w.out_dtype))
    lse = torch.empty(1, 1, rows, dtype=torch.float32)
    per_row = sum(t.numel() * t.element_size() for t in (inp.q, inp.k, inp.v, o, lse)) // rows
    assert bench.min_hbm_bytes(w) == w.batch * w.heads * w.n * per_row
    assert bench.min_hbm_bytes(w) == oracle.min_hbm_bytes(w.batch, w.heads, w.n, w.d_k, w.dtype, w.out_dtype)
    # S = Q K^T and O = P V: 2 n d_k FLOP per (query, key) each, over all n^2
    # pairs, halved by convention under the causal mask
    pairs = w.n * w.n
    assert bench.algorithmic_flops(w) == w.batch * w.heads * 2 * (2 * w.d_k) * pairs / (2 if w.causal else 1)
    assert bench.algorithmic_flops(w) == oracle.flops(w.batch, w.heads, w.n, w.d_k, w.causal)


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
