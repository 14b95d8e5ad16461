"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the count of
query-key pairs a block pattern keeps (against brute force), the gate that
reports measured HBM traffic only for the anchor source it was measured on,
and the CPU-baseline sampler on a tiny workload."""
import os
import subprocess
import sys
import types

import numpy as np
import pytest
import torch

import bench
from workloads.sparsity import random_pattern

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _pairs_brute(N, offsets, indices):
    nkb = -(-N // 64)
    keep = np.zeros((N, N), dtype=bool)
    for qb in range(len(offsets) - 1):
        for b in indices[offsets[qb]:offsets[qb + 1]]:
            if 0 <= b < nkb:
                keep[qb * 256:(qb + 1) * 256, b * 64:(b + 1) * 64] = True
    return int(keep.sum())


@pytest.mark.parametrize("N", [1, 63, 300, 700, 1025])
def test_pattern_pairs_match_brute_force(N):
    off, idx = random_pattern(N, keep=0.4, seed=N, empty_every=3, invalid=2, shuffle=True)
    lists = [list(idx[off[q]:off[q + 1]]) for q in range(len(off) - 1)]
    for blocks in lists:
        if blocks:
            blocks.append(blocks[0])          # a repeated index counts once
    off = np.cumsum([0] + [len(b) for b in lists]).astype(np.int32)
    idx = np.asarray([b for blocks in lists for b in blocks], dtype=np.int32)
    assert bench.pattern_pairs(N, off, idx) == _pairs_brute(N, off, idx)
    for qb in range(len(off) - 1):
        sub = idx[off[qb]:off[qb + 1]]
        off_q = np.zeros_like(off)
        off_q[qb + 1:] = sub.size
        assert bench.pattern_pairs(N, off, idx, only=qb) == _pairs_brute(N, off_q, sub)


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    path = tmp_path / "anchor_toy_pmc.txt"
    monkeypatch.setattr(bench, "pmc_summary_path", lambda label: str(path))
    assert bench.measured_traffic("toy") is None                 # no summary
    path.write_text(f"# header\nworkload: toy\nanchor_source_sha256: {bench.anchor_source_hash()}\n"
                    "traffic_bytes_per_launch: 12345.0\n")
    assert bench.measured_traffic("toy") == 12345.0
    assert bench.measured_traffic("other") is None               # another workload
    path.write_text("workload: toy\nanchor_source_sha256: 0000000000000000\n"
                    "traffic_bytes_per_launch: 12345.0\n")
    assert bench.measured_traffic("toy") is None                 # kernel changed since


def test_cpu_baseline_sampler_on_a_tiny_workload():
    w = types.SimpleNamespace(B=1, H=3, N=300, d=16)
    g = torch.Generator().manual_seed(0)
    x = {n: torch.randn((4, w.B, w.H, w.N, w.d), generator=g) for n in "QKVG"}
    r = bench.cpu_baseline(w, x, rows_sampled=64, lin_heads=2)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "64 of 300" in r["sample"] and "2 of 3 heads" in r["sample"]
    # more rows than the sequence: every row, once
    r = bench.cpu_baseline(w, x, rows_sampled=10_000, lin_heads=9)
    assert "300 of 300" in r["sample"] and "3 of 3 heads" in r["sample"]
