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


def test_telemetry_summary_and_absence():
    # (metrics timestamp, clock MHz, power W): the first sample may predate the
    # window and repeats of a timestamp are stale, so both are dropped
    s = bench.summarize_telemetry([(1, 127, 250.0), (1, 127, 250.0), (2, 2400, 900.0), (2, 2400, 900.0),
                                   (3, 2300, None), (4, None, 1000.0)])
    assert s["gfx_clock_mhz"] == {"median": 2350.0, "min": 2300, "max": 2400}
    assert s["socket_power_w"] == {"median": 950.0, "min": 900.0, "max": 1000.0}
    assert s["fresh_samples"] == 3
    # without timestamps (the fallback queries) every sample after the first counts
    s = bench.summarize_telemetry([(None, 10, 1.0), (None, 20, 2.0), (None, 30, 3.0)])
    assert s["gfx_clock_mhz"]["median"] == 25.0 and s["fresh_samples"] == 2
    assert bench.summarize_telemetry([]) is None
    assert bench.summarize_telemetry([(1, 2400, 900.0)]) is None
    assert bench.summarize_telemetry([(1, 2400, 900.0), (1, 2400, 900.0)]) is None
    # where amdsmi has no device (as on a host without the driver) nothing is
    # sampled and the line carries null
    t = bench.Telemetry(0, period_s=0.001)
    with t:
        pass
    if not t.available:
        assert t.summary() is None
        assert bench.sample_telemetry(lambda: None, types.SimpleNamespace(index=0), seconds=0.0) is None


def test_annotate_adds_fraction_of_achievable():
    peaks = {"mfma_bf16_tflops": 2000.0, "hbm_read_gbs": 6000.0, "hbm_copy_gbs": 5000.0,
             "hbm_copy_nontemporal_gbs": 6400.0}
    line = {"roofline": {"bound": "mfma", "achieved": 1000.0}}
    bench.annotate(line, peaks, None)
    assert line["roofline"]["achievable_peak"] == 2000.0 and line["roofline"]["frac_of_achievable"] == 0.5
    assert line["achievable"] is peaks and line["telemetry"] is None
    line = {"roofline": {"bound": "hbm", "achieved": 3200.0}}
    bench.annotate(line, peaks, {"samples": 1})
    assert line["roofline"]["achievable_peak"] == 6400.0 and line["roofline"]["frac_of_achievable"] == 0.5
    # the sustained MFMA rate, where measured, is the one a steady kernel meets
    line = {"roofline": {"bound": "mfma", "achieved": 1000.0}}
    bench.annotate(line, dict(peaks, mfma_bf16_tflops_sustained=1600.0), None)
    assert line["roofline"]["achievable_peak"] == 1600.0 and line["roofline"]["frac_of_achievable"] == 0.625
    # the MFMA loop on random operands, where measured, is reported beside it;
    # an HBM-bound line does not take it
    both = dict(peaks, mfma_bf16_tflops_sustained=1600.0, mfma_bf16_tflops_random_operands_sustained=1250.0)
    line = {"roofline": {"bound": "mfma", "achieved": 1000.0}}
    bench.annotate(line, both, None)
    assert line["roofline"]["achievable_peak"] == 1600.0
    assert line["roofline"]["achievable_peak_random_operands"] == 1250.0
    assert line["roofline"]["frac_of_achievable_random_operands"] == 0.8
    line = {"roofline": {"bound": "hbm", "achieved": 3200.0}}
    bench.annotate(line, both, None)
    assert "achievable_peak_random_operands" not in line["roofline"]
    line = {"roofline": {"bound": "mfma", "achieved": 1.0}}
    bench.annotate(line, None, None)                 # --no-peaks
    assert "achievable_peak" not in line["roofline"] and line["achievable"] is None


def test_train_and_stack_cpu_baselines_on_a_tiny_workload():
    import dataclasses

    from workloads import get
    w = dataclasses.replace(get("480p"), N=300, H=2, d=16)
    g = torch.Generator().manual_seed(1)
    x = {n: torch.randn((4, 1, w.H, w.N, w.d), generator=g) for n in "QKVG"}
    dO4 = torch.randn((4, 1, w.H, w.N, w.d), generator=g)
    r = bench.train_cpu_baseline(w, x, dO4, rows_sampled=64)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert "64 of 300 query rows" in r["sample"] and "2 of 2 heads" in r["sample"]
    C, nb = w.H * w.d, 3
    blk = {"x": torch.randn((1, w.N, C), generator=g), "W_in": torch.randn((4, 4 * C, C), generator=g),
           "W_out": torch.randn((4, C, C), generator=g)}
    summaries = torch.randn((nb, 1, w.N, C), generator=g)
    w_route = torch.randn((nb, 4, C), generator=g)
    r = bench.stack_cpu_baseline(w, nb, blk, summaries, w_route, rows_sampled=50)
    assert r["kind"] == "oracle" and r["value"] > 0
    assert "3 blocks on 50 token rows" in r["sample"]


def test_linear_kernel_split_arithmetic():
    # 720p/5s shape: R1 reads K, V (0.929 GB), R2 reads Q, G and writes O (1.393 GB)
    k = bench.linear_kernel_split(1, 24, 75600, 128, r1_ms=0.2, reduce_ms=0.015, apply_ms=0.25)
    th = 24 * 75600
    assert k["r2_apply_ms"] == 0.25 and k["r1_reduce_ms"] == 0.015
    assert abs(k["r1_hbm_gbs"] - th * 512 / 0.2e-3 / 1e9) < 0.1
    assert abs(k["r2_hbm_gbs"] - th * 768 / 0.25e-3 / 1e9) < 0.1
    assert abs(k["r1_hbm_frac"] - k["r1_hbm_gbs"] / 8000.0) < 1e-4
    assert abs(k["r1_mfma_frac"] - th * (2 * 128 * 128 + 128) / 0.2e-3 / 1e12 / 2500.0) < 1e-4
    assert abs(k["r2_mfma_frac"] - th * (2 * 128 * 128 + 6 * 128) / 0.25e-3 / 1e12 / 2500.0) < 1e-4


def test_cpu_baseline_records_the_host():
    w = types.SimpleNamespace(B=1, H=2, N=200, d=16)
    g = torch.Generator().manual_seed(1)
    x = {n: torch.randn((4, w.B, w.H, w.N, w.d), generator=g) for n in "QKVG"}
    r = bench.cpu_baseline(w, x, rows_sampled=32, lin_heads=1)
    host = r["host"]
    assert host["affinity_cores"] == len(os.sched_getaffinity(0))
    assert host["blas_threads"] == r["cores"] >= 1
    assert isinstance(host["cpu_model"], str) and host["cpu_model"]
    assert isinstance(host["blas"], str) and host["blas"]


def test_single_thread_baselines_on_small_workloads():
    from workloads import get

    tiny = get("tiny")
    lin = types.SimpleNamespace(**{**vars(get("480p")), "N": 512, "H": 6})
    r = bench.single_thread_baselines(tiny=tiny, lin=lin, lin_heads=2)
    assert r["tiny_group"]["seconds"] > 0 and r["tiny_group"]["tokens_per_s"] > 0
    assert "N=256" in r["tiny_group"]["shape"]
    assert r["linear_layer_480p"]["tokens_per_s"] > 0
    assert "2 of 6 heads" in r["linear_layer_480p"]["sample"]
    # the BLAS thread limit is lifted again afterwards
    assert bench._blas_threads() >= 1


def test_overlap_summary_fractions():
    """valu_hidden is 1 for full overlap (mixed time = the longer part), 0 for
    none (the sum) and is read per waves-per-SIMD setting; the split run is
    compared with the one-wave-per-SIMD times."""
    t = {("mfma", 1): 2.0, ("valu", 1): 1.0, ("both", 1): 2.0,      # full overlap
         ("mfma", 2): 4.0, ("valu", 2): 2.0, ("both", 2): 6.0,      # none
         ("split", 2): 2.5}                                         # half of the one-wave VALU time hidden
    s = bench.overlap_summary(t)
    assert s["waves_per_simd_1"]["valu_hidden"] == 1.0
    assert s["waves_per_simd_2"]["valu_hidden"] == 0.0
    assert s["split_valu_hidden"] == 0.5 and s["split_ms"] == 2.5
    assert s["waves_per_simd_2"]["mfma_ms"] == 4.0
