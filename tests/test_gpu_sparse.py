"""Block-sparse anchor parity: the kernel against the float64 oracle's
block-sparse softmax on the same seeded inputs and patterns -- unstructured
patterns with empty query blocks, out-of-range indices and unsorted lists,
LVSA-structured frame patterns, the full pattern (bitwise equal to the dense
anchor), and sampled rows of the 720p / 60 s workload with its LVSA pattern."""
import dataclasses
import time

import numpy as np
import pytest
import torch

import hybrid_linear_softmax_amd as ha
import oracle
from gpu_util import TOL, rel_err, sample_rows, say
from workloads import get, layer_inputs_device, layer_inputs_host, to_f64
from workloads.sparsity import full_pattern, lvsa_pattern, pattern_density, random_pattern

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
VARIANTS = [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)]


def _inputs(dtype, d, B, H, N):
    base = get("tiny") if dtype == "f32" else get("480p")
    return layer_inputs_host(dataclasses.replace(base, d=d), 3, B=B, H=H, N=N, device=DEV)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _run(x, offsets, indices):
    out = ha.hybrid_attn_softmax_blocksparse(x["Q"], x["K"], x["V"], x["G"], _dev(offsets), _dev(indices))
    torch.cuda.synchronize()
    return out


def _check_full(x, out, offsets, indices, tol, label):
    B, H = x["Q"].shape[:2]
    got = to_f64(out)
    assert np.all(np.isfinite(got)), label
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ref = oracle.softmax_attention_blocksparse(*(to_f64(x[k][b, h]) for k in "QKVG"), offsets, indices)
            e = rel_err(got[b, h], ref)
            worst = max(worst, e)
            assert e < tol, f"{label} b={b} h={h}: {e:.3e}"
            # a query block with no valid key block is exactly zero
            nqb = len(offsets) - 1
            for qb in range(nqb):
                if oracle.allowed_keys(x["Q"].shape[2], offsets, indices, qb).size == 0:
                    assert not np.any(got[b, h, qb * 256:(qb + 1) * 256]), (label, b, h, qb)
    say(f"  {label}: worst max rel err {worst:.2e}")


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("N", [65, 1000, 4099])
def test_random_pattern_parity(dtype, d, N):
    B, H = (2, 3) if N <= 1000 else (1, 2)
    offsets, indices = random_pattern(N, keep=0.35, seed=N + d, empty_every=3, invalid=2, shuffle=True)
    say(f"blocksparse random {dtype} d={d} B={B} H={H} N={N} nnz={indices.size}")
    x = _inputs(dtype, d, B, H, N)
    out = _run(x, offsets, indices)
    _check_full(x, out, offsets, indices, TOL[dtype], f"random {dtype} d={d} N={N}")


@pytest.mark.parametrize("dtype,d", VARIANTS)
def test_lvsa_pattern_parity(dtype, d):
    frames, tpf = 9, 300                      # N = 2700: ragged query and key tails
    offsets, indices = lvsa_pattern(frames, tpf, C=5, T_per=3, step=1)
    N = frames * tpf
    say(f"blocksparse lvsa {dtype} d={d} N={N} density={pattern_density(offsets, N):.3f}")
    x = _inputs(dtype, d, 1, 2, N)
    out = _run(x, offsets, indices)
    _check_full(x, out, offsets, indices, TOL[dtype], f"lvsa {dtype} d={d}")


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("N", [1, 63, 1000, 4099])
def test_full_pattern_equals_dense_bitwise(dtype, d, N):
    say(f"blocksparse full pattern vs dense {dtype} d={d} N={N}")
    x = _inputs(dtype, d, 1, 2, N)
    offsets, indices = full_pattern(N)
    sparse = _run(x, offsets, indices)
    dense = ha.hybrid_attn_softmax(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    assert torch.equal(sparse, dense)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_order_and_invalid_indices(dtype, d):
    N = 3000
    say(f"blocksparse order / invalid indices {dtype} d={d} N={N}")
    x = _inputs(dtype, d, 1, 2, N)
    offsets, indices = random_pattern(N, keep=0.5, seed=7)
    base = _run(x, offsets, indices)
    shuffled = _run(x, *random_pattern(N, keep=0.5, seed=7, shuffle=True))
    with_bad = _run(x, *random_pattern(N, keep=0.5, seed=7, invalid=5))
    # the listed order changes only the summation order
    assert rel_err(to_f64(shuffled), to_f64(base)) < TOL[dtype]
    # out-of-range indices name no key: bitwise the same as leaving them out
    assert torch.equal(with_bad, base)


def test_empty_pattern_writes_zero():
    N = 700
    say(f"blocksparse empty pattern bf16 N={N}")
    x = _inputs("bf16", 128, 1, 2, N)
    nqb = -(-N // 256)
    out = _run(x, np.zeros(nqb + 1, np.int32), np.zeros(0, np.int32))
    assert not torch.any(out)
    # only out-of-range blocks listed: also empty
    offsets = np.arange(nqb + 1, dtype=np.int32)
    out = _run(x, offsets, np.full(nqb, 10 ** 6, np.int32))
    assert not torch.any(out)


def test_720p60s_lvsa_sampled():
    w = get("720p60s")
    offsets, indices = lvsa_pattern(w.frames, w.grid[0] * w.grid[1])
    assert len(offsets) - 1 == -(-w.N // 256)
    say(f"blocksparse 720p60s: B={w.B} H={w.H} N={w.N} nnz={indices.size} "
        f"density={pattern_density(offsets, w.N):.4f}: generating inputs")
    x = layer_inputs_device(w, 3, DEV)
    off_d, idx_d = _dev(offsets), _dev(indices)
    say("blocksparse 720p60s: running")
    out = ha.hybrid_attn_softmax_blocksparse(x["Q"], x["K"], x["V"], x["G"], off_d, idx_d)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ha.hybrid_attn_softmax_blocksparse(x["Q"], x["K"], x["V"], x["G"], off_d, idx_d, O=out)
    torch.cuda.synchronize()
    say(f"  720p60s block-sparse anchor: {1e3 * (time.perf_counter() - t0):.1f} ms")
    assert torch.isfinite(out).all()
    rows = sample_rows(w.N, n_rand=96, seed=5)
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        q, k, v, g = (to_f64(x[t][b, h]) for t in "QKVG")
        ref = oracle.softmax_attention_blocksparse(q, k, v, g, offsets, indices, rows=rows)
        e = rel_err(to_f64(out[b, h])[rows], ref)
        say(f"  720p60s lvsa b={b} h={h} rows {rows.size}: max rel err {e:.2e}")
        assert e < TOL[w.dtype]
    del x, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_leading_invalid_blocks_then_growing_logits(dtype, d):
    """Every list starts with entries that name no key (so the running maximum
    is still -inf when the first valid keys arrive), then valid blocks whose
    logits grow along the sequence, so that a later block raises the maximum
    and rescales what the first valid blocks contributed."""
    N = 1100
    x = _inputs(dtype, d, 1, 2, N)
    f = 1.0 if dtype == "f32" else d ** 0.5
    ramp = torch.linspace(0.5, 4.0, N, device=DEV)[None, None, :, None]
    x["Q"] = (x["Q"].float() * f).to(x["Q"].dtype)
    x["K"] = (x["K"].float() * f * ramp).to(x["K"].dtype)
    nqb, nkb = -(-N // 256), -(-N // 64)
    lists = [[-1, nkb + 5] + list(range(nkb)) for _ in range(nqb)]
    offsets = np.cumsum([0] + [len(l) for l in lists]).astype(np.int32)
    indices = np.asarray([b for l in lists for b in l], dtype=np.int32)
    say(f"sparse leading invalid blocks {dtype} d={d}")
    out = _run(x, offsets, indices)
    _check_full(x, out, offsets, indices, TOL[dtype], f"leading-invalid {dtype} d={d}")
    # the same sets without the invalid entries: the same output up to rounding
    off2 = np.arange(nqb + 1, dtype=np.int32) * nkb
    idx2 = np.tile(np.arange(nkb, dtype=np.int32), nqb)
    ref_out = _run(x, off2, idx2)
    assert rel_err(to_f64(out), to_f64(ref_out)) < TOL[dtype]
