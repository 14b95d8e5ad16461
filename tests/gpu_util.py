"""Helpers shared by the GPU parity tests: tolerance metric, oracle on sampled
heads/rows, and a print that names the case before each GPU step."""
import numpy as np

import oracle
from workloads import to_f64

# Tolerances of the method's checks: max relative error 2e-2 for bfloat16 I/O,
# 1e-4 for float32, measured as max|gpu - ref| / max|ref| over one layer's output.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


def elem_err(got, ref, floor=1e-2):
    """Diagnostic: elementwise |d|/|ref| over elements with |ref| >= floor*max|ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mask = np.abs(ref) >= floor * np.abs(ref).max()
    r = np.abs(got - ref)[mask] / np.abs(ref)[mask]
    return float(r.max()), float(np.quantile(r, 0.999))


def say(*a):
    print(*a, flush=True)


def sample_rows(N, n_rand=512, seed=0, extra=()):
    """First 64 rows, the last (ragged) tile, seeded random rows and extras."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(64, N))) | set(range(max(0, N - 80), N))
    rows |= set(rng.choice(N, size=min(n_rand, N), replace=False).tolist())
    rows |= {int(r) for r in extra if 0 <= r < N}
    return np.array(sorted(rows), dtype=np.int64)


def _f64_dev(t):
    """Exact widening to float64 done on the device, then copied back (faster
    than widening large bfloat16 slabs on the host)."""
    import torch

    return t.detach().to(torch.float64).cpu().numpy()


def _oracle_rows(kind, q_rows, k, v, g_rows):
    """Oracle output of the given query rows of one head (rows are independent:
    the linear layer's rows need only that head's full S and z, the anchor's
    rows only all of that head's keys)."""
    if kind == "linear":
        return oracle.linear_attention(q_rows, k, v, g_rows)
    return oracle.softmax_attention(q_rows, k, v, g_rows)


def check_layer_sampled(kind, Q, K, V, G, O, heads, rows, tol, label, elem_bound=None):
    """Compare a [B, H, N, d] device output with the oracle on selected (b, h)
    heads and query rows; inputs are copied back exactly (widened to float64).
    Besides the max relative error (the tolerance metric) it reports the
    elementwise diagnostic (max and 99.9th percentile of |d|/|ref| over elements
    with |ref| >= 1e-2 max|ref|) and, when elem_bound = (max, p999) is given,
    checks it."""
    worst, worst_el = 0.0, (0.0, 0.0)
    idx = __import__("torch").as_tensor(rows, device=O.device)
    for (b, h) in heads:
        k, v = _f64_dev(K[b, h]), _f64_dev(V[b, h])
        q, g = _f64_dev(Q[b, h].index_select(0, idx)), _f64_dev(G[b, h].index_select(0, idx))
        got = _f64_dev(O[b, h].index_select(0, idx))
        ref = _oracle_rows(kind, q, k, v, g)
        assert np.all(np.isfinite(got)), (label, b, h)
        e = rel_err(got, ref)
        el = elem_err(got, ref)
        worst = max(worst, e)
        worst_el = (max(worst_el[0], el[0]), max(worst_el[1], el[1]))
        assert e < tol, f"{label} {kind} b={b} h={h}: max rel err {e:.3e} >= {tol}"
        if elem_bound is not None:
            assert el[0] < elem_bound[0] and el[1] < elem_bound[1], \
                f"{label} {kind} b={b} h={h}: elementwise err max {el[0]:.3e} p99.9 {el[1]:.3e} vs {elem_bound}"
    say(f"  {label} {kind}: heads {heads if len(heads) <= 4 else f'{len(heads)} (all)'} rows {rows.size}: "
        f"worst max rel err {worst:.2e}; elementwise max {worst_el[0]:.2e} p99.9 {worst_el[1]:.2e}")
    return worst, worst_el


def small_row_sample(N, seed, n_rand=32, tail=16):
    """A small per-head sample: seeded random rows plus the last `tail` rows
    (the ragged final tile of every kernel)."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(n_rand, N), replace=False).tolist()) | set(range(max(0, N - tail), N))
    return np.array(sorted(rows), dtype=np.int64)
