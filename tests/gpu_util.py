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


def check_layer_sampled(kind, Q, K, V, G, O, heads, rows, tol, label):
    """Compare a [B, H, N, d] device output with the oracle on selected (b, h)
    heads and query rows; inputs are copied back exactly (widened to float64)."""
    worst = 0.0
    for (b, h) in heads:
        q, k, v, g = (to_f64(x[b, h]) for x in (Q, K, V, G))
        got = to_f64(O[b, h])[rows]
        if kind == "linear":
            ref = oracle.linear_attention(q, k, v, g)[rows]
        else:
            ref = oracle.softmax_attention(q, k, v, g, rows=rows)
        assert np.all(np.isfinite(got)), (label, b, h)
        e = rel_err(got, ref)
        worst = max(worst, e)
        assert e < tol, f"{label} {kind} b={b} h={h}: max rel err {e:.3e} >= {tol}"
    say(f"  {label} {kind}: heads {heads} rows {rows.size}: worst max rel err {worst:.2e}")
    return worst
