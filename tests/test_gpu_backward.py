"""Backward-pass parity: the gradient kernels against the float64 backward
oracle (which is pinned by finite differences, library autograd and
invariances) on the same seeded inputs and upstream gradients."""
import dataclasses

import numpy as np
import pytest
import torch

import hybrid_linear_softmax_amd as ha
import oracle
from gpu_util import TOL, elem_err, rel_err, say
from workloads import get, layer_inputs_device, layer_inputs_host, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
VARIANTS = [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)]


def _inputs(dtype, d, B, H, N, layer=0):
    base = get("tiny") if dtype == "f32" else get("480p")
    w = dataclasses.replace(base, d=d)
    x = layer_inputs_host(w, layer, B=B, H=H, N=N, device=DEV)
    gen = torch.Generator(device="cpu").manual_seed(1000 + N + d)
    x["dO"] = torch.randn((B, H, N, d), generator=gen).to(x["Q"].dtype).to(DEV)
    return x


def _linear_term_scales(Q, K, V, G, dO, eps=1e-6):
    """Sizes of the terms whose difference makes dQ and dK of the linear layer
    (for one head): dQ = (dn S^T + dden z) [q > 0] and dK = (v dS^T + dz) [k > 0]
    are each a difference of two terms of comparable size -- exactly zero at
    N = 1, where the layer is invariant to scaling q or k -- so their rounding
    error is measured against |dn| |S|^T + |dden| |z| and |v| |dS|^T + |dz|,
    with |dS| and |dz| the sums of the absolute terms."""
    fq, fk = np.maximum(Q, 0), np.maximum(K, 0)
    S, z = fk.T @ V, fk.sum(axis=0)
    den = fq @ z + eps
    a = (fq @ S) / den[:, None]
    s = 1.0 / (1.0 + np.exp(-G))
    da = dO * s
    dn = da / den[:, None]
    dden = -(da * a).sum(axis=1) / den
    dS_abs, dz_abs = fq.T @ np.abs(dn), fq.T @ np.abs(dden)
    sq = (np.abs(dn) @ np.abs(S).T + np.abs(dden)[:, None] * np.abs(z)[None, :]) * (Q > 0)
    sk = (np.abs(V) @ dS_abs.T + dz_abs[None, :]) * (K > 0)
    return sq, sk


def _check(got, ref, tol, label, scales=(None, None, None, None)):
    worst = 0.0
    diag = []
    for name, g, r, sc in zip(("dQ", "dK", "dV", "dG"), got, ref, scales):
        g = to_f64(g)
        assert np.all(np.isfinite(g)), (label, name)
        e = rel_err(g, r) if sc is None else float(np.abs(g - r).max() / max(np.abs(sc).max(), 1e-300))
        worst = max(worst, e)
        assert e < tol, f"{label} {name}: max rel err {e:.3e} >= {tol}"
        if np.abs(r).max() > 0:
            em, e999 = elem_err(g, r)
            diag.append(f"{name} {em:.1e}/{e999:.1e}")
    # elementwise |d|/|ref| (max / 99.9th percentile over |ref| >= 1e-2 max|ref|), reported only
    say(f"  {label}: worst max rel err {worst:.2e}; elementwise {', '.join(diag)}")


def _linear_scales_bhnd(Q, K, V, G, dO):
    sq, sk = (np.empty_like(Q) for _ in range(2))
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            sq[b, h], sk[b, h] = _linear_term_scales(Q[b, h], K[b, h], V[b, h], G[b, h], dO[b, h])
    return sq, sk, None, None


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("N", [1, 63, 65, 1000, 4099])
def test_linear_backward_parity(dtype, d, N):
    B, H = (2, 3) if N <= 1000 else (1, 2)
    say(f"linear backward {dtype} d={d} B={B} H={H} N={N}")
    x = _inputs(dtype, d, B, H, N)
    got = ha.hybrid_attn_linear_backward(x["Q"], x["K"], x["V"], x["G"], x["dO"])
    torch.cuda.synchronize()
    inp = [to_f64(x[k]) for k in ("Q", "K", "V", "G", "dO")]
    ref = oracle.layer_backward("linear", *inp)
    _check(got, ref, TOL[dtype], f"linear bwd {dtype} d={d} N={N}", _linear_scales_bhnd(*inp))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_linear_backward_deterministic_and_zero(dtype, d):
    say(f"linear backward determinism {dtype} d={d}")
    x = _inputs(dtype, d, 1, 2, 3000)
    a = ha.hybrid_attn_linear_backward(x["Q"], x["K"], x["V"], x["G"], x["dO"])
    b = ha.hybrid_attn_linear_backward(x["Q"], x["K"], x["V"], x["G"], x["dO"])
    z = ha.hybrid_attn_linear_backward(x["Q"], x["K"], x["V"], x["G"], torch.zeros_like(x["dO"]))
    torch.cuda.synchronize()
    assert all(torch.equal(u, v) for u, v in zip(a, b))
    assert all(not torch.any(t) for t in z)


def test_linear_backward_720p5s_heads():
    w = get("720p5s")
    say(f"linear backward 720p5s B={w.B} H={w.H} N={w.N}: generating inputs")
    x = layer_inputs_device(w, 0, DEV)
    gen = torch.Generator(device=DEV).manual_seed(77)
    x["dO"] = torch.randn((w.B, w.H, w.N, w.d), generator=gen, device=DEV).to(x["Q"].dtype)
    got = ha.hybrid_attn_linear_backward(x["Q"], x["K"], x["V"], x["G"], x["dO"])
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        inp = [to_f64(x[k][b, h]) for k in ("Q", "K", "V", "G", "dO")]
        ref = oracle.linear_attention_backward(*inp)
        _check([g[b, h] for g in got], ref, TOL["bf16"], f"720p5s linear bwd head ({b},{h})",
               (*_linear_term_scales(*inp), None, None))
    del x, got
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- anchor


def _softmax_inputs(dtype, d, B, H, N):
    x = _inputs(dtype, d, B, H, N, layer=3)
    return x


def _softmax_term_scales(Q, K, V, G, dO):
    """Sizes of the terms behind dQ and dK of the anchor (one head, full N x N):
    dS = P (dP - D) is a difference of comparable terms -- exactly zero at N = 1,
    where P = 1 and dP = D -- so the dQ = dS K / sqrt(d) and dK = dS^T Q / sqrt(d)
    errors are measured against P (|dP| + |D|) |K| / sqrt(d) and its transpose."""
    d = Q.shape[1]
    L = Q @ K.T / np.sqrt(d)
    P = np.exp(L - L.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    s = 1.0 / (1.0 + np.exp(-G))
    da = dO * s
    a = P @ V
    D = (da * a).sum(axis=1)
    T = P * (np.abs(da @ V.T) + np.abs(D)[:, None])
    return T @ np.abs(K) / np.sqrt(d), T.T @ np.abs(Q) / np.sqrt(d)


def _softmax_scales_bhnd(Q, K, V, G, dO):
    sq, sk = (np.empty_like(Q) for _ in range(2))
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            sq[b, h], sk[b, h] = _softmax_term_scales(Q[b, h], K[b, h], V[b, h], G[b, h], dO[b, h])
    return sq, sk, None, None


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("N", [1, 63, 200, 1000, 2051])
def test_softmax_lse_forward(dtype, d, N):
    B, H = (1, 2)
    say(f"softmax lse {dtype} d={d} N={N}")
    x = _softmax_inputs(dtype, d, B, H, N)
    O, lse = ha.hybrid_attn_softmax_lse(x["Q"], x["K"], x["V"], x["G"])
    O2 = ha.hybrid_attn_softmax(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    assert torch.equal(O, O2)                     # the same kernel, one more output
    for h in range(H):
        ref = oracle.softmax_lse(to_f64(x["Q"][0, h]), to_f64(x["K"][0, h]))
        err = np.abs(lse[0, h].cpu().numpy().astype(np.float64) - ref).max()
        assert err < (5e-3 if dtype == "bf16" else 1e-5), err


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("N", [1, 63, 200, 1000, 2051])
def test_softmax_backward_parity(dtype, d, N):
    B, H = (2, 2) if N <= 1000 else (1, 2)
    say(f"softmax backward {dtype} d={d} B={B} H={H} N={N}")
    x = _softmax_inputs(dtype, d, B, H, N)
    O, lse = ha.hybrid_attn_softmax_lse(x["Q"], x["K"], x["V"], x["G"])
    got = ha.hybrid_attn_softmax_backward(x["Q"], x["K"], x["V"], x["G"], O, x["dO"], lse)
    torch.cuda.synchronize()
    inp = [to_f64(x[k]) for k in ("Q", "K", "V", "G", "dO")]
    ref = oracle.layer_backward("softmax", *inp)
    _check(got, ref, TOL[dtype], f"softmax bwd {dtype} d={d} N={N}", _softmax_scales_bhnd(*inp))


def test_softmax_backward_deterministic():
    x = _softmax_inputs("bf16", 128, 1, 2, 3000)
    O, lse = ha.hybrid_attn_softmax_lse(x["Q"], x["K"], x["V"], x["G"])
    a = ha.hybrid_attn_softmax_backward(x["Q"], x["K"], x["V"], x["G"], O, x["dO"], lse)
    b = ha.hybrid_attn_softmax_backward(x["Q"], x["K"], x["V"], x["G"], O, x["dO"], lse)
    torch.cuda.synchronize()
    assert all(torch.equal(u, v) for u, v in zip(a, b))


def test_softmax_backward_keys_at_12k():
    """dK, dV for sampled keys against the oracle's key-sampled form (which
    normalises every query over all keys) at N = 12,000."""
    N = 12000
    say(f"softmax backward sampled keys bf16 N={N}")
    x = _softmax_inputs("bf16", 128, 1, 1, N)
    O, lse = ha.hybrid_attn_softmax_lse(x["Q"], x["K"], x["V"], x["G"])
    dQ, dK, dV, dG = ha.hybrid_attn_softmax_backward(x["Q"], x["K"], x["V"], x["G"], O, x["dO"], lse)
    torch.cuda.synchronize()
    keys = np.unique(np.concatenate([np.arange(64), np.arange(N - 70, N),
                                     np.random.default_rng(4).choice(N, 256, replace=False)]))
    inp = [to_f64(x[k][0, 0]) for k in ("Q", "K", "V", "G", "dO")]
    rk, rv = oracle.softmax_attention_backward_keys(*inp, keys)
    assert rel_err(to_f64(dK[0, 0])[keys], rk) < TOL["bf16"]
    assert rel_err(to_f64(dV[0, 0])[keys], rv) < TOL["bf16"]


def test_softmax_backward_720p5s_sampled():
    w = get("720p5s")
    say(f"softmax backward 720p5s B={w.B} H={w.H} N={w.N}: generating inputs")
    x = layer_inputs_device(w, 3, DEV)
    gen = torch.Generator(device=DEV).manual_seed(91)
    x["dO"] = torch.randn((w.B, w.H, w.N, w.d), generator=gen, device=DEV).to(x["Q"].dtype)
    O, lse = ha.hybrid_attn_softmax_lse(x["Q"], x["K"], x["V"], x["G"])
    dQ, dK, dV, dG = ha.hybrid_attn_softmax_backward(x["Q"], x["K"], x["V"], x["G"], O, x["dO"], lse)
    torch.cuda.synchronize()
    for t in (dQ, dK, dV, dG):
        assert torch.isfinite(t).all()
    rows = np.unique(np.concatenate([np.arange(64), np.arange(w.N - 80, w.N),
                                     np.random.default_rng(6).choice(w.N, 192, replace=False)]))
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        inp = [to_f64(x[k][b, h]) for k in ("Q", "K", "V", "G", "dO")]
        rq, rg = oracle.softmax_attention_backward_rows(*inp, rows)
        gq, gg = to_f64(dQ[b, h])[rows], to_f64(dG[b, h])[rows]
        eq, eg = rel_err(gq, rq), rel_err(gg, rg)
        say(f"  720p5s head ({b},{h}) rows {rows.size}: dQ {eq:.2e} dG {eg:.2e}; elementwise max/p99.9 "
            f"dQ {'/'.join(f'{v:.1e}' for v in elem_err(gq, rq))} dG {'/'.join(f'{v:.1e}' for v in elem_err(gg, rg))}")
        assert eq < TOL["bf16"] and eg < TOL["bf16"]
        # a common shift of every key leaves the anchor unchanged: the key
        # gradients of a head sum to zero (relative to their total size)
        dk = to_f64(dK[b, h])
        assert np.abs(dk.sum(axis=0)).max() < 2e-2 * np.abs(dk).sum(axis=0).max()
    del x, O, lse, dQ, dK, dV, dG
    torch.cuda.empty_cache()
