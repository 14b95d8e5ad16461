"""Degenerate cases, invariances and determinism of the HIP path."""
import dataclasses

import numpy as np
import pytest
import torch

import hybrid_linear_softmax_amd as ha
import oracle
from gpu_util import TOL, rel_err, say
from workloads import get, layer_inputs_host, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
VARIANTS = [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)]


def _inputs(dtype, d, B=1, H=2, N=1000, layer=0, name=None):
    base = get(name) if name else (get("tiny") if dtype == "f32" else get("480p"))
    return layer_inputs_host(dataclasses.replace(base, d=d), layer, B=B, H=H, N=N, device=DEV)


def _run(kind, x, **kw):
    fn = ha.hybrid_attn_linear if kind == "linear" else ha.hybrid_attn_softmax
    out = fn(x["Q"], x["K"], x["V"], x["G"], **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("kind", ["linear", "softmax"])
def test_gate_limits(kind, dtype, d):
    x = _inputs(dtype, d, N=777)
    say(f"gate limits {kind} {dtype} d={d}")
    closed = dict(x, G=torch.full_like(x["G"], -float("inf")))
    out = _run(kind, closed)
    assert torch.all(out == 0), "G = -inf must give exactly 0"
    opened = dict(x, G=torch.full_like(x["G"], float("inf")))
    got = to_f64(_run(kind, opened))
    ref = oracle.layer(kind, *(to_f64(opened[k]) for k in "QKVG"))
    assert np.all(np.isfinite(got)) and rel_err(got, ref) < TOL[dtype]


@pytest.mark.parametrize("dtype,d", VARIANTS)
def test_softmax_weights_sum_to_one(dtype, d):
    x = _inputs(dtype, d, N=1500)
    say(f"softmax V=1 {dtype} d={d}")
    x["V"] = torch.ones_like(x["V"])
    got = to_f64(_run("softmax", x))
    ref = 1.0 / (1.0 + np.exp(-to_f64(x["G"])))
    # only the output rounding (and the fp32 sum) separates O from sigmoid(G)
    assert rel_err(got, ref) < (2.0 ** -7 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("dtype,d", VARIANTS)
def test_softmax_key_shift_invariance(dtype, d):
    """Adding one vector to every key adds q.c to a whole row of logits: the
    output must not change.  Large shifts exercise the running-max rescale."""
    x = _inputs(dtype, d, N=2000, layer=3)
    say(f"softmax key shift {dtype} d={d}")
    base = to_f64(_run("softmax", x))
    c = torch.linspace(-2.0, 2.0, d, device=DEV, dtype=torch.float32)
    shifted = dict(x, K=(x["K"].float() + c).to(x["K"].dtype))
    got = to_f64(_run("softmax", shifted))
    ref = oracle.layer("softmax", *(to_f64(shifted[k]) for k in "QKVG"))
    assert rel_err(got, ref) < TOL[dtype]
    assert rel_err(base, oracle.layer("softmax", *(to_f64(x[k]) for k in "QKVG"))) < TOL[dtype]


@pytest.mark.parametrize("dtype,d", VARIANTS)
def test_softmax_peaked_logits(dtype, d):
    """Unit-variance Q and K scaled x3: logits with standard deviation ~9, so
    nearly one-hot rows and maxima that move across key blocks."""
    x = _inputs(dtype, d, N=3000, layer=3)
    f = 3.0 if dtype == "f32" else 3.0 * d ** 0.5     # q, k ~ N(0, 9) in both cases
    x["Q"] = (x["Q"].float() * f).to(x["Q"].dtype)
    x["K"] = (x["K"].float() * f).to(x["K"].dtype)
    say(f"softmax peaked {dtype} d={d}")
    got = to_f64(_run("softmax", x))
    ref = oracle.layer("softmax", *(to_f64(x[k]) for k in "QKVG"))
    assert np.all(np.isfinite(got)) and rel_err(got, ref) < TOL[dtype]


@pytest.mark.parametrize("dtype,d", VARIANTS)
def test_linear_power_of_two_scaling_is_exact(dtype, d):
    """phi(2^k q) = 2^k phi(q) and S, z scale exactly with K: numerator and
    denominator scale by the same power of two, eps sits below one ulp of the
    denominator here, so the output is bitwise unchanged."""
    x = _inputs(dtype, d, N=4096)
    say(f"linear 2^k scaling {dtype} d={d}")
    base = _run("linear", x)
    for key, f in (("Q", 2.0), ("Q", 4.0), ("K", 2.0)):
        y = dict(x, **{key: x[key] * f})
        assert torch.equal(_run("linear", y), base), (key, f)


@pytest.mark.parametrize("dtype,d", VARIANTS)
def test_linear_zero_features(dtype, d):
    x = _inputs(dtype, d, N=513)
    say(f"linear zero features {dtype} d={d}")
    x["Q"][0, 0, 7] = -x["Q"][0, 0, 7].abs()        # phi(q) = 0 for one query
    x["Q"][0, 1, 512] = 0
    out = _run("linear", x)
    assert torch.all(out[0, 0, 7] == 0) and torch.all(out[0, 1, 512] == 0)
    assert torch.isfinite(out).all()
    neg = dict(x, K=-x["K"].abs())                  # phi(K) = 0 everywhere
    assert torch.all(_run("linear", neg) == 0)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_empty_sequence(dtype, d):
    say(f"empty sequence {dtype} d={d}")
    x = _inputs(dtype, d, B=2, H=3, N=0)
    for kind in ("linear", "softmax"):
        out = _run(kind, x)
        assert out.shape == (2, 3, 0, d)
    S = torch.full((2, 3, d, d), 7.0, device=DEV)
    z = torch.full((2, 3, d), 7.0, device=DEV)
    ha.hybrid_attn_kv_state(x["K"], x["V"], S, z)
    torch.cuda.synchronize()
    assert torch.all(S == 0) and torch.all(z == 0)


def _group_inputs(dtype, d, B, H, N, name=None):
    layers = [_inputs(dtype, d, B, H, N, layer=l, name=name) for l in range(4)]
    return {k: torch.stack([L[k] for L in layers]).contiguous() for k in "QKVG"}, layers


@pytest.mark.parametrize("dtype,d", VARIANTS)
def test_group_equals_layers_and_is_deterministic(dtype, d):
    x, layers = _group_inputs(dtype, d, 2, 2, 1031)
    say(f"group vs layers {dtype} d={d}")
    o1 = ha.hybrid_attn_group(x["Q"], x["K"], x["V"], x["G"])
    o2 = ha.hybrid_attn_group(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "two runs on the same inputs must be bitwise equal"
    for l, kind in enumerate(ha.hybrid_attn_group_schedule()):
        single = _run(kind, layers[l])
        assert torch.equal(o1[l], single), ("group layer", l, kind)
    ref = oracle.group(*(to_f64(x[k]) for k in "QKVG"))
    for l in range(4):
        assert rel_err(to_f64(o1[l]), ref[l]) < TOL[dtype]


def test_group_timed_events():
    x, _ = _group_inputs("bf16", 128, 1, 2, 2048)
    say("group timed events")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    o1 = ha.hybrid_attn_group(x["Q"], x["K"], x["V"], x["G"], events=evs)
    o2 = ha.hybrid_attn_group(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    times = [evs[i].elapsed_time(evs[i + 1]) for i in range(4)]
    assert all(t >= 0 for t in times), times


def test_linear_timed_events():
    x = _inputs("bf16", 128, N=5000)
    say("linear timed events")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    o1 = ha.hybrid_attn_linear(x["Q"], x["K"], x["V"], x["G"], events=evs)
    o2 = ha.hybrid_attn_linear(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    times = [evs[i].elapsed_time(evs[i + 1]) for i in range(3)]
    assert all(t >= 0 for t in times), times


def test_workspace_too_small_raises():
    x = _inputs("bf16", 128, N=100)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ha.HybridAttnError):
        ha.hybrid_attn_linear(x["Q"], x["K"], x["V"], x["G"], workspace=ws)


def test_heavy_tailed_rows():
    """720p/60s value distribution (5 % of K/V rows x4) at a reduced length."""
    w = get("720p60s")
    say("heavy-tailed rows bf16 d=128 N=8192")
    x = layer_inputs_host(w, 0, B=1, H=2, N=8192, device=DEV)
    for kind in ("linear", "softmax"):
        got = to_f64(_run(kind, x))
        ref = oracle.layer(kind, *(to_f64(x[k]) for k in "QKVG"))
        err = rel_err(got, ref)
        say(f"  {kind}: {err:.2e}")
        assert err < TOL["bf16"]


@pytest.mark.parametrize("dtype,d", VARIANTS)
def test_softmax_growing_logits_rescale(dtype, d):
    """Keys whose norm grows along the sequence: each row's maximum keeps
    rising from one key block to the next, so the running maximum is raised
    (and the output rescaled) many times.  Output and log-sum-exp against the
    oracle."""
    x = _inputs(dtype, d, N=4099, layer=3)
    f = 1.0 if dtype == "f32" else d ** 0.5          # unit-variance q, k in both cases
    ramp = torch.linspace(0.25, 4.0, x["K"].shape[2], device=DEV)[None, None, :, None]
    x["Q"] = (x["Q"].float() * f).to(x["Q"].dtype)
    x["K"] = (x["K"].float() * f * ramp).to(x["K"].dtype)
    say(f"softmax growing logits {dtype} d={d}")
    O, lse = ha.hybrid_attn_softmax_lse(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    got = to_f64(O)
    ref = oracle.layer("softmax", *(to_f64(x[k]) for k in "QKVG"))
    assert np.all(np.isfinite(got)) and rel_err(got, ref) < TOL[dtype]
    for h in range(x["Q"].shape[1]):
        lref = oracle.softmax_lse(to_f64(x["Q"][0, h]), to_f64(x["K"][0, h]))
        err = np.abs(lse[0, h].cpu().numpy().astype(np.float64) - lref).max()
        assert err < (5e-3 if dtype == "bf16" else 1e-5), err
    # the plain entry point gives the same output
    assert torch.equal(_run("softmax", x), O)
