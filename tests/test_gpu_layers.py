"""Kernel parity: every layer kind, both dtypes and head sizes, against the
float64 oracle element by element, over sizes that span several tiles and a
ragged tail."""
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


def _workload(dtype, d):
    base = get("tiny") if dtype == "f32" else get("480p")
    return dataclasses.replace(base, d=d)


VARIANTS = [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)]
NS = [1, 15, 17, 63, 65, 129, 257, 1000, 4099]


def _inputs(dtype, d, B, H, N, layer=0):
    return layer_inputs_host(_workload(dtype, d), layer, B=B, H=H, N=N, device=DEV)


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("N", [1, 63, 65, 1000, 4099])
def test_kv_state(dtype, d, N):
    x = _inputs(dtype, d, 2, 3, N)
    say(f"kv_state {dtype} d={d} B=2 H=3 N={N}")
    S, z = ha.hybrid_attn_kv_state(x["K"], x["V"])
    torch.cuda.synchronize()
    S, z = to_f64(S), to_f64(z)
    for b in range(2):
        for h in range(3):
            Sr, zr = oracle.kv_state(to_f64(x["K"][b, h]), to_f64(x["V"][b, h]))
            assert rel_err(S[b, h], Sr) < 1e-5, (b, h, rel_err(S[b, h], Sr))
            assert rel_err(z[b, h], zr) < 1e-5, (b, h, rel_err(z[b, h], zr))


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("N", NS)
@pytest.mark.parametrize("kind", ["linear", "softmax"])
def test_layer_parity(kind, dtype, d, N):
    B, H = (2, 3) if N <= 1000 else (1, 2)
    x = _inputs(dtype, d, B, H, N, layer=0 if kind == "linear" else 3)
    say(f"{kind} {dtype} d={d} B={B} H={H} N={N}")
    fn = ha.hybrid_attn_linear if kind == "linear" else ha.hybrid_attn_softmax
    out = fn(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    got = to_f64(out)
    ref = oracle.layer(kind, *(to_f64(x[k]) for k in "QKVG"))
    assert np.all(np.isfinite(got))
    err = rel_err(got, ref)
    say(f"  max rel err {err:.2e}")
    assert err < TOL[dtype], err
