"""The five workloads at their full sizes, run as one hybrid group in the same
launch configuration the bench times, checked against the oracle on sampled
heads and query rows (rows are independent, so a sampled row is an exact check)."""
import numpy as np
import pytest
import torch

import hybrid_linear_softmax_amd as ha
import oracle
from gpu_util import TOL, check_layer_sampled, rel_err, sample_rows, say, small_row_sample
from workloads import CONFIGS, get, group_inputs_device, heavy_token_positions, layer_inputs_host, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_tiny_group_full():
    w = get("tiny")
    say("config tiny: full group vs oracle")
    layers = [layer_inputs_host(w, l, device="cuda") for l in range(4)]
    x = {k: torch.stack([L[k] for L in layers]).contiguous() for k in "QKVG"}
    out = ha.hybrid_attn_group(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    ref = oracle.group(*(to_f64(x[k]) for k in "QKVG"))
    got = to_f64(out)
    for l in range(4):
        err = rel_err(got[l], ref[l])
        say(f"  layer {l} ({oracle.SCHEDULE[l]}): {err:.2e}")
        assert err < TOL["f32"]


# Elementwise bounds (max, 99.9th percentile of |got - ref| / |ref| over
# elements with |ref| >= 1e-2 max |ref|), about three times what the full-size
# runs measure: the linear layer's elements carry the bf16 rounding of the
# output (measured max 3.9e-3); the softmax's small elements also carry the
# bf16 rounding of each probability summed over ~N keys (measured max
# 0.09-0.16, p99.9 0.03-0.07).  An indexing or masking mistake gives O(1).
ELEM_BOUND = {"linear": (1.2e-2, 1.2e-2), "softmax": (0.5, 0.2)}


@pytest.mark.parametrize("name", [n for n in CONFIGS if n != "tiny"])
def test_config_group_sampled(name):
    w = get(name)
    say(f"config {name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}: generating inputs")
    x = group_inputs_device(w, "cuda")
    ws = torch.empty(ha.workspace_bytes(w.B, w.H, w.N, w.d, torch.bfloat16), dtype=torch.uint8, device="cuda")
    say(f"config {name}: running group")
    out = ha.hybrid_attn_group(x["Q"], x["K"], x["V"], x["G"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    others = [(b, h) for b in range(w.B) for h in range(w.H) if (b, h) not in heads]
    for l, kind in enumerate(oracle.SCHEDULE):
        heavy = heavy_token_positions(w, l)[:256]
        rows = sample_rows(w.N, n_rand=512 if kind == "softmax" else 4096, seed=l, extra=heavy)
        args = (x["Q"][l], x["K"][l], x["V"][l], x["G"][l], out[l])
        bound = ELEM_BOUND[kind] if w.dtype == "bf16" else None
        check_layer_sampled(kind, *args, heads, rows, TOL[w.dtype], f"{name} layer {l}", elem_bound=bound)
        # every other (b, h) on a small seeded sample (a head-indexing or block
        # remap error confined to middle heads would show here)
        check_layer_sampled(kind, *args, others, small_row_sample(w.N, seed=100 + l), TOL[w.dtype],
                            f"{name} layer {l} (all heads)", elem_bound=bound)
    del x, out, ws
    torch.cuda.empty_cache()
