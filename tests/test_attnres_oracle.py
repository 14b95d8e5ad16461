"""The AttnRes oracle against its pins, and plausible mistakes planted in
copies of it (on the CPU), each of which must fail at least one pin."""
import types

import numpy as np
import pytest

import attnres_pins
from oracle import block_ref as R
from oracle import hybrid_ref


def _impl(mix=R.attnres_mix, route_anchor=False, stream_candidate=True, summaries_before=False):
    def block_routed(x, summaries, w_route, W_in4, W_out4, H, kinds=hybrid_ref.SCHEDULE, store=None):
        x = np.asarray(x, dtype=np.float64)
        summaries = np.asarray(summaries, dtype=np.float64).reshape((-1,) + x.shape)
        for l, kind in enumerate(kinds):
            src = x
            if kind == "linear" or route_anchor:
                cands = np.concatenate([summaries, x[None]], axis=0) if stream_candidate else summaries
                src = mix(cands, w_route[l]) if len(cands) else x
            Q, K, V, G = R.project_in(src, W_in4[l], H)
            x = R.project_out(hybrid_ref.layer(kind, Q, K, V, G), W_out4[l], x)
        return x

    def stack_routed(x, w_route, W_in, W_out, H, store=None):
        x = np.asarray(x, dtype=np.float64)
        summaries = []
        for k in range(len(W_in)):
            if summaries_before:
                summaries.append(x)
                prev = np.stack(summaries[:-1]) if k else np.zeros((0,) + x.shape)
            else:
                prev = np.stack(summaries) if summaries else np.zeros((0,) + x.shape)
            x = block_routed(x, prev, w_route[k], W_in[k], W_out[k], H)
            if not summaries_before:
                summaries.append(x)
        return x

    return types.SimpleNamespace(attnres_mix=mix, block=R.block, block_routed=block_routed,
                                 stack_routed=stack_routed)


def _mix_mut(kind):
    def mix(candidates, w, eps=R.RMS_EPS):
        V = np.asarray(candidates, dtype=np.float64)
        C = V.shape[-1]
        if kind == "std":
            norm = np.sqrt(V.var(axis=-1) + eps)
        else:
            norm = np.sqrt((V * V).mean(axis=-1) + eps)
        score = (V @ np.asarray(w, dtype=np.float64)) / norm
        if kind != "noscale":
            score = score / np.sqrt(C)
        axis = 1 if kind == "tokenaxis" else 0
        score = score - score.max(axis=axis, keepdims=True)
        a = np.exp(score)
        a /= a.sum(axis=axis, keepdims=True)
        return (a[..., None] * V).sum(axis=0)
    return mix


@pytest.mark.parametrize("pin", attnres_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_attnres_oracle_pin(pin):
    pin(R)


def test_reference_copy_passes():
    for pin in attnres_pins.ALL_PINS:
        pin(_impl())


MUTANTS = {
    "keys normalised by standard deviation": _impl(mix=_mix_mut("std")),
    "score not divided by sqrt(C)": _impl(mix=_mix_mut("noscale")),
    "softmax over tokens": _impl(mix=_mix_mut("tokenaxis")),
    "anchor also reads the mixture": _impl(route_anchor=True),
    "stream not a candidate": _impl(stream_candidate=False),
    "summaries include the current block input": _impl(summaries_before=True),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attnres_mutant_is_caught(name):
    failed = []
    for pin in attnres_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(MUTANTS[name])
        except (AssertionError, ValueError, IndexError, ZeroDivisionError):
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passed every pin"
