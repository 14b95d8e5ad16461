"""The attention-block oracle against its pins, and plausible mistakes planted
in copies of it (on the CPU), each of which must fail at least one pin."""
import types

import numpy as np
import pytest

import block_pins
from oracle import block_ref as R
from oracle import hybrid_ref


def _truncate_bf16(a):
    u = np.asarray(a, dtype=np.float32).view(np.uint32)
    return ((u >> 16) << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def _round_half_up_bf16(a):
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return (((u + 0x8000) >> 16) << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def _impl(split=R.split_heads, merge=R.merge_heads, order=(0, 1, 2, 3), transpose_out=True,
          residual=True, stack="sequential", rounding=R.round_bf16):
    def project_in(x, W_in, H):
        x = np.asarray(x, dtype=np.float64)
        C = x.shape[-1]
        P = x @ np.asarray(W_in, dtype=np.float64).T
        blocks = [split(P[..., t * C:(t + 1) * C], H) for t in range(4)]
        return tuple(blocks[i] for i in order)

    def project_out(O, W_out, x):
        W = np.asarray(W_out, dtype=np.float64)
        y = merge(np.asarray(O, dtype=np.float64)) @ (W.T if transpose_out else W)
        return (np.asarray(x, dtype=np.float64) + y) if residual else y

    def block(x, W_in4, W_out4, H, kinds=hybrid_ref.SCHEDULE, store=None):
        keep = (lambda a: a) if store is None else store
        x = np.asarray(x, dtype=np.float64)
        x0 = x
        layers = list(enumerate(kinds))
        if stack == "reversed":
            layers = layers[::-1]
        for l, kind in layers:
            src = x0 if stack == "parallel" else x
            Wi = W_in4[0] if stack == "shared_in" else W_in4[l]
            Q, K, V, G = (keep(t) for t in project_in(src, Wi, H))
            x = keep(project_out(keep(hybrid_ref.layer(kind, Q, K, V, G)), W_out4[l], x))
        return x

    return types.SimpleNamespace(project_in=project_in, project_out=project_out, block=block,
                                 round_bf16=rounding)


@pytest.mark.parametrize("pin", block_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_block_oracle_pin(pin):
    pin(R)


def _split_d_major(P, H):
    B, N, C = P.shape
    return P.reshape(B, N, C // H, H).transpose(0, 3, 1, 2)


def _merge_d_major(O):
    B, H, N, d = O.shape
    return O.transpose(0, 2, 3, 1).reshape(B, N, H * d)


MUTANTS = {
    "heads split feature-major": _impl(split=_split_d_major),
    "heads merged feature-major": _impl(merge=_merge_d_major),
    "Q and K swapped": _impl(order=(1, 0, 2, 3)),
    "V and G swapped": _impl(order=(0, 1, 3, 2)),
    "gate taken from the Q block": _impl(order=(0, 1, 2, 0)),
    "W_out not transposed": _impl(transpose_out=False),
    "no residual": _impl(residual=False),
    "sub-layers read the block input": _impl(stack="parallel"),
    "sub-layers in reverse order": _impl(stack="reversed"),
    "one input projection for all": _impl(stack="shared_in"),
    "bf16 storage truncates": _impl(rounding=_truncate_bf16),
    "bf16 storage rounds ties up": _impl(rounding=_round_half_up_bf16),
}


def test_reference_impl_passes_all_pins():
    good = _impl()
    for pin in block_pins.ALL_PINS:
        pin(good)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_block_mutant_is_caught(name):
    impl = MUTANTS[name]
    failed = []
    for pin in block_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passed every pin"
