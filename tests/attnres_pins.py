"""Checks that pin the AttnRes reading of the oracle (attnres_mix and the
routed block / stack in oracle/block_ref.py) to facts other than itself.

Each pin takes an `impl` exposing attnres_mix, block, block_routed and
stack_routed (block itself is pinned in block_pins.py), so that broken copies
are caught (test_attnres_oracle.py).

Sources of truth: the mixture written out with explicit loops over tokens,
candidates and features; closed forms (one candidate gives it back, w = 0 gives
the mean, scaling one candidate keeps its weight, a dominant score selects its
candidate); invariance to the order of the candidates and equivariance under a
token permutation; the routed block with no completed summaries equals the
plain block; a stack of one block equals that block.
"""
import math

import numpy as np


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def pin_mix_loops(impl):
    r = np.random.default_rng(60)
    M, B, N, C = 3, 2, 3, 5
    V = r.standard_normal((M, B, N, C)) * r.uniform(0.5, 3, size=(M, 1, 1, 1))
    w = r.standard_normal(C)
    got = impl.attnres_mix(V, w)
    for b in range(B):
        for n in range(N):
            scores = []
            for m in range(M):
                ms = sum(V[m, b, n, c] ** 2 for c in range(C)) / C
                rms = math.sqrt(ms + 1e-6)
                scores.append(sum(w[c] * V[m, b, n, c] for c in range(C)) / rms / math.sqrt(C))
            e = [math.exp(sc - max(scores)) for sc in scores]
            for c in range(C):
                want = sum(e[m] * V[m, b, n, c] for m in range(M)) / sum(e)
                assert abs(got[b, n, c] - want) < 1e-12, (b, n, c)


def pin_mix_closed_forms(impl):
    r = np.random.default_rng(61)
    V = r.standard_normal((4, 1, 6, 8))
    w = r.standard_normal(8)
    assert np.array_equal(impl.attnres_mix(V[:1], w), V[0])            # one candidate
    assert _rel(impl.attnres_mix(V, np.zeros(8)), V.mean(axis=0)) < 1e-13
    # scaling candidate 0 by 3 keeps every weight (its key is RMS-normalised)
    V3 = V.copy()
    V3[0] *= 3.0
    h, h3 = impl.attnres_mix(V, w), impl.attnres_mix(V3, w)
    C = V.shape[-1]
    rms = np.sqrt((V * V).mean(axis=-1) + 1e-6)
    s = (V @ w) / rms / np.sqrt(C)
    a0 = np.exp(s[0]) / np.exp(s).sum(axis=0)
    assert _rel(h3, h + 2.0 * a0[..., None] * V[0]) < 1e-6
    # a dominant score selects its candidate
    big = 1e4 * V[2, 0, 0] / np.linalg.norm(V[2, 0, 0])
    assert _rel(impl.attnres_mix(V[:, :, :1], big), V[2, :, :1]) < 1e-6


def pin_mix_symmetries(impl):
    r = np.random.default_rng(62)
    V = r.standard_normal((5, 2, 7, 6))
    w = r.standard_normal(6)
    h = impl.attnres_mix(V, w)
    assert _rel(impl.attnres_mix(V[[3, 0, 4, 1, 2]], w), h) < 1e-13
    perm = r.permutation(7)
    assert _rel(impl.attnres_mix(V[:, :, perm], w), h[:, perm]) < 1e-13


def pin_routed_block_reduces_to_block(impl):
    r = np.random.default_rng(63)
    B, N, H, d = 1, 10, 2, 4
    C = H * d
    x = r.standard_normal((B, N, C))
    Wi = r.standard_normal((4, 4 * C, C)) / np.sqrt(C)
    Wo = r.standard_normal((4, C, C)) / np.sqrt(C)
    wr = r.standard_normal((4, C))
    none = np.zeros((0, B, N, C))
    assert _rel(impl.block_routed(x, none, wr, Wi, Wo, H), impl.block(x, Wi, Wo, H)) < 1e-12
    one = impl.stack_routed(x, wr[None], Wi[None], Wo[None], H)
    assert _rel(one, impl.block(x, Wi, Wo, H)) < 1e-12


def pin_routing_reaches_linear_layers_only(impl):
    """With W_out of the linear sub-layers zero, only the anchor updates the
    stream, and it reads the stream, not the mixture: the summaries do not
    matter.  With the anchor's W_out zero instead, they do."""
    r = np.random.default_rng(64)
    B, N, H, d = 1, 9, 2, 3
    C = H * d
    x = r.standard_normal((B, N, C))
    S = r.standard_normal((2, B, N, C)) * 3
    Wi = r.standard_normal((4, 4 * C, C)) / np.sqrt(C)
    Wo = r.standard_normal((4, C, C))
    wr = r.standard_normal((4, C)) * 4
    Wl = Wo.copy()
    Wl[:3] = 0.0
    a = impl.block_routed(x, S, wr, Wi, Wl, H)
    b = impl.block_routed(x, S * 0.5 + 1.0, wr, Wi, Wl, H)
    assert _rel(a, b) < 1e-13
    Wa = Wo.copy()
    Wa[3] = 0.0
    a = impl.block_routed(x, S, wr, Wi, Wa, H)
    b = impl.block_routed(x, S * 0.5 + 1.0, wr, Wi, Wa, H)
    assert _rel(a, b) > 1e-3


def pin_stack_routes_completed_blocks(impl):
    """Block k of a stack sees exactly the outputs of blocks 0 .. k-1."""
    r = np.random.default_rng(65)
    B, N, H, d = 1, 8, 2, 2
    C = H * d
    x = r.standard_normal((B, N, C))
    Wi = r.standard_normal((3, 4, 4 * C, C)) / np.sqrt(C)
    Wo = r.standard_normal((3, 4, C, C)) / np.sqrt(C)
    wr = r.standard_normal((3, 4, C)) * 2
    x1 = impl.block_routed(x, np.zeros((0, B, N, C)), wr[0], Wi[0], Wo[0], H)
    x2 = impl.block_routed(x1, x1[None], wr[1], Wi[1], Wo[1], H)
    x3 = impl.block_routed(x2, np.stack([x1, x2]), wr[2], Wi[2], Wo[2], H)
    assert _rel(impl.stack_routed(x, wr, Wi, Wo, H), x3) < 1e-12


def pin_first_routed_sublayer(impl):
    """With only sub-layer 0 updating, the routed block is
    x + update(h0) where h0 = mix([summary, x]) (the stream is a candidate) and
    update(h) = block(h, one linear sub-layer) - h (the update goes to x)."""
    r = np.random.default_rng(66)
    B, N, H, d = 1, 7, 2, 3
    C = H * d
    x = r.standard_normal((B, N, C))
    S = r.standard_normal((1, B, N, C)) * 2
    Wi = r.standard_normal((4, 4 * C, C)) / np.sqrt(C)
    Wo = r.standard_normal((4, C, C))
    Wo[1:] = 0.0
    wr = r.standard_normal((4, C)) * 3
    h0 = impl.attnres_mix(np.concatenate([S, x[None]], axis=0), wr[0])
    upd = impl.block(h0, Wi[:1], Wo[:1], H, kinds=("linear",)) - h0
    assert _rel(impl.block_routed(x, S, wr, Wi, Wo, H), x + upd) < 1e-12


ALL_PINS = [
    pin_first_routed_sublayer,
    pin_mix_loops,
    pin_mix_closed_forms,
    pin_mix_symmetries,
    pin_routed_block_reduces_to_block,
    pin_routing_reaches_linear_layers_only,
    pin_stack_routes_completed_blocks,
]
