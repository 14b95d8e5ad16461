"""Checks that pin the attention-block oracle (oracle/block_ref.py) to facts
other than itself.

Each pin takes an `impl` exposing project_in, project_out, block and layer, so
the same checks run against deliberately broken copies of the oracle
(test_block_oracle.py): every plausible mistake there must fail a pin.

Sources of truth:
  * the projections written out element by element with explicit loops over
    features (the oracle uses matrix products and reshapes);
  * closed forms: a zero output projection leaves the stream unchanged; zero
    keys make a linear layer output exactly zero and a softmax layer the
    gated mean of V, written without any head split; one token (N = 1);
  * structure: equivariance under a token permutation, invariance under a
    joint relabelling of heads, independence of batch items, linearity of one
    sub-layer's update in W_out, and the block as the composition of its
    sub-layers in order.
"""
import numpy as np

SCHEDULE = ("linear", "linear", "linear", "softmax")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def _weights(seed, L, C, s_in=None, s_out=None):
    r = np.random.default_rng(seed)
    s_in = 1.0 / np.sqrt(C) if s_in is None else s_in
    s_out = 1.0 / np.sqrt(C) if s_out is None else s_out
    return r.standard_normal((L, 4 * C, C)) * s_in, r.standard_normal((L, C, C)) * s_out


def pin_project_in_loops(impl):
    B, N, H, d = 2, 3, 2, 3
    C = H * d
    r = np.random.default_rng(10)
    x = r.standard_normal((B, N, C))
    W = r.standard_normal((4 * C, C))
    got = impl.project_in(x, W, H)
    for t in range(4):
        for b in range(B):
            for h in range(H):
                for n in range(N):
                    for e in range(d):
                        want = sum(x[b, n, c] * W[t * C + h * d + e, c] for c in range(C))
                        assert abs(got[t][b, h, n, e] - want) < 1e-12, (t, b, h, n, e)


def pin_project_out_loops(impl):
    B, N, H, d = 2, 3, 2, 3
    C = H * d
    r = np.random.default_rng(11)
    O = r.standard_normal((B, H, N, d))
    W = r.standard_normal((C, C))
    x = r.standard_normal((B, N, C))
    got = impl.project_out(O, W, x)
    for b in range(B):
        for n in range(N):
            for c in range(C):
                want = x[b, n, c] + sum(O[b, h, n, e] * W[c, h * d + e] for h in range(H) for e in range(d))
                assert abs(got[b, n, c] - want) < 1e-12, (b, n, c)


def pin_zero_output_projection_is_identity(impl):
    B, N, H, d = 1, 9, 2, 4
    x = np.random.default_rng(12).standard_normal((B, N, H * d))
    Wi, Wo = _weights(13, 4, H * d)
    assert np.array_equal(impl.block(x, Wi, np.zeros_like(Wo), H), x)


def pin_zero_keys_closed_forms(impl):
    """K = 0: phi(K) = 0, so a linear layer outputs sigmoid(g) * 0 / eps = 0;
    a softmax layer sees equal logits and outputs sigmoid(g) * mean_j v_j.
    Written without heads: the gate and the mean act feature by feature."""
    B, N, H, d = 2, 7, 2, 3
    C = H * d
    r = np.random.default_rng(14)
    x = r.standard_normal((B, N, C))
    Wi, Wo = _weights(15, 1, C, s_in=1.0)
    Wi[0, C:2 * C] = 0.0                       # the K rows
    assert np.array_equal(impl.block(x, Wi, Wo, H, kinds=("linear",)), x)
    Wv, Wg = Wi[0, 2 * C:3 * C], Wi[0, 3 * C:]
    want = np.empty_like(x)
    for b in range(B):
        mean_v = x[b].mean(axis=0) @ Wv.T       # [C]
        y = _sig(x[b] @ Wg.T) * mean_v[None, :]
        want[b] = x[b] + y @ Wo[0].T
    assert _rel(impl.block(x, Wi, Wo, H, kinds=("softmax",)), want) < 1e-12


def pin_single_token(impl):
    """N = 1: softmax gives sigmoid(g) v; linear gives sigmoid(g) v a / (a + eps)
    with a = phi(q) . phi(k), per head."""
    B, H, d = 1, 3, 2
    C = H * d
    r = np.random.default_rng(16)
    x = r.standard_normal((B, 1, C))
    Wi, Wo = _weights(17, 1, C, s_in=1.0, s_out=1.0)
    P = x[0, 0] @ Wi[0].T
    q, k, v, g = (P[t * C:(t + 1) * C] for t in range(4))
    y_soft = _sig(g) * v
    y_lin = np.empty(C)
    for h in range(H):
        sl = slice(h * d, (h + 1) * d)
        a = float(np.maximum(q[sl], 0) @ np.maximum(k[sl], 0))
        y_lin[sl] = _sig(g[sl]) * v[sl] * a / (a + 1e-6)
    for kind, y in (("softmax", y_soft), ("linear", y_lin)):
        want = x[0, 0] + Wo[0] @ y
        assert _rel(impl.block(x, Wi, Wo, H, kinds=(kind,))[0, 0], want) < 1e-12, kind


def pin_token_permutation(impl):
    B, N, H, d = 2, 11, 2, 4
    r = np.random.default_rng(18)
    x = r.standard_normal((B, N, H * d))
    Wi, Wo = _weights(19, 4, H * d)
    perm = r.permutation(N)
    assert _rel(impl.block(x[:, perm], Wi, Wo, H), impl.block(x, Wi, Wo, H)[:, perm]) < 1e-12


def pin_head_relabelling(impl):
    B, N, H, d = 1, 10, 3, 2
    C = H * d
    r = np.random.default_rng(20)
    x = r.standard_normal((B, N, C))
    Wi, Wo = _weights(21, 4, C)
    hp = np.array([2, 0, 1])
    feat = np.concatenate([np.arange(h * d, (h + 1) * d) for h in hp])     # new feature order
    rows = np.concatenate([t * C + feat for t in range(4)])
    Wi2 = Wi[:, rows, :]
    Wo2 = Wo[:, :, feat]
    assert _rel(impl.block(x, Wi2, Wo2, H), impl.block(x, Wi, Wo, H)) < 1e-12


def pin_batch_independence(impl):
    N, H, d = 8, 2, 4
    r = np.random.default_rng(22)
    x = r.standard_normal((2, N, H * d))
    Wi, Wo = _weights(23, 4, H * d)
    both = impl.block(x, Wi, Wo, H)
    for b in range(2):
        assert _rel(both[b:b + 1], impl.block(x[b:b + 1], Wi, Wo, H)) < 1e-13


def pin_update_linear_in_output_projection(impl):
    B, N, H, d = 1, 9, 2, 3
    r = np.random.default_rng(24)
    x = r.standard_normal((B, N, H * d))
    Wi, Wo = _weights(25, 1, H * d)
    for kind in ("linear", "softmax"):
        y1 = impl.block(x, Wi, Wo, H, kinds=(kind,)) - x
        y3 = impl.block(x, Wi, 3.0 * Wo, H, kinds=(kind,)) - x
        assert _rel(y3, 3.0 * y1) < 1e-12, kind
        assert np.abs(y1).max() > 1e-3, kind     # the update is not trivially zero


def pin_block_is_composition_in_order(impl):
    B, N, H, d = 1, 12, 2, 4
    r = np.random.default_rng(26)
    x = r.standard_normal((B, N, H * d))
    Wi, Wo = _weights(27, 4, H * d, s_out=1.0)
    want = x
    for l, kind in enumerate(SCHEDULE):
        want = impl.block(want, Wi[l:l + 1], Wo[l:l + 1], H, kinds=(kind,))
    assert _rel(impl.block(x, Wi, Wo, H), want) < 1e-12
    # and the sub-layers do not commute: the order is observable
    rev = x
    for l in reversed(range(4)):
        rev = impl.block(rev, Wi[l:l + 1], Wo[l:l + 1], H, kinds=(SCHEDULE[l],))
    assert _rel(rev, want) > 1e-6


def pin_round_bf16_matches_library(impl):
    """The storage rounding against torch's float32 -> bfloat16 conversion (round
    to nearest even) on random values of every magnitude and on exact ties."""
    import torch
    r = np.random.default_rng(28)
    v = (r.standard_normal(20000) * np.exp2(r.integers(-30, 30, 20000))).astype(np.float32)
    ties = (np.arange(1, 4001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)   # half-way bit patterns
    for a in (v, ties, -ties, np.array([0.0, -0.0, 1.0, 65504.0, 1e-38], dtype=np.float32)):
        want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
        assert np.array_equal(impl.round_bf16(a), want)


def pin_storage_rounding_is_applied(impl):
    """With a storage rounding the block differs from the exact one by a few
    bf16 ulps of the stream, and identity storage changes nothing."""
    B, N, H, d = 1, 16, 2, 4
    x = np.random.default_rng(29).standard_normal((B, N, H * d))
    Wi, Wo = _weights(30, 4, H * d)
    exact = impl.block(x, Wi, Wo, H)
    assert np.array_equal(impl.block(x, Wi, Wo, H, store=lambda a: a), exact)
    rounded = impl.block(x, Wi, Wo, H, store=impl.round_bf16)
    assert 0 < _rel(rounded, exact) < 2.0 ** -5
    assert np.array_equal(impl.round_bf16(rounded), rounded)   # the stream is stored


ALL_PINS = [
    pin_round_bf16_matches_library,
    pin_storage_rounding_is_applied,
    pin_project_in_loops,
    pin_project_out_loops,
    pin_zero_output_projection_is_identity,
    pin_zero_keys_closed_forms,
    pin_single_token,
    pin_token_permutation,
    pin_head_relabelling,
    pin_batch_independence,
    pin_update_linear_in_output_projection,
    pin_block_is_composition_in_order,
]
