"""Checks that pin the backward oracle (oracle/backward_ref.py) to facts other
than its own chain-rule derivation.

Each pin takes an `impl` exposing the forward functions (linear_attention,
softmax_attention: pinned elsewhere) and the backward ones, so that broken
copies of the backward (test_backward_oracle.py) are caught.

Sources of truth:
  * central finite differences of the forward (the gradient's definition) on
    tiny inputs;
  * a library: torch autograd in float64 through torch's own
    scaled_dot_product_attention for the anchor, and through the pairwise
    O(N^2) form of the linear layer (not the state form the oracle uses);
  * invariances: a common shift of all keys leaves the anchor unchanged, so
    its key gradients sum to zero; the linear layer is (up to eps) invariant
    to scaling Q or K, so sum_i q_i . dq_i = 0 and sum_j k_j . dk_j = 0;
  * closed forms: dG = dO * o * (1 - sigmoid(g)) for both layers; dV = 0
    when dO = 0 on every row; V enters linearly, so dV does not depend on V.
"""
import math

import numpy as np
import torch


def _rand(seed, N, d, scale=1.0):
    r = np.random.default_rng(seed)
    return tuple(r.standard_normal((N, d)) * scale for _ in range(5))


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def _fd_grads(fwd, X, dO, h=1e-6):
    """Central differences of L = sum(dO * fwd(*X)) with respect to every input."""
    grads = []
    for t in range(len(X)):
        g = np.zeros_like(X[t])
        for idx in np.ndindex(X[t].shape):
            Xp = [x.copy() for x in X]
            Xm = [x.copy() for x in X]
            Xp[t][idx] += h
            Xm[t][idx] -= h
            g[idx] = ((dO * fwd(*Xp)).sum() - (dO * fwd(*Xm)).sum()) / (2 * h)
        grads.append(g)
    return grads


def pin_linear_finite_differences(impl):
    Q, K, V, G, dO = _rand(40, 5, 3)
    Q[0, 0] = 0.3   # keep every entry away from the ReLU kink
    num = _fd_grads(impl.linear_attention, [Q, K, V, G], dO)
    got = impl.linear_attention_backward(Q, K, V, G, dO)
    for name, a, b in zip("QKVG", got, num):
        assert _rel(a, b) < 1e-5, (name, _rel(a, b))


def pin_softmax_finite_differences(impl):
    Q, K, V, G, dO = _rand(41, 6, 3)
    num = _fd_grads(impl.softmax_attention, [Q, K, V, G], dO)
    got = impl.softmax_attention_backward(Q, K, V, G, dO)
    for name, a, b in zip("QKVG", got, num):
        assert _rel(a, b) < 1e-6, (name, _rel(a, b))


def pin_softmax_matches_library_autograd(impl):
    Q, K, V, G, dO = _rand(42, 37, 8)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V, G)]
    att = torch.nn.functional.scaled_dot_product_attention(t[0][None, None], t[1][None, None],
                                                           t[2][None, None])[0, 0]
    (torch.sigmoid(t[3]) * att * torch.tensor(dO)).sum().backward()
    got = impl.softmax_attention_backward(Q, K, V, G, dO)
    for name, a, ref in zip("QKVG", got, t):
        assert _rel(a, ref.grad.numpy()) < 1e-12, name


def pin_linear_matches_pairwise_autograd(impl):
    """torch autograd through the O(N^2) pairwise form (weights phi(q).phi(k)),
    a different expression of the layer than the oracle's state form."""
    Q, K, V, G, dO = _rand(43, 29, 6)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V, G)]
    A = torch.relu(t[0]) @ torch.relu(t[1]).T
    out = torch.sigmoid(t[3]) * (A @ t[2]) / (A.sum(dim=1, keepdim=True) + impl.EPS)
    (out * torch.tensor(dO)).sum().backward()
    got = impl.linear_attention_backward(Q, K, V, G, dO)
    for name, a, ref in zip("QKVG", got, t):
        assert _rel(a, ref.grad.numpy()) < 1e-10, name


def pin_softmax_key_shift(impl):
    Q, K, V, G, dO = _rand(44, 40, 8)
    dQ, dK, dV, dG = impl.softmax_attention_backward(Q, K, V, G, dO)
    assert np.abs(dK.sum(axis=0)).max() < 1e-12 * max(1.0, np.abs(dK).max() * 40)


def pin_linear_scale_invariance(impl):
    Q, K, V, G, dO = _rand(45, 40, 8)
    dQ, dK, dV, dG = impl.linear_attention_backward(Q, K, V, G, dO)
    # d/dl O(lQ) at l = 1 is 0 up to the eps term (eps / den ~ 1e-8 here)
    assert abs((Q * dQ).sum()) < 1e-6 * np.abs(Q * dQ).sum()
    assert abs((K * dK).sum()) < 1e-6 * np.abs(K * dK).sum()


def pin_gate_closed_form(impl):
    Q, K, V, G, dO = _rand(46, 20, 4)
    for fwd, bwd in ((impl.linear_attention, impl.linear_attention_backward),
                     (impl.softmax_attention, impl.softmax_attention_backward)):
        o = fwd(Q, K, V, G)
        s = 1.0 / (1.0 + np.exp(-G))
        assert _rel(bwd(Q, K, V, G, dO)[3], dO * o * (1.0 - s)) < 1e-12


def pin_v_enters_linearly(impl):
    Q, K, V, G, dO = _rand(47, 15, 4)
    V2 = np.random.default_rng(48).standard_normal(V.shape)
    for bwd in (impl.linear_attention_backward, impl.softmax_attention_backward):
        assert _rel(bwd(Q, K, V2, G, dO)[2], bwd(Q, K, V, G, dO)[2]) < 1e-12
        zero = bwd(Q, K, V, G, np.zeros_like(dO))
        assert all(np.abs(g).max() == 0.0 for g in zero)


ALL_PINS = [
    pin_linear_finite_differences,
    pin_softmax_finite_differences,
    pin_softmax_matches_library_autograd,
    pin_linear_matches_pairwise_autograd,
    pin_softmax_key_shift,
    pin_linear_scale_invariance,
    pin_gate_closed_form,
    pin_v_enters_linearly,
]
