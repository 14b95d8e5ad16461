"""The backward oracle against its pins, the row- and key-sampled forms against
the full one, and plausible mistakes planted in copies of it (on the CPU), each
of which must fail at least one pin."""
import math
import types

import numpy as np
import pytest

import backward_pins
from oracle import backward_ref as B
from oracle import hybrid_ref as R


def _impl(lin=B.linear_attention_backward, soft=B.softmax_attention_backward):
    return types.SimpleNamespace(EPS=R.EPS, linear_attention=R.linear_attention,
                                 softmax_attention=R.softmax_attention,
                                 linear_attention_backward=lin, softmax_attention_backward=soft)


@pytest.mark.parametrize("pin", backward_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(_impl())


def test_sampled_forms_match_full():
    r = np.random.default_rng(3)
    Q, K, V, G, dO = (r.standard_normal((70, 8)) for _ in range(5))
    dQ, dK, dV, dG = B.softmax_attention_backward(Q, K, V, G, dO, row_block=16)
    rows = np.array([0, 5, 69])
    q, g = B.softmax_attention_backward_rows(Q, K, V, G, dO, rows)
    assert np.allclose(q, dQ[rows], rtol=1e-12, atol=1e-14) and np.allclose(g, dG[rows], rtol=1e-12, atol=1e-14)
    keys = np.array([1, 33, 68])
    k, v = B.softmax_attention_backward_keys(Q, K, V, G, dO, keys, row_block=32)
    assert np.allclose(k, dK[keys], rtol=1e-11, atol=1e-14) and np.allclose(v, dV[keys], rtol=1e-11, atol=1e-14)
    lse = B.softmax_lse(Q, K, row_block=16)
    L = Q @ K.T / math.sqrt(8)
    assert np.allclose(lse, np.log(np.exp(L).sum(axis=1)), rtol=1e-13)


# --- planted mistakes ---------------------------------------------------------

def _lin_mut(kind):
    def f(Q, K, V, G, dO, eps=R.EPS):
        Q, K, V, G, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, G, dO))
        S, z = R.kv_state(K, V)
        fq, fk = R.phi(Q), R.phi(K)
        den = fq @ z + eps
        a = (fq @ S) / den[:, None]
        s = R.sigmoid(G)
        dG = dO * a * ((1.0 - s) if kind == "gate" else s * (1.0 - s))
        da = dO * s
        dn = da / den[:, None]
        dden = (1 if kind == "sign" else -1) * (da * a).sum(axis=1) / den
        dS = fq.T @ dn
        dz = fq.T @ dden
        mask_q = 1.0 if kind == "qmask" else (Q > 0)
        dQ = (dn @ (S if kind == "transpose" else S.T) + dden[:, None] * z[None, :]) * mask_q
        dK = (V @ dS.T + (0.0 if kind == "dz" else dz[None, :])) * (K > 0)
        dV = fk @ dS
        return dQ, dK, dV, dG
    return f


def _soft_mut(kind):
    def f(Q, K, V, G, dO):
        Q, K, V, G, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, G, dO))
        d = Q.shape[1]
        scale = 1.0 / math.sqrt(d)
        L = Q @ K.T * scale
        P = np.exp(L - L.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        a = P @ V
        s = R.sigmoid(G)
        dG = dO * a * s * (1.0 - s)
        da = dO * s
        D = (da * a).sum(axis=1) if kind != "noD" else 0.0
        dS = P * (da @ V.T - (D[:, None] if kind != "noD" else 0.0))
        qs = 1.0 if kind == "noscale" else scale
        dQ = dS @ K * qs
        dK = dS.T @ Q * scale
        dV = (P @ da) if kind == "PnotT" else (P.T @ da)
        if kind == "dOgate":
            dV = P.T @ dO
        return dQ, dK, dV, dG
    return f


MUTANTS = {
    "linear: dG uses (1 - s) for s (1 - s)": _impl(lin=_lin_mut("gate")),
    "linear: wrong sign of dden": _impl(lin=_lin_mut("sign")),
    "linear: ReLU mask missing on dQ": _impl(lin=_lin_mut("qmask")),
    "linear: S instead of S^T in dQ": _impl(lin=_lin_mut("transpose")),
    "linear: dz missing from dK": _impl(lin=_lin_mut("dz")),
    "softmax: D_i term missing": _impl(soft=_soft_mut("noD")),
    "softmax: 1/sqrt(d) missing in dQ": _impl(soft=_soft_mut("noscale")),
    "softmax: P instead of P^T in dV": _impl(soft=_soft_mut("PnotT")),
    "softmax: dV from dO, not dO * sigmoid(g)": _impl(soft=_soft_mut("dOgate")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name):
    failed = []
    for pin in backward_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(MUTANTS[name])
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passed every pin"
