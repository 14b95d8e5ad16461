"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them."""
import math
import types

import numpy as np
import pytest

import oracle
import oracle_pins
from oracle import hybrid_ref as R


def _impl(**over):
    ns = {k: getattr(R, k) for k in ("EPS", "SCHEDULE", "phi", "sigmoid", "kv_state", "linear_attention",
                                     "linear_attention_bruteforce", "softmax_attention", "group", "layer",
                                     "SPARSE_BLOCK_Q", "SPARSE_BLOCK_K", "softmax_attention_blocksparse")}
    ns.update(over)
    impl = types.SimpleNamespace(**ns)

    # rebind the composite functions so they call the (possibly mutated) pieces
    def kv_state(K, V):
        return ns["kv_state"](K, V)

    def group(Q4, K4, V4, G4):
        outs = []
        for l, kind in enumerate(impl.SCHEDULE):
            fn = impl.linear_attention if kind == "linear" else impl.softmax_attention
            B, H = Q4.shape[1:3]
            outs.append(np.stack([np.stack([fn(Q4[l, b, h], K4[l, b, h], V4[l, b, h], G4[l, b, h])
                                            for h in range(H)]) for b in range(B)]))
        return np.stack(outs)

    impl.group = group
    impl.kv_state = kv_state
    return impl


def _linear_with(kv=None, phi_q=R.phi, sig=R.sigmoid, eps=R.EPS, den_eps=True, gate="mul"):
    def lin(Q, K, V, G, eps=eps):
        S, z = (kv or R.kv_state)(K, V)
        fq = phi_q(np.asarray(Q, dtype=np.float64))
        num = fq @ S
        den = fq @ z + (eps if den_eps else 0.0)
        if gate == "mul":
            return sig(G) * num / den[:, None]
        return sig(G) + num / den[:, None]
    return lin


def _softmax_with(scale=lambda d: 1.0 / math.sqrt(d), axis=1, sub_max=True, sig=R.sigmoid, values="V"):
    def sm(Q, K, V, G, rows=None):
        Q, K, V, G = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, G))
        rows = np.arange(Q.shape[0]) if rows is None else np.asarray(rows)
        L = (Q[rows] @ K.T) * scale(Q.shape[1])
        with np.errstate(over="ignore", invalid="ignore"):
            if sub_max:
                L = L - L.max(axis=axis, keepdims=True)
            P = np.exp(L)
            P = P / P.sum(axis=axis, keepdims=True)
        Vs = V if values == "V" else K
        return sig(G[rows]) * (P @ Vs)
    return sm


def _kv_transposed(K, V):
    S, z = R.kv_state(K, V)
    return S.T, z


def _kv_phi_on_v(K, V):
    return R.kv_state(K, np.maximum(V, 0.0))


def _kv_z_without_phi(K, V):
    S, _ = R.kv_state(K, V)
    return S, np.asarray(K).sum(0)


def _kv_no_phi(K, V):
    K = np.asarray(K, dtype=np.float64)
    return K.T @ np.asarray(V, dtype=np.float64), K.sum(0)


def _sig_flipped(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(np.asarray(x, dtype=np.float64)))


def _bad_bruteforce_no_eps(Q, K, V, G, eps=R.EPS):
    return R.linear_attention_bruteforce(Q, K, V, G, eps=0.0)


def _sparse_with(key_block=None, query_block=None, drop_tail=False, empty_uniform=False):
    def sp(Q, K, V, G, offsets, indices, rows=None, block_q=R.SPARSE_BLOCK_Q, block_k=R.SPARSE_BLOCK_K):
        Q, K, V, G = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, G))
        N, d = Q.shape
        rows = np.arange(N) if rows is None else np.asarray(rows)
        bq = query_block or block_q
        bk = key_block or block_k
        out = np.zeros((rows.size, V.shape[1]))
        for n, i in enumerate(rows):
            qb = min(i // bq, len(offsets) - 2)
            blocks = sorted({int(b) for b in indices[offsets[qb]:offsets[qb + 1]] if 0 <= b < -(-N // block_k)})
            keys = [k for b in blocks for k in range(b * bk, (b + 1) * bk) if (k < N or not drop_tail) and k < N + (0 if not drop_tail else 0)]
            if drop_tail:
                keys = [k for k in keys if k < (N // bk) * bk]
            if not keys:
                out[n] = (1.0 / (1.0 + np.exp(-G[i]))) / V.shape[1] if empty_uniform else 0.0
                continue
            keys = np.asarray(keys)
            s = Q[i] @ K[keys].T / math.sqrt(d)
            w = np.exp(s - s.max())
            out[n] = (1.0 / (1.0 + np.exp(-G[i]))) * (w @ V[keys]) / w.sum()
        return out
    return sp


MUTANTS = {
    "S transposed": dict(linear_attention=_linear_with(kv=_kv_transposed)),
    "phi applied to V": dict(linear_attention=_linear_with(kv=_kv_phi_on_v)),
    "z without phi": dict(linear_attention=_linear_with(kv=_kv_z_without_phi)),
    "no feature map on K": dict(linear_attention=_linear_with(kv=_kv_no_phi)),
    "no feature map on Q": dict(linear_attention=_linear_with(phi_q=lambda x: x)),
    "eps dropped": dict(linear_attention=_linear_with(den_eps=False),
                        linear_attention_bruteforce=_bad_bruteforce_no_eps),
    "eps 1e-2": dict(linear_attention=_linear_with(eps=1e-2)),
    "additive gate": dict(linear_attention=_linear_with(gate="add")),
    "gate sign flipped": dict(sigmoid=_sig_flipped, linear_attention=_linear_with(sig=_sig_flipped),
                              softmax_attention=_softmax_with(sig=_sig_flipped)),
    "softmax scale 1/d": dict(softmax_attention=_softmax_with(scale=lambda d: 1.0 / d)),
    "softmax unscaled": dict(softmax_attention=_softmax_with(scale=lambda d: 1.0)),
    "softmax over queries": dict(softmax_attention=_softmax_with(axis=0)),
    "softmax without max subtraction": dict(softmax_attention=_softmax_with(sub_max=False)),
    "softmax mixes keys for values": dict(softmax_attention=_softmax_with(values="K")),
    "anchor first in the period": dict(SCHEDULE=("softmax", "linear", "linear", "linear")),
    "all-linear group": dict(SCHEDULE=("linear", "linear", "linear", "linear")),
    "2:2 group": dict(SCHEDULE=("linear", "softmax", "linear", "softmax")),
    "sparse: key blocks of 32": dict(softmax_attention_blocksparse=_sparse_with(key_block=32)),
    "sparse: query blocks of 128": dict(softmax_attention_blocksparse=_sparse_with(query_block=128)),
    "sparse: ragged key tail dropped": dict(softmax_attention_blocksparse=_sparse_with(drop_tail=True)),
    "sparse: empty rows not zero": dict(softmax_attention_blocksparse=_sparse_with(empty_uniform=True)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    impl = _impl(**MUTANTS[name])
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"


def test_unmutated_copy_passes_every_pin():
    impl = _impl()
    for pin in oracle_pins.ALL_PINS:
        pin(impl)
    assert impl.SCHEDULE == oracle.SCHEDULE
