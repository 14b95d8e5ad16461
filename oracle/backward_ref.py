"""CPU oracle for the backward pass of the two gated layers.

TEST INFRASTRUCTURE ONLY: the plain float64 reference the library's backward
kernels are checked against.  It shares no code with the library.

The pages train the model from scratch (review page, section 3; news item,
"Prestaties"), so each layer needs the gradients of a loss L with respect to
its Q, K, V and G given dO = dL/dO.  Both are written out from the forward
definitions by the chain rule (no library differentiation), per head, with
phi = ReLU (derivative 1 where the input is > 0, else 0) and
sigmoid'(x) = sigmoid(x) (1 - sigmoid(x)).

Gated linear layer, o_i = s_i * a_i with s_i = sigmoid(g_i), a_i = n_i / den_i,
n_i = phi(q_i) S, den_i = phi(q_i) . z + eps, S = sum_j phi(k_j)^T v_j,
z = sum_j phi(k_j):
    da_i   = dO_i * s_i                  dG_i = dO_i * a_i * s_i (1 - s_i)
    dn_i   = da_i / den_i                dden_i = -(da_i . a_i) / den_i
    dS     = sum_i phi(q_i)^T dn_i       dz = sum_i dden_i phi(q_i)
    dQ_i   = (dn_i S^T + dden_i z) * [q_i > 0]
    dK_j   = (v_j dS^T + dz) * [k_j > 0] dV_j = phi(k_j) dS

Gated softmax anchor, o_i = s_i * a_i, a_i = sum_j P_ij v_j,
P = softmax_j(q_i . k_j / sqrt(d)):
    da_i   = dO_i * s_i                  dG_i = dO_i * a_i * s_i (1 - s_i)
    D_i    = da_i . a_i  (= dO_i . o_i)  dP_ij = da_i . v_j
    dS_ij  = P_ij (dP_ij - D_i)
    dQ_i   = sum_j dS_ij k_j / sqrt(d)   dK_j = sum_i dS_ij q_i / sqrt(d)
    dV_j   = sum_i P_ij da_i
"""
import math

import numpy as np

from .hybrid_ref import EPS, kv_state, phi, sigmoid


def _f64(*xs):
    return tuple(np.asarray(x, dtype=np.float64) for x in xs)


def linear_attention_backward(Q, K, V, G, dO, eps=EPS):
    """dQ, dK, dV, dG of the gated linear layer of one head ([N, d] each)."""
    Q, K, V, G, dO = _f64(Q, K, V, G, dO)
    S, z = kv_state(K, V)
    fq, fk = phi(Q), phi(K)
    n = fq @ S
    den = fq @ z + eps
    a = n / den[:, None]
    s = sigmoid(G)
    dG = dO * a * s * (1.0 - s)
    da = dO * s
    dn = da / den[:, None]
    dden = -(da * a).sum(axis=1) / den
    dS = fq.T @ dn
    dz = fq.T @ dden
    dQ = (dn @ S.T + dden[:, None] * z[None, :]) * (Q > 0)
    dK = (V @ dS.T + dz[None, :]) * (K > 0)
    dV = fk @ dS
    return dQ, dK, dV, dG


def softmax_lse(Q, K, row_block=512):
    """Natural log of sum_j exp(q_i . k_j / sqrt(d)) for every query row."""
    Q, K = _f64(Q, K)
    scale = 1.0 / math.sqrt(Q.shape[1])
    out = np.empty(Q.shape[0])
    for r0 in range(0, Q.shape[0], row_block):
        L = (Q[r0:r0 + row_block] @ K.T) * scale
        m = L.max(axis=1)
        out[r0:r0 + row_block] = m + np.log(np.exp(L - m[:, None]).sum(axis=1))
    return out


def softmax_attention_backward(Q, K, V, G, dO, row_block=512):
    """dQ, dK, dV, dG of the gated softmax anchor of one head ([N, d] each),
    query rows taken row_block at a time (memory only; every sum is complete)."""
    Q, K, V, G, dO = _f64(Q, K, V, G, dO)
    N, d = Q.shape
    scale = 1.0 / math.sqrt(d)
    dQ = np.empty_like(Q)
    dG = np.empty_like(G)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for r0 in range(0, N, row_block):
        r = slice(r0, r0 + row_block)
        L = (Q[r] @ K.T) * scale
        P = np.exp(L - L.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        a = P @ V
        s = sigmoid(G[r])
        dG[r] = dO[r] * a * s * (1.0 - s)
        da = dO[r] * s
        D = (da * a).sum(axis=1)
        dP = da @ V.T
        dS = P * (dP - D[:, None])
        dQ[r] = (dS @ K) * scale
        dK += (dS.T @ Q[r]) * scale
        dV += P.T @ da
    return dQ, dK, dV, dG


def softmax_attention_backward_rows(Q, K, V, G, dO, rows):
    """dQ and dG of the anchor for the query rows `rows` only (each row's
    gradient depends on its own dO row and all keys)."""
    Q, K, V, G, dO = _f64(Q, K, V, G, dO)
    rows = np.asarray(rows, dtype=np.int64)
    scale = 1.0 / math.sqrt(Q.shape[1])
    L = (Q[rows] @ K.T) * scale
    P = np.exp(L - L.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    a = P @ V
    s = sigmoid(G[rows])
    da = dO[rows] * s
    D = (da * a).sum(axis=1)
    dS = P * (da @ V.T - D[:, None])
    return (dS @ K) * scale, dO[rows] * a * s * (1.0 - s)


def softmax_attention_backward_keys(Q, K, V, G, dO, keys, row_block=2048):
    """dK and dV of the anchor for the key rows `keys` only: sums over every
    query, each query's softmax normalised over all keys (its log-sum-exp)."""
    Q, K, V, G, dO = _f64(Q, K, V, G, dO)
    keys = np.asarray(keys, dtype=np.int64)
    scale = 1.0 / math.sqrt(Q.shape[1])
    dK = np.zeros((keys.size, K.shape[1]))
    dV = np.zeros((keys.size, V.shape[1]))
    for r0 in range(0, Q.shape[0], row_block):
        r = slice(r0, r0 + row_block)
        L = (Q[r] @ K.T) * scale
        m = L.max(axis=1, keepdims=True)
        E = np.exp(L - m)
        P = E / E.sum(axis=1, keepdims=True)
        a = P @ V
        da = dO[r] * sigmoid(G[r])
        D = (da * a).sum(axis=1)
        Pk = P[:, keys]
        dS = Pk * (da @ V[keys].T - D[:, None])
        dK += (dS.T @ Q[r]) * scale
        dV += Pk.T @ da
    return dK, dV


def layer_backward(kind, Q, K, V, G, dO):
    """Gradients of one gated layer over [B, H, N, d] arrays."""
    fn = linear_attention_backward if kind == "linear" else softmax_attention_backward
    Q, K, V, G, dO = _f64(Q, K, V, G, dO)
    out = [np.empty_like(Q) for _ in range(4)]
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            for t, g in zip(out, fn(Q[b, h], K[b, h], V[b, h], G[b, h], dO[b, h])):
                t[b, h] = g
    return tuple(out)
