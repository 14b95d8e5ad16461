"""CPU oracle for one Hybrid Linear-Softmax Attention group.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct reference
the HIP kernels are checked against.  It shares no code with the library, and
the library never imports it.

What it computes (float64 throughout, on the exact values the GPU sees):

* Gated linear attention layer -- the O(N) layer of the hybrid group (SANA-Video
  2.0 summary page, section 03; review page, section 1, "Hybrid Linear-Softmax
  Attention").  The pages name the layer but print no formula; the form used
  here is the one fixed for this library: feature map phi = ReLU, per-head state
  S = sum_j phi(k_j) v_j^T and normaliser z = sum_j phi(k_j), output
  o_i = sigmoid(g_i) * (phi(q_i)^T S) / (phi(q_i) . z + eps), with eps = 1e-6
  inside the denominator and "*" elementwise (G has the shape of O).
* Gated softmax anchor layer -- the O(N^2) layer (same passages):
  o_i = sigmoid(g_i) * sum_j softmax_j(q_i . k_j / sqrt(d)) v_j.
* The group: three linear layers then one softmax anchor, the 3:1 ratio of the
  pages (summary page, section 03; review page, section 3: 25 % softmax), with
  the anchor last in the period.  Every layer has its own Q, K, V, G; nothing
  links the layers inside this attention-only slice.

Attention is bidirectional: every query sees all N tokens of its (batch, head);
nothing is masked and nothing crosses batch items or heads.

Every function here is pinned by the CPU tests against something other than
itself (the O(N^2) form of the linear layer, closed forms, invariances, a
library softmax-attention routine and hand-worked examples).
"""
import math

import numpy as np

EPS = 1e-6
SCHEDULE = ("linear", "linear", "linear", "softmax")
# Block-sparse anchor: a pattern lists, for every block of SPARSE_BLOCK_Q
# consecutive queries, the blocks of SPARSE_BLOCK_K consecutive keys it sees.
SPARSE_BLOCK_Q = 256
SPARSE_BLOCK_K = 64


def phi(x):
    """Feature map of the linear layer: ReLU, max(x, 0)."""
    return np.maximum(x, 0.0)


def sigmoid(x):
    """Logistic gate 1 / (1 + exp(-x)); exactly 0 at -inf and 1 at +inf."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def kv_state(K, V):
    """Linear-attention state of one head: S = sum_j phi(k_j) v_j^T (d x d) and
    z = sum_j phi(k_j) (d).  K, V: [N, d]."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    fk = phi(K)
    S = fk.T @ V
    z = fk.sum(axis=0)
    return S, z


def linear_attention(Q, K, V, G, eps=EPS):
    """Gated linear attention of one head in state form.  Q, K, V, G: [N, d]."""
    Q = np.asarray(Q, dtype=np.float64)
    S, z = kv_state(K, V)
    fq = phi(Q)
    num = fq @ S
    den = fq @ z + eps
    return sigmoid(G) * num / den[:, None]


def linear_attention_bruteforce(Q, K, V, G, eps=EPS):
    """The same layer in its O(N^2) form: weights A_ij = phi(q_i) . phi(k_j),
    o_i = sigmoid(g_i) * sum_j A_ij v_j / (sum_j A_ij + eps)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    A = phi(Q) @ phi(K).T
    num = A @ V
    den = A.sum(axis=1) + eps
    return sigmoid(G) * num / den[:, None]


def softmax_attention(Q, K, V, G, rows=None, row_block=512):
    """Gated softmax attention of one head.  Q, K, V, G: [N, d].

    rows: optional index array of query rows to evaluate (rows are independent,
    so a sampled row is an exact check of that row); the result then has
    len(rows) rows.  Query rows are processed row_block at a time only to bound
    memory; each row is evaluated on its own, over all N keys.  The row maximum
    is subtracted before exponentiating, which leaves softmax unchanged and keeps
    exp finite.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    if rows is None:
        rows = np.arange(Q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    d = Q.shape[1]
    scale = 1.0 / math.sqrt(d)
    out = np.empty((rows.size, V.shape[1]), dtype=np.float64)
    for s in range(0, rows.size, row_block):
        r = rows[s:s + row_block]
        logits = (Q[r] @ K.T) * scale
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        l = p.sum(axis=1, keepdims=True)
        out[s:s + r.size] = sigmoid(G[r]) * (p @ V) / l
    return out


def allowed_keys(N, offsets, indices, qb, block_k=SPARSE_BLOCK_K):
    """Sorted key positions that query block qb may attend to: the union of the
    listed key blocks, each clipped to [0, N); indices outside [0, ceil(N/block_k))
    are ignored and a block listed twice counts once."""
    nkb = -(-N // block_k)
    beg, end = int(offsets[qb]), int(offsets[qb + 1])
    blocks = sorted({int(b) for b in indices[beg:end] if 0 <= int(b) < nkb})
    if not blocks:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(b * block_k, min((b + 1) * block_k, N)) for b in blocks])


def softmax_attention_blocksparse(Q, K, V, G, offsets, indices, rows=None,
                                  block_q=SPARSE_BLOCK_Q, block_k=SPARSE_BLOCK_K):
    """Gated softmax attention where query i sees only the keys of the blocks its
    query block (i // block_q) lists -- the block-sparse form of the anchor that
    the long-sequence pages point to (Sol-Engine's sparse attention, LoSA's and
    LVSA's block patterns).  o_i = sigmoid(g_i) * sum_{j in A(i)} softmax_j(q_i.k_j
    / sqrt(d)) v_j; a query whose set A(i) is empty gets o_i = 0."""
    Q, K, V, G = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, G))
    N, d = Q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, V.shape[1]), dtype=np.float64)
    scale = 1.0 / math.sqrt(d)
    for qb in np.unique(rows // block_q):
        sel = np.nonzero(rows // block_q == qb)[0]
        keys = allowed_keys(N, offsets, indices, qb, block_k)
        if keys.size == 0:
            continue
        r = rows[sel]
        logits = (Q[r] @ K[keys].T) * scale
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        out[sel] = sigmoid(G[r]) * (p @ V[keys]) / p.sum(axis=1, keepdims=True)
    return out


def layer(kind, Q, K, V, G, rows=None):
    """One gated layer over [B, H, N, d] arrays; returns [B, H, N, d] (or
    [B, H, len(rows), d] for a softmax layer evaluated on sampled rows)."""
    Q, K, V, G = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, G))
    B, H = Q.shape[:2]
    outs = []
    for b in range(B):
        per_h = []
        for h in range(H):
            if kind == "linear":
                o = linear_attention(Q[b, h], K[b, h], V[b, h], G[b, h])
                if rows is not None:
                    o = o[np.asarray(rows)]
            elif kind == "softmax":
                o = softmax_attention(Q[b, h], K[b, h], V[b, h], G[b, h], rows=rows)
            else:
                raise ValueError(f"unknown layer kind {kind!r}")
            per_h.append(o)
        outs.append(np.stack(per_h))
    return np.stack(outs)


def group(Q4, K4, V4, G4):
    """One hybrid group over stacked [4, B, H, N, d] inputs, layer l of kind
    SCHEDULE[l]; returns stacked [4, B, H, N, d] outputs."""
    if len(Q4) != len(SCHEDULE):
        raise ValueError(f"a group has {len(SCHEDULE)} layers, got {len(Q4)}")
    return np.stack([layer(kind, Q4[l], K4[l], V4[l], G4[l]) for l, kind in enumerate(SCHEDULE)])
