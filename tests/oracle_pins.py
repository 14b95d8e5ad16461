"""Checks that pin the CPU oracle to facts other than itself.

Each pin takes an `impl` object exposing the oracle's API (SCHEDULE, EPS,
sigmoid, kv_state, linear_attention, linear_attention_bruteforce,
softmax_attention, group) so the same checks can be run against deliberately
broken copies of the oracle (test_oracle_mutations.py): every plausible mistake
there must fail at least one pin.

Sources of truth used here:
  * the O(N^2) form of the linear layer, written out with explicit loops over
    token pairs (the oracle itself uses the O(N d^2) state form);
  * closed forms (N = 1, identical keys, two keys, V = 1, phi(q) = 0);
  * invariances (joint permutation of K and V, shift of every key by the same
    vector, linearity in V);
  * a library routine: torch's scaled_dot_product_attention in float64 on CPU;
  * hand-worked examples under tests/golden/.
"""
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(seed, N, d, scale=1.0):
    r = _rng(seed)
    return tuple(r.standard_normal((N, d)) * scale for _ in range(4))


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / den


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def linear_pairwise_loops(Q, K, V, G, eps):
    """O(N^2) gated linear attention from its pairwise definition, pure Python:
    w_ij = sum_a max(q_ia,0) max(k_ja,0); o_i = sigmoid(g_i) sum_j w_ij v_j / (sum_j w_ij + eps)."""
    N, d = len(Q), len(Q[0])
    dv = len(V[0])
    out = []
    for i in range(N):
        w = [sum(max(Q[i][a], 0.0) * max(K[j][a], 0.0) for a in range(d)) for j in range(N)]
        den = sum(w) + eps
        row = []
        for c in range(dv):
            num = sum(w[j] * V[j][c] for j in range(N))
            gate = 1.0 / (1.0 + math.exp(-G[i][c])) if G[i][c] > -700 else 0.0
            row.append(gate * num / den)
        out.append(row)
    return np.array(out)


# ----------------------------------------------------------------------------- linear layer

def pin_linear_matches_pairwise_loops(impl):
    for seed, (N, d) in enumerate([(1, 1), (5, 3), (17, 4), (40, 8)]):
        Q, K, V, G = _rand(seed, N, d)
        ref = linear_pairwise_loops(Q.tolist(), K.tolist(), V.tolist(), G.tolist(), impl.EPS)
        got = impl.linear_attention(Q, K, V, G)
        assert _rel(got, ref) < 1e-12, ("state form vs pairwise loops", N, d, _rel(got, ref))


def pin_linear_state_equals_bruteforce(impl):
    for seed, (N, d) in enumerate([(64, 16), (300, 32), (129, 64)]):
        Q, K, V, G = _rand(100 + seed, N, d)
        a = impl.linear_attention(Q, K, V, G)
        b = impl.linear_attention_bruteforce(Q, K, V, G)
        assert _rel(a, b) < 1e-12, ("state vs O(N^2) form", N, d)
        ref = linear_pairwise_loops(Q[:6].tolist(), K[:6].tolist(), V[:6].tolist(), G[:6].tolist(), impl.EPS)
        assert _rel(impl.linear_attention_bruteforce(Q[:6], K[:6], V[:6], G[:6]), ref) < 1e-12


def pin_kv_state_definition(impl):
    Q, K, V, _ = _rand(7, 23, 5)
    S, z = impl.kv_state(K, V)
    S_loop = np.zeros((5, 5))
    z_loop = np.zeros(5)
    for j in range(23):
        fk = np.maximum(K[j], 0.0)
        S_loop += np.outer(fk, V[j])
        z_loop += fk
    assert _rel(S, S_loop) < 1e-13 and _rel(z, z_loop) < 1e-13


def pin_linear_closed_forms(impl):
    eps = impl.EPS
    r = _rng(11)
    # N = 1: o = sigmoid(g) * v * a / (a + eps), a = phi(q).phi(k)
    q, k, v, g = (r.standard_normal((1, 6)) for _ in range(4))
    q[0, :3] = np.abs(q[0, :3]) + 0.5
    k[0, :3] = np.abs(k[0, :3]) + 0.5
    a = float((np.maximum(q, 0) @ np.maximum(k, 0).T)[0, 0])
    sig = 1.0 / (1.0 + np.exp(-g))
    assert _rel(impl.linear_attention(q, k, v, g), sig * v * a / (a + eps)) < 1e-13
    # identical keys: o_i = sigmoid(g_i) * a_i * sum_j v_j / (N a_i + eps)
    N, d = 9, 4
    Q, _, V, G = (r.standard_normal((N, d)) for _ in range(4))
    kk = np.abs(r.standard_normal(d)) + 0.1
    K = np.tile(kk, (N, 1))
    ai = np.maximum(Q, 0) @ kk
    ref = (1.0 / (1.0 + np.exp(-G))) * (ai[:, None] * V.sum(0)[None, :]) / (N * ai + eps)[:, None]
    assert _rel(impl.linear_attention(Q, K, V, G), ref) < 1e-13
    # a query with phi(q) = 0 gives exactly 0; keys all <= 0 give O = 0
    Q[2] = -np.abs(Q[2])
    out = impl.linear_attention(Q, K, V, G)
    assert np.all(out[2] == 0.0) and np.all(np.isfinite(out))
    out = impl.linear_attention(Q, -np.abs(K), V, G)
    assert np.all(out == 0.0)


def pin_linear_golden(impl):
    f = _load("linear_small.json")
    got = impl.linear_attention(*(np.array(f[k], dtype=np.float64) for k in "QKVG"))
    ref = np.array(f["O"], dtype=np.float64)
    assert np.allclose(got, ref, rtol=f["rtol"], atol=1e-12), (got, ref)


def pin_linear_invariances(impl):
    Q, K, V, G = _rand(21, 50, 8)
    o = impl.linear_attention(Q, K, V, G)
    p = _rng(22).permutation(50)
    assert _rel(impl.linear_attention(Q, K[p], V[p], G), o) < 1e-13        # keys are a set
    assert _rel(impl.linear_attention(Q[p], K, V, G[p]), o[p]) < 1e-13     # queries are independent
    assert _rel(impl.linear_attention(Q, K, -V, G), -o) < 1e-13            # linear in V
    assert _rel(impl.linear_attention(Q, K, 3.0 * V, G), 3.0 * o) < 1e-13


# ----------------------------------------------------------------------------- gate

def pin_gate(impl):
    for fn in (impl.linear_attention, impl.softmax_attention):
        Q, K, V, G = _rand(31, 40, 8)
        closed = fn(Q, K, V, np.full_like(G, -np.inf))
        assert np.all(closed == 0.0), "G = -inf must give exactly 0"
        open_ = fn(Q, K, V, np.full_like(G, np.inf))
        half = fn(Q, K, V, np.zeros_like(G))
        assert np.all(np.isfinite(open_))
        assert _rel(half, 0.5 * open_) < 1e-15, "G = 0 must give half the ungated output"
        got = fn(Q, K, V, G)
        assert _rel(got, open_ / (1.0 + np.exp(-G))) < 1e-13
    s = impl.sigmoid(np.array([-np.inf, -1.0986122886681098, 0.0, 1.0986122886681098, np.inf]))
    assert np.allclose(s, [0.0, 0.25, 0.5, 0.75, 1.0], rtol=1e-15, atol=0) and s[0] == 0.0 and s[-1] == 1.0


# ----------------------------------------------------------------------------- softmax anchor

def pin_softmax_matches_library(impl):
    for seed, (N, d) in enumerate([(1, 4), (33, 16), (200, 64), (77, 128)]):
        Q, K, V, _ = _rand(40 + seed, N, d, scale=2.0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(x)[None, None] for x in (Q, K, V)))[0, 0].numpy()
        got = impl.softmax_attention(Q, K, V, np.full((N, d), np.inf))
        assert _rel(got, ref) < 1e-12, ("softmax vs torch SDPA", N, d, _rel(got, ref))


def pin_softmax_closed_forms(impl):
    r = _rng(51)
    # weights sum to one: V = 1 gives O = sigmoid(G)
    N, d = 60, 16
    Q, K, _, G = (r.standard_normal((N, d)) * 3 for _ in range(4))
    out = impl.softmax_attention(Q, K, np.ones((N, d)), G)
    assert _rel(out, 1.0 / (1.0 + np.exp(-G))) < 1e-14
    # one token: o = sigmoid(g) v
    q, k, v, g = (r.standard_normal((1, 8)) for _ in range(4))
    assert _rel(impl.softmax_attention(q, k, v, g), v / (1.0 + np.exp(-g))) < 1e-15
    # two tokens: weight of key 1 = logistic(s1 - s2)
    Q, K, V, G = (r.standard_normal((2, 8)) for _ in range(4))
    s = Q @ K.T / math.sqrt(8)
    w1 = 1.0 / (1.0 + np.exp(-(s[:, 0] - s[:, 1])))
    ref = (w1[:, None] * V[0] + (1 - w1)[:, None] * V[1]) / (1.0 + np.exp(-G))
    assert _rel(impl.softmax_attention(Q, K, V, G), ref) < 1e-14


def pin_softmax_invariances(impl):
    Q, K, V, G = _rand(61, 70, 16)
    o = impl.softmax_attention(Q, K, V, G)
    c = _rng(62).standard_normal(16) * 400.0        # huge common shift of every key
    assert _rel(impl.softmax_attention(Q, K + c, V, G), o) < 1e-9
    p = _rng(63).permutation(70)
    assert _rel(impl.softmax_attention(Q, K[p], V[p], G), o) < 1e-13
    rows = np.array([0, 5, 69, 33])
    assert _rel(impl.softmax_attention(Q, K, V, G, rows=rows), o[rows]) < 1e-15


def pin_softmax_golden(impl):
    f = _load("softmax_small.json")
    got = impl.softmax_attention(*(np.array(f[k], dtype=np.float64) for k in "QKVG"))
    ref = np.array(f["O"], dtype=np.float64)
    assert np.all(np.isfinite(got)) and np.allclose(got, ref, rtol=f["rtol"], atol=1e-12), (got, ref)


# ----------------------------------------------------------------------------- group

def pin_group_structure(impl):
    kinds = list(impl.SCHEDULE)
    assert len(kinds) == 4 and kinds.count("linear") == 3 and kinds.count("softmax") == 1
    assert kinds[-1] == "softmax"
    r = _rng(71)
    B, H, N, d = 1, 2, 24, 8
    X = [r.standard_normal((4, B, H, N, d)) for _ in range(4)]
    out = impl.group(*X)
    assert out.shape == (4, B, H, N, d)
    for l in range(4):
        for h in range(H):
            q, k, v, g = (x[l, 0, h] for x in X)
            if l < 3:
                ref = linear_pairwise_loops(q.tolist(), k.tolist(), v.tolist(), g.tolist(), impl.EPS)
            else:
                ref = torch.nn.functional.scaled_dot_product_attention(
                    *(torch.from_numpy(x)[None, None] for x in (q, k, v)))[0, 0].numpy()
                ref = ref / (1.0 + np.exp(-g))
            assert _rel(out[l, 0, h], ref) < 1e-12, ("group layer", l, h)


# ----------------------------------------------------------------------------- block-sparse anchor

def _csr(lists):
    offsets = np.cumsum([0] + [len(l) for l in lists]).astype(np.int32)
    indices = np.asarray([b for l in lists for b in l], dtype=np.int32)
    return offsets, indices


def pin_sparse_full_pattern_is_dense(impl):
    for seed, (N, d) in enumerate([(300, 16), (700, 32)]):
        Q, K, V, G = _rand(80 + seed, N, d, scale=2.0)
        nqb, nkb = -(-N // impl.SPARSE_BLOCK_Q), -(-N // impl.SPARSE_BLOCK_K)
        off, idx = _csr([list(range(nkb))] * nqb)
        got = impl.softmax_attention_blocksparse(Q, K, V, G, off, idx)
        assert _rel(got, impl.softmax_attention(Q, K, V, G)) < 1e-13


def pin_sparse_matches_masked_library(impl):
    N, d = 600, 16
    Q, K, V, G = _rand(90, N, d, scale=2.0)
    r = _rng(91)
    nqb, nkb = -(-N // impl.SPARSE_BLOCK_Q), -(-N // impl.SPARSE_BLOCK_K)
    lists = [sorted(r.choice(nkb, size=int(r.integers(0, nkb + 1)), replace=False).tolist()) for _ in range(nqb)]
    lists[1] = []                                  # an empty row set
    off, idx = _csr(lists)
    mask = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for b in lists[i // impl.SPARSE_BLOCK_Q]:
            mask[i, b * impl.SPARSE_BLOCK_K:min(N, (b + 1) * impl.SPARSE_BLOCK_K)] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x)[None, None] for x in (Q, K, V)), attn_mask=torch.from_numpy(mask)[None, None])[0, 0].numpy()
    ref = ref / (1.0 + np.exp(-G))
    got = impl.softmax_attention_blocksparse(Q, K, V, G, off, idx)
    live = mask.any(axis=1)
    assert np.all(got[~live] == 0.0), "a query with no allowed key gets 0"
    assert _rel(got[live], ref[live]) < 1e-12


def pin_sparse_single_block_and_tail(impl):
    N, d = 530, 8                                    # last key block holds 530 - 8*64 = 18 keys
    Q, K, V, G = _rand(95, N, d)
    nqb, nkb = -(-N // impl.SPARSE_BLOCK_Q), -(-N // impl.SPARSE_BLOCK_K)
    lists = [[3], [nkb - 1], [0]]
    off, idx = _csr(lists)
    got = impl.softmax_attention_blocksparse(Q, K, V, G, off, idx)
    for qb, (b,) in enumerate(lists):
        rows = slice(qb * 256, min(N, (qb + 1) * 256))
        keys = slice(b * 64, min(N, (b + 1) * 64))
        # queries of block qb against only that key slice: plain softmax attention
        Qs, Gs = Q[rows], G[rows]
        Kb, Vb = K[keys], V[keys]
        s = Qs @ Kb.T / math.sqrt(d)
        w = np.exp(s - s.max(1, keepdims=True))
        ref = (w @ Vb) / w.sum(1, keepdims=True) / (1.0 + np.exp(-Gs))
        assert _rel(got[rows], ref) < 1e-13, ("single block", qb, b)


def pin_sparse_set_semantics(impl):
    N, d = 520, 8
    Q, K, V, G = _rand(97, N, d)
    base = [[0, 2, 5], [1, 3], [8]]
    off, idx = _csr(base)
    o = impl.softmax_attention_blocksparse(Q, K, V, G, off, idx)
    off2, idx2 = _csr([[5, 0, 2, 2], [3, 1, 99, -4], [8, 8]])   # reordered, repeated, out of range
    assert _rel(impl.softmax_attention_blocksparse(Q, K, V, G, off2, idx2), o) < 1e-15
    rows = np.array([0, 255, 256, 511, 519])
    assert _rel(impl.softmax_attention_blocksparse(Q, K, V, G, off, idx, rows=rows), o[rows]) < 1e-15


ALL_PINS = [
    pin_linear_matches_pairwise_loops,
    pin_linear_state_equals_bruteforce,
    pin_kv_state_definition,
    pin_linear_closed_forms,
    pin_linear_golden,
    pin_linear_invariances,
    pin_gate,
    pin_softmax_matches_library,
    pin_softmax_closed_forms,
    pin_softmax_invariances,
    pin_softmax_golden,
    pin_group_structure,
    pin_sparse_full_pattern_is_dense,
    pin_sparse_matches_masked_library,
    pin_sparse_single_block_and_tail,
    pin_sparse_set_semantics,
]
