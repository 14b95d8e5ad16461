"""CPU oracle for the attention block around the hybrid group.

TEST INFRASTRUCTURE ONLY: the slow, plain float64 reference the library's
projection kernels and block entry point are checked against.  It shares no
code with the library, and the library never imports it.

The block (SANA-Video 2.0 review page, section 3, where the hybrid layers sit
inside the DiT blocks the compiled forward runs; summary page, section 03, the
3:1 interleave) is read as four attention sub-layers on a residual stream
x [B, N, C], C = H * d, layer l of kind SCHEDULE[l]:

    P   = x W_in[l]^T                 W_in[l]: [4C, C], rows = output features
    Q, K, V, G = the four C-wide column blocks of P, in that order, each split
                 into H heads of d consecutive features: [B, H, N, d]
    O   = layer kind l (Q, K, V, G)   gated linear or gated softmax attention
    x  <- x + concat_h(O) W_out[l]^T  W_out[l]: [C, C]; head h fills columns
                                      h*d .. h*d + d - 1 of the concatenation

The pages print neither the projections nor the residual; this is the plainest
reading (the gate G is one more projection of x, like Q, K and V).  Norms,
time-step modulation, cross-attention and the MLP of a DiT block lie outside.
"""
import numpy as np

from .hybrid_ref import SCHEDULE, layer


def split_heads(P, H):
    """[B, N, C] -> [B, H, N, d]: head h takes features h*d .. h*d + d - 1."""
    B, N, C = P.shape
    d = C // H
    return P.reshape(B, N, H, d).transpose(0, 2, 1, 3)


def merge_heads(O):
    """[B, H, N, d] -> [B, N, H*d], the inverse of split_heads."""
    B, H, N, d = O.shape
    return O.transpose(0, 2, 1, 3).reshape(B, N, H * d)


def project_in(x, W_in, H):
    """Q, K, V, G [B, H, N, d] of x [B, N, C] through W_in [4C, C]."""
    x = np.asarray(x, dtype=np.float64)
    W_in = np.asarray(W_in, dtype=np.float64)
    C = x.shape[-1]
    if W_in.shape != (4 * C, C) or C % H:
        raise ValueError(f"W_in must be [{4 * C}, {C}] and H must divide C, got {W_in.shape}, H={H}")
    P = x @ W_in.T
    return tuple(split_heads(P[..., t * C:(t + 1) * C], H) for t in range(4))


def project_out(O, W_out, x):
    """x + concat_h(O) W_out^T for O [B, H, N, d], W_out [C, C], x [B, N, C]."""
    O = np.asarray(O, dtype=np.float64)
    W_out = np.asarray(W_out, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return x + merge_heads(O) @ W_out.T


def round_bf16(a):
    """Round to the nearest bfloat16 (ties to even) by way of float32, the
    storage format of a bf16 tensor: keep the top 16 bits of the float32
    pattern after adding 0x7FFF plus the lowest kept bit.  Returns float64."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def block(x, W_in4, W_out4, H, kinds=SCHEDULE, store=None):
    """The four sub-layers in order; W_in4 [L, 4C, C], W_out4 [L, C, C].

    `store`, when given, is applied to every tensor the block hands from one
    stage to the next (Q, K, V, G, O and the updated x): round_bf16 models a
    path that keeps those tensors in bfloat16 while its arithmetic is exact."""
    x = np.asarray(x, dtype=np.float64)
    keep = (lambda a: a) if store is None else store
    if len(W_in4) != len(kinds) or len(W_out4) != len(kinds):
        raise ValueError(f"{len(kinds)} layers need {len(kinds)} weight pairs")
    for l, kind in enumerate(kinds):
        Q, K, V, G = (keep(t) for t in project_in(x, W_in4[l], H))
        x = keep(project_out(keep(layer(kind, Q, K, V, G)), W_out4[l], x))
    return x


# ---------------------------------------------------------------------------
# Block attention residuals (AttnRes).  The pages (summary page, section 03;
# review page, sections 1 and 3; news item) describe it only in words: instead
# of a layer reading just the running sum of earlier outputs, summaries of
# completed blocks are routed into later linear layers.  The reading used here:
# a block is one hybrid group, its summary is the stream after it, and the
# projections of each linear sub-layer of a later group read a depth-wise
# softmax mixture of the completed summaries and the current stream (the stream
# itself is one candidate, so the plain residual path is kept):
#     score_b = w . (v_b / rms(v_b)) / sqrt(C),  rms(v) = sqrt(mean(v^2) + eps)
#     h       = sum_b softmax_b(score) v_b
# per token, with w a learned routing vector of the sub-layer.  The anchor reads
# the stream; every residual update still goes to the stream.

RMS_EPS = 1e-6


def attnres_mix(candidates, w, eps=RMS_EPS):
    """h [B, N, C] = softmax-over-candidates mixture of candidates [M, B, N, C]
    with scores w . rmsnorm(v) / sqrt(C), per token."""
    V = np.asarray(candidates, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    C = V.shape[-1]
    rms = np.sqrt((V * V).mean(axis=-1) + eps)                # [M, B, N]
    score = (V @ w) / rms / np.sqrt(C)                        # [M, B, N]
    score = score - score.max(axis=0, keepdims=True)
    a = np.exp(score)
    a /= a.sum(axis=0, keepdims=True)
    return (a[..., None] * V).sum(axis=0)


def block_routed(x, summaries, w_route, W_in4, W_out4, H, kinds=SCHEDULE, store=None):
    """One block whose linear sub-layers read attnres_mix(summaries + [stream],
    w_route[l]); summaries [M, B, N, C] (M may be 0), w_route [L, C]."""
    x = np.asarray(x, dtype=np.float64)
    keep = (lambda a: a) if store is None else store
    summaries = np.asarray(summaries, dtype=np.float64).reshape((-1,) + x.shape)
    for l, kind in enumerate(kinds):
        src = x
        if kind == "linear":
            src = keep(attnres_mix(np.concatenate([summaries, x[None]], axis=0), w_route[l]))
        Q, K, V, G = (keep(t) for t in project_in(src, W_in4[l], H))
        x = keep(project_out(keep(layer(kind, Q, K, V, G)), W_out4[l], x))
    return x


def stack_routed(x, w_route, W_in, W_out, H, store=None):
    """n blocks in sequence (W_in [n, 4, 4C, C], W_out [n, 4, C, C], w_route
    [n, 4, C]); block k routes the summaries of blocks 0 .. k-1."""
    x = np.asarray(x, dtype=np.float64)
    summaries = []
    for k in range(len(W_in)):
        prev = np.stack(summaries) if summaries else np.zeros((0,) + x.shape)
        x = block_routed(x, prev, w_route[k], W_in[k], W_out[k], H, store=store)
        summaries.append(x)
    return x
