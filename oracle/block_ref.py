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
