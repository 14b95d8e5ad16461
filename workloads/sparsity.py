"""Block-sparse attention patterns for the long-sequence anchor.

The long-video page (LVSA, "2. Method", "Core mechanism") restricts the frames a
query frame t attends to A(t) = G_s  U  W(t): G_s, a periodic set of global
anchor frames that shifts by s (mod T_per) at every denoising step s, so that
over T_per steps every frame is a global anchor once; W(t), a local window
around t that is extended when it overlaps global frames so that |A(t)| stays
at the budget C.  The page leaves the window's exact shape open; the reading
used here: W(t) holds the frames nearest to t (ties to the earlier frame) that
are not global, as many as bring |A(t)| to min(C, T).

Frames are mapped to token blocks: query block qb (SPARSE_BLOCK_Q tokens) sees
the union of A(t) over the frames its tokens belong to, and a key block
(SPARSE_BLOCK_K tokens) is listed when it overlaps any of those frames.  The
result is a CSR pattern (offsets per query block, sorted unique key-block
indices) shared by every head and batch item.  This module only builds index
sets; it computes no part of the attention.
"""
import math

import numpy as np

SPARSE_BLOCK_Q = 256
SPARSE_BLOCK_K = 64


def lvsa_frame_sets(T: int, C: int, T_per: int, step: int = 0) -> list:
    """A(t) for t = 0..T-1 as sorted frame lists."""
    glob = [f for f in range(T) if (f - step) % T_per == 0]
    gset = set(glob)
    budget = min(C, T)
    sets = []
    for t in range(T):
        chosen = set(glob) if len(glob) < budget else set(sorted(glob, key=lambda f: (abs(f - t), f))[:budget])
        others = sorted((f for f in range(T) if f not in gset), key=lambda f: (abs(f - t), f))
        for f in others:
            if len(chosen) >= budget:
                break
            chosen.add(f)
        sets.append(sorted(chosen))
    return sets


def block_pattern_from_frames(frame_sets, tokens_per_frame: int, N: int,
                              block_q: int = SPARSE_BLOCK_Q, block_k: int = SPARSE_BLOCK_K):
    """CSR (offsets int32 [nqb+1], indices int32) of key blocks per query block."""
    nqb = -(-N // block_q)
    offsets = [0]
    indices = []
    for qb in range(nqb):
        t0 = (qb * block_q) // tokens_per_frame
        t1 = (min(N, (qb + 1) * block_q) - 1) // tokens_per_frame
        frames = set()
        for t in range(t0, t1 + 1):
            frames.update(frame_sets[t])
        blocks = set()
        for f in frames:
            k_lo, k_hi = f * tokens_per_frame, min(N, (f + 1) * tokens_per_frame)
            blocks.update(range(k_lo // block_k, (k_hi - 1) // block_k + 1))
        indices.extend(sorted(blocks))
        offsets.append(len(indices))
    return np.asarray(offsets, dtype=np.int32), np.asarray(indices, dtype=np.int32)


def lvsa_pattern(frames: int, tokens_per_frame: int, C: int = 21, T_per: int | None = None, step: int = 0):
    """LVSA-structured pattern for a latent of `frames` x `tokens_per_frame`
    tokens.  T_per defaults to a period giving about C/2 global frames."""
    if T_per is None:
        T_per = max(1, math.ceil(frames / max(1, C // 2)))
    N = frames * tokens_per_frame
    sets = lvsa_frame_sets(frames, C, T_per, step)
    return block_pattern_from_frames(sets, tokens_per_frame, N)


def pattern_density(offsets, N: int, block_q: int = SPARSE_BLOCK_Q, block_k: int = SPARSE_BLOCK_K) -> float:
    """Fraction of the dense query-key pairs the pattern keeps."""
    nqb = len(offsets) - 1
    nkb = -(-N // block_k)
    return float(np.diff(offsets).sum()) / (nqb * nkb)


def full_pattern(N: int, block_q: int = SPARSE_BLOCK_Q, block_k: int = SPARSE_BLOCK_K):
    """Every key block for every query block (the dense anchor as a pattern)."""
    nqb, nkb = -(-N // block_q), -(-N // block_k)
    offsets = np.arange(nqb + 1, dtype=np.int64) * nkb
    indices = np.tile(np.arange(nkb, dtype=np.int32), nqb)
    return offsets.astype(np.int32), indices


def random_pattern(N: int, keep: float = 0.3, seed: int = 0, empty_every: int = 0,
                   invalid: int = 0, shuffle: bool = False,
                   block_q: int = SPARSE_BLOCK_Q, block_k: int = SPARSE_BLOCK_K):
    """Seeded unstructured pattern: each query block keeps a random subset of
    about keep * nkb distinct key blocks (at least one).  empty_every > 0 leaves
    every empty_every-th query block with no block; invalid > 0 appends that many
    out-of-range indices (-1, nkb, nkb + 7, ...) to every list; shuffle puts each
    list in random order.  Indices stay distinct within a query block."""
    rng = np.random.default_rng(seed)
    order_rng = np.random.default_rng([seed, 1])   # the order never changes the sets
    nqb, nkb = -(-N // block_q), -(-N // block_k)
    bad = [-1, nkb, nkb + 7, -1000, 2 * nkb + 3][:invalid]
    offsets = [0]
    indices = []
    for qb in range(nqb):
        if empty_every and qb % empty_every == 0:
            blocks = []
        else:
            n = min(nkb, max(1, int(round(keep * nkb))))
            blocks = sorted(rng.choice(nkb, size=n, replace=False).tolist())
        blocks = blocks + bad
        if shuffle:
            order_rng.shuffle(blocks)
        indices.extend(blocks)
        offsets.append(len(indices))
    return np.asarray(offsets, dtype=np.int32), np.asarray(indices, dtype=np.int32)
