"""The LVSA-structured block pattern builder (input construction, CPU)."""
import numpy as np

from workloads.sparsity import block_pattern_from_frames, lvsa_frame_sets, lvsa_pattern, pattern_density


def test_frame_sets_budget_and_rotation():
    T, C, T_per = 41, 9, 8
    for step in range(T_per):
        sets = lvsa_frame_sets(T, C, T_per, step)
        glob = {f for f in range(T) if (f - step) % T_per == 0}
        for t, A in enumerate(sets):
            assert len(A) == min(C, T) and A == sorted(set(A))
            assert glob <= set(A)                 # every global anchor is attended
            assert t in A                         # a frame always sees itself
    # over T_per consecutive steps every frame is a global anchor exactly once
    counts = np.zeros(T, int)
    for step in range(T_per):
        for f in range(T):
            counts[f] += (f - step) % T_per == 0
    assert np.all(counts == 1)


def test_block_pattern_covers_frames():
    T, P = 13, 100                                # frames of 100 tokens: blocks straddle frames
    N = T * P
    sets = lvsa_frame_sets(T, 5, 4)
    off, idx = block_pattern_from_frames(sets, P, N)
    assert off[0] == 0 and off[-1] == idx.size and np.all(np.diff(off) >= 0)
    for qb in range(len(off) - 1):
        blocks = idx[off[qb]:off[qb + 1]]
        assert np.all(np.diff(blocks) > 0)        # sorted, unique
        assert blocks.min() >= 0 and blocks.max() < -(-N // 64)
        for i in range(qb * 256, min(N, (qb + 1) * 256), 37):
            for f in sets[i // P]:
                for k in range(f * P, (f + 1) * P, 13):
                    assert k // 64 in blocks      # every key of an allowed frame is covered


def test_full_budget_is_dense():
    off, idx = lvsa_pattern(6, 64, C=6)
    assert pattern_density(off, 6 * 64) == 1.0


def test_random_and_full_patterns():
    from workloads.sparsity import full_pattern, random_pattern
    N = 3000
    nqb, nkb = -(-N // 256), -(-N // 64)
    off, idx = full_pattern(N)
    assert off.dtype == np.int32 and idx.dtype == np.int32 and len(off) == nqb + 1
    assert all(list(idx[off[q]:off[q + 1]]) == list(range(nkb)) for q in range(nqb))
    base = random_pattern(N, keep=0.4, seed=3, empty_every=4)
    mixed = random_pattern(N, keep=0.4, seed=3, empty_every=4, invalid=3, shuffle=True)
    for q in range(nqb):
        a = base[1][base[0][q]:base[0][q + 1]]
        b = mixed[1][mixed[0][q]:mixed[0][q + 1]]
        assert len(set(a)) == len(a) and len(set(b)) == len(b)          # distinct
        assert set(a) == {x for x in b if 0 <= x < nkb}                 # same valid set
        assert len(b) == len(a) + 3
        assert (len(a) == 0) == (q % 4 == 0)
