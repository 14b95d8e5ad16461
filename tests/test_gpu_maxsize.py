"""The largest sequence the library accepts (N = 2^23 tokens per head, where
one bf16 head of d = 128 is exactly 2^31 bytes and the anchor's 32-bit buffer
offsets and record counts sit at their limit), one head, checked against the
oracle on sampled query rows (rows are independent, so each is an exact check).
The anchor's backward at this length would run for minutes; it runs at half
of it (2^22 tokens, one head), with dQ and dG exact on sampled rows and dK, dV
through identities that hold at any length.

Sums over millions of keys are where fp32 accumulation breaks down: with the
near-flat logits of these inputs every probability is close to one, and a
plain running sum whose ulp has grown past their spread rounds each of them the
same way.  The anchor's log-sum-exp is therefore checked against a bound that
follows from the arithmetic, at 2^23 keys in bf16 and at 2^19 keys in fp32
(one sum over every key per query there)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import hybrid_linear_softmax_amd as ha
import oracle
from gpu_util import TOL, rel_err, sample_rows, say
from workloads import get, layer_inputs_device, to_f64

pytestmark = pytest.mark.gpu

MAX_N = 1 << 23
F32_N = 1 << 19

# |lse - lse_ref| bounds.  All summed terms are positive, so the relative error
# of the row sum is at most the largest relative error of a term plus that of
# the summation.  bf16: each probability is rounded to bf16 (at most 2^-9)
# before it is summed, compensated fp32 addition contributes O(2^-23) at any
# length, exp2 and the fp32 logits about 1e-6.  fp32: probabilities stay fp32;
# 32-key block sums (at most 32 ulp) join a compensated running sum.
LSE_BOUND = {"bf16": math.log1p(2.0 ** -9) + 1e-5, "f32": 1e-5}


@pytest.fixture(scope="module")
def inputs():
    w = dataclasses.replace(get("720p5s"), name="maxn", H=1, N=MAX_N)
    say(f"max-size inputs: B=1 H=1 N={MAX_N} d=128 bf16")
    x = layer_inputs_device(w, 0, "cuda")
    torch.cuda.synchronize()
    k = to_f64(x["K"][0, 0])
    v = to_f64(x["V"][0, 0])
    return w, x, k, v


def _rows():
    # first and last tiles (the last query block is full: 2^23 is a multiple of 256)
    return sample_rows(MAX_N, n_rand=24, seed=7)


def test_linear_at_max_n(inputs):
    w, x, k, v = inputs
    say("max-size linear layer")
    O = ha.hybrid_attn_linear(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    rows = _rows()
    ref = oracle.linear_attention(to_f64(x["Q"][0, 0][rows]), k, v, to_f64(x["G"][0, 0][rows]))
    got = to_f64(O[0, 0][rows])
    assert np.all(np.isfinite(got))
    e = rel_err(got, ref)
    say(f"  linear N=2^23: {rows.size} rows, max rel err {e:.2e}")
    assert e < TOL["bf16"]


def _check_anchor_lse(x, k, v, rows, dtype, label):
    """The anchor's output and log-sum-exp (the same kernel as
    hybrid_attn_softmax, which only skips the lse store) on sampled rows."""
    O, lse = ha.hybrid_attn_softmax_lse(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    q, g = to_f64(x["Q"][0, 0][rows]), to_f64(x["G"][0, 0][rows])
    ref = oracle.softmax_attention(q, k, v, g)
    ref_lse = oracle.softmax_lse(q, k)
    got = to_f64(O[0, 0][rows])
    got_lse = lse[0, 0][rows].double().cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_lse))
    e = rel_err(got, ref)
    e_lse = float(np.abs(got_lse - ref_lse).max())
    say(f"  {label}: {rows.size} rows, max rel err {e:.2e}, lse err {e_lse:.2e} "
        f"(bound {LSE_BOUND[dtype]:.2e}, mean {np.mean(got_lse - ref_lse):+.1e})")
    assert e < TOL[dtype]
    assert e_lse < LSE_BOUND[dtype]


def test_anchor_at_max_n(inputs):
    w, x, k, v = inputs
    say("max-size softmax anchor (about 30 s on the GPU)")
    _check_anchor_lse(x, k, v, _rows(), "bf16", "anchor N=2^23")


def test_anchor_f32_long():
    w = dataclasses.replace(get("720p5s"), name="long_f32", H=1, N=F32_N, dtype="f32")
    say(f"fp32 softmax anchor: B=1 H=1 N={F32_N} d=128")
    x = layer_inputs_device(w, 0, "cuda")
    torch.cuda.synchronize()
    rows = sample_rows(F32_N, n_rand=24, seed=11)
    _check_anchor_lse(x, to_f64(x["K"][0, 0]), to_f64(x["V"][0, 0]), rows, "f32", "fp32 anchor N=2^19")


def test_blocksparse_anchor_at_max_n(inputs):
    w, x, k, v = inputs
    nqb, nkb = MAX_N // 256, MAX_N // 64
    # every query block sees the first key block, the four covering its own
    # tokens and the last one (the largest offsets a key load takes)
    lists = [sorted({0, 4 * qb, 4 * qb + 1, 4 * qb + 2, 4 * qb + 3, nkb - 1}) for qb in range(nqb)]
    off = np.cumsum([0] + [len(b) for b in lists]).astype(np.int32)
    idx = np.asarray([b for blocks in lists for b in blocks], dtype=np.int32)
    say(f"max-size block-sparse anchor: {idx.size} listed blocks")
    O = ha.hybrid_attn_softmax_blocksparse(x["Q"], x["K"], x["V"], x["G"], torch.from_numpy(off).cuda(),
                                          torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    rows = _rows()
    q, g = to_f64(x["Q"][0, 0]), to_f64(x["G"][0, 0])
    ref = oracle.softmax_attention_blocksparse(q, k, v, g, off, idx, rows=rows)
    got = to_f64(O[0, 0][rows])
    assert np.all(np.isfinite(got))
    e = rel_err(got, ref)
    say(f"  block-sparse N=2^23: {rows.size} rows, max rel err {e:.2e}")
    assert e < TOL["bf16"]


def test_linear_and_anchor_at_max_n_d64():
    # the other head size at the largest sequence: one bf16 head of d = 64 is
    # 2^30 bytes; the anchor's lse held to the same derived bound
    w = dataclasses.replace(get("720p5s"), name="maxn_d64", H=1, N=MAX_N, d=64)
    say(f"max-size inputs: B=1 H=1 N={MAX_N} d=64 bf16")
    x = layer_inputs_device(w, 0, "cuda")
    torch.cuda.synchronize()
    k, v = to_f64(x["K"][0, 0]), to_f64(x["V"][0, 0])
    rows = sample_rows(MAX_N, n_rand=24, seed=9)
    O = ha.hybrid_attn_linear(x["Q"], x["K"], x["V"], x["G"])
    torch.cuda.synchronize()
    ref = oracle.linear_attention(to_f64(x["Q"][0, 0][rows]), k, v, to_f64(x["G"][0, 0][rows]))
    e = rel_err(to_f64(O[0, 0][rows]), ref)
    say(f"  linear N=2^23 d=64: {rows.size} rows, max rel err {e:.2e}")
    assert e < TOL["bf16"]
    del O
    say("  anchor N=2^23 d=64 (about 15 s on the GPU)")
    _check_anchor_lse(x, k, v, rows, "bf16", "anchor N=2^23 d=64")


BWD_N = 1 << 22


def _sum_rows_f64(t, chunk=1 << 20):
    """Column sums of a [N, d] device tensor, widened exactly to float64."""
    return sum(to_f64(t[r:r + chunk]).sum(axis=0) for r in range(0, t.shape[0], chunk))


@pytest.mark.timeout(300)
def test_anchor_backward_at_4m():
    w = dataclasses.replace(get("720p5s"), name="bwd4m", H=1, N=BWD_N)
    say(f"backward inputs: B=1 H=1 N={BWD_N} d=128 bf16")
    x = layer_inputs_device(w, 3, "cuda")
    gen = torch.Generator(device="cuda").manual_seed(31)
    dO = torch.randn((1, 1, BWD_N, w.d), generator=gen, device="cuda").to(torch.bfloat16)
    say("  anchor forward with lse and backward at N=2^22 (about 40 s on the GPU)")
    O, lse = ha.hybrid_attn_softmax_lse(x["Q"], x["K"], x["V"], x["G"])
    dQ, dK, dV, dG = ha.hybrid_attn_softmax_backward(x["Q"], x["K"], x["V"], x["G"], O, dO, lse)
    torch.cuda.synchronize()
    del O, lse
    # dQ, dG: exact on sampled query rows (a row's gradient needs its own row
    # and every key)
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(BWD_N - 8, BWD_N), rng.choice(BWD_N, 16, replace=False)]))
    k, v = to_f64(x["K"][0, 0]), to_f64(x["V"][0, 0])
    q, g, do = (to_f64(t[0, 0][rows]) for t in (x["Q"], x["G"], dO))
    rq, rg = oracle.softmax_attention_backward_rows(q, k, v, g, do, np.arange(rows.size))
    del k, v
    eq, eg = rel_err(to_f64(dQ[0, 0][rows]), rq), rel_err(to_f64(dG[0, 0][rows]), rg)
    say(f"  dQ, dG on {rows.size} rows: {eq:.2e}, {eg:.2e}")
    assert eq < TOL["bf16"] and eg < TOL["bf16"]
    # dV: every query's probabilities sum to one over the keys, so the key sum
    # of dV = P^T da is the query sum of da = dO * sigmoid(G).  Bound per
    # feature: the bf16 roundings of da, of each probability and of the lse
    # each move a term by at most 2^-9 of |da| (3 x 2^-9 sum |da|), the bf16
    # store of dV by 2^-9 sum |dV|; doubled for fp32 accumulation
    sd, sad = np.zeros(w.d), np.zeros(w.d)
    chunk = 1 << 20
    for r in range(0, BWD_N, chunk):
        da = to_f64(dO[0, 0][r:r + chunk]) * oracle.sigmoid(to_f64(x["G"][0, 0][r:r + chunk]))
        sd += da.sum(axis=0)
        sad += np.abs(da).sum(axis=0)
    sv = _sum_rows_f64(dV[0, 0])
    sav = sum(np.abs(to_f64(dV[0, 0][r:r + chunk])).sum(axis=0) for r in range(0, BWD_N, chunk))
    ev = np.abs(sv - sd)
    bound = 2.0 * (3 * 2.0 ** -9 * sad + 2.0 ** -9 * sav)
    say(f"  dV key sum vs da query sum: max {ev.max():.3e} (bound {bound.min():.3e})")
    assert np.all(ev <= bound)
    # dK: a common shift of every key leaves the anchor unchanged, so the key
    # gradients sum to zero (relative to their total size)
    sk = _sum_rows_f64(dK[0, 0])
    sak = sum(np.abs(to_f64(dK[0, 0][r:r + chunk])).sum(axis=0) for r in range(0, BWD_N, chunk))
    say(f"  dK key sum: {np.abs(sk).max():.3e} of {sak.max():.3e}")
    assert np.abs(sk).max() < 2e-2 * sak.max()
    for t in (dQ, dK, dV, dG):
        assert torch.isfinite(t).all()
