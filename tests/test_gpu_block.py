"""Attention-block parity: the projection kernels and the block entry point
against the float64 block oracle on the same seeded inputs -- both dtypes and
head sizes, ragged token and feature tiles, in-place updates, the block as the
bitwise composition of its stages, and sampled rows at the 720p / 5 s shape."""
import dataclasses

import numpy as np
import pytest
import torch

import hybrid_linear_softmax_amd as ha
import oracle
from gpu_util import TOL, rel_err, sample_rows, say
from workloads import block_inputs_device, block_inputs_host, get, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
VARIANTS = [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)]
# (B, N, H): single token, ragged token tiles, C below one 256-feature tile
SHAPES = [(1, 1, 2), (2, 300, 2), (1, 1000, 3), (2, 517, 1)]


def _w(dtype, d):
    base = get("tiny") if dtype == "f32" else get("480p")
    return dataclasses.replace(base, d=d)


def _inputs(dtype, d, B, N, H, out_scale=1.0):
    return block_inputs_host(_w(dtype, d), B=B, N=N, H=H, d=d, device=DEV, out_scale=out_scale)


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("B,N,H", SHAPES)
def test_proj_in_parity(dtype, d, B, N, H):
    say(f"proj_in {dtype} d={d} B={B} N={N} H={H}")
    t = _inputs(dtype, d, B, N, H)
    got = ha.hybrid_attn_proj_in(t["x"], t["W_in"][1], H)
    torch.cuda.synchronize()
    ref = oracle.project_in(to_f64(t["x"]), to_f64(t["W_in"][1]), H)
    for name, g, r in zip("QKVG", got, ref):
        e = rel_err(to_f64(g), r)
        assert e < TOL[dtype], (name, e)
    say(f"  max rel err {max(rel_err(to_f64(g), r) for g, r in zip(got, ref)):.2e}")


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("B,N,H", SHAPES)
@pytest.mark.parametrize("in_place", [False, True])
def test_proj_out_parity(dtype, d, B, N, H, in_place):
    say(f"proj_out {dtype} d={d} B={B} N={N} H={H} in_place={in_place}")
    t = _inputs(dtype, d, B, N, H, out_scale=4.0)
    gen = torch.Generator(device="cpu").manual_seed(N + H)
    O = torch.randn((B, H, N, d), generator=gen).to(t["x"].dtype).to(DEV)
    x = t["x"].clone()
    ref = oracle.project_out(to_f64(O), to_f64(t["W_out"][2]), to_f64(x))
    out = ha.hybrid_attn_proj_out(O, t["W_out"][2], x, x_out=x if in_place else None)
    torch.cuda.synchronize()
    if in_place:
        assert out.data_ptr() == x.data_ptr()
    e = rel_err(to_f64(out), ref)
    say(f"  max rel err {e:.2e}")
    assert e < TOL[dtype], e


@pytest.mark.parametrize("dtype,d", VARIANTS)
@pytest.mark.parametrize("B,N,H", [(1, 200, 2), (2, 300, 1)])
def test_block_parity(dtype, d, B, N, H):
    say(f"block {dtype} d={d} B={B} N={N} H={H}")
    # out_scale 3 gives each sub-layer's update about the size of x, so the
    # check sees the attention and not only the residual; much larger weights
    # grow the stream layer by layer until the anchor's logits are large and
    # the result is ill-conditioned (a 1-ulp change of Q moves it by percents)
    t = _inputs(dtype, d, B, N, H, out_scale=3.0)
    out = ha.hybrid_attn_block(t["x"], t["W_in"], t["W_out"], H)
    torch.cuda.synchronize()
    x0, Wi, Wo = to_f64(t["x"]), to_f64(t["W_in"]), to_f64(t["W_out"])
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    exact = oracle.block(x0, Wi, Wo, H)
    if dtype == "bf16":
        # the path stores Q, K, V, G, O and the stream in bf16 between its 12
        # stages: the parity reference is the oracle with that storage
        ref = oracle.block(x0, Wi, Wo, H, store=oracle.round_bf16)
    else:
        ref = exact
    e, eu = rel_err(got, ref), rel_err(got - x0, ref - x0)
    ex = rel_err(got, exact)
    say(f"  max rel err {e:.2e} (update alone {eu:.2e}); vs exact arithmetic and storage {ex:.2e}")
    assert e < TOL[dtype] and eu < TOL[dtype], (e, eu)
    # bf16 storage alone moves the exact result by about 5e-3 at these weights
    assert ex < TOL[dtype], ex


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_block_is_bitwise_composition_and_in_place(dtype, d):
    B, N, H = 1, 700, 2
    say(f"block composition {dtype} d={d} N={N} H={H}")
    t = _inputs(dtype, d, B, N, H, out_scale=3.0)
    blk = ha.hybrid_attn_block(t["x"], t["W_in"], t["W_out"], H)
    x = t["x"].clone()
    for l, kind in enumerate(ha.hybrid_attn_group_schedule()):
        Q, K, V, G = ha.hybrid_attn_proj_in(x, t["W_in"][l], H)
        fn = ha.hybrid_attn_linear if kind == "linear" else ha.hybrid_attn_softmax
        O = fn(Q, K, V, G)
        ha.hybrid_attn_proj_out(O, t["W_out"][l], x, x_out=x)
    inplace = t["x"].clone()
    ha.hybrid_attn_block(inplace, t["W_in"], t["W_out"], H, x_out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(blk, x)
    assert torch.equal(blk, inplace)
    again = ha.hybrid_attn_block(t["x"], t["W_in"], t["W_out"], H)
    torch.cuda.synchronize()
    assert torch.equal(blk, again)                  # deterministic


def test_720p5s_stages_sampled():
    w = get("720p5s")
    C = w.H * w.d
    say(f"block stages 720p5s: B={w.B} N={w.N} C={C}: generating inputs")
    t = block_inputs_device(w, DEV)
    rows = sample_rows(w.N, n_rand=256, seed=3)
    x = t["x"]
    Q, K, V, G = ha.hybrid_attn_proj_in(x, t["W_in"][0], w.H)
    torch.cuda.synchronize()
    xr = to_f64(x[:, rows])
    ref = oracle.project_in(xr, to_f64(t["W_in"][0]), w.H)
    for name, g, r in zip("QKVG", (Q, K, V, G), ref):
        e = rel_err(to_f64(g[:, :, rows]), r)
        assert e < TOL["bf16"], (name, e)
    say("  proj_in sampled rows ok")
    gen = torch.Generator(device=DEV).manual_seed(5)
    O = (torch.randn((w.B, w.H, w.N, w.d), generator=gen, device=DEV) * 0.05).to(x.dtype)
    x1 = ha.hybrid_attn_proj_out(O, t["W_out"][0], x)
    torch.cuda.synchronize()
    ref1 = oracle.project_out(to_f64(O[:, :, rows]), to_f64(t["W_out"][0]), xr)
    e = rel_err(to_f64(x1[:, rows]), ref1)
    e_upd = rel_err(to_f64(x1[:, rows]) - xr, ref1 - xr)
    say(f"  proj_out sampled rows: {e:.2e} (update {e_upd:.2e})")
    assert e < TOL["bf16"]
    # the whole block at full size: finite, and bitwise the composition of stages
    out = ha.hybrid_attn_block(x, t["W_in"], t["W_out"], w.H)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    y = x.clone()
    for l, kind in enumerate(ha.hybrid_attn_group_schedule()):
        Q, K, V, G = ha.hybrid_attn_proj_in(y, t["W_in"][l], w.H, Q, K, V, G)
        fn = ha.hybrid_attn_linear if kind == "linear" else ha.hybrid_attn_softmax
        fn(Q, K, V, G, O)
        ha.hybrid_attn_proj_out(O, t["W_out"][l], y, x_out=y)
    torch.cuda.synchronize()
    assert torch.equal(out, y)
    del t, Q, K, V, G, O, out, y
    torch.cuda.empty_cache()


def test_14b_b2_projections_sampled():
    # the widest shape of the workloads (C = 5120: 160 K steps of 32 per tile,
    # 80 feature tiles in proj_in), both batch items
    w = get("14b_b2")
    C = w.H * w.d
    say(f"projections 14b_b2: B={w.B} N={w.N} C={C}: generating inputs")
    t = block_inputs_device(w, DEV, layers=1)
    rows = sample_rows(w.N, n_rand=96, seed=4)
    x = t["x"]
    Q, K, V, G = ha.hybrid_attn_proj_in(x, t["W_in"][0], w.H)
    torch.cuda.synchronize()
    xr = to_f64(x[:, rows])
    ref = oracle.project_in(xr, to_f64(t["W_in"][0]), w.H)
    for name, g, r in zip("QKVG", (Q, K, V, G), ref):
        e = rel_err(to_f64(g[:, :, rows]), r)
        assert e < TOL["bf16"], (name, e)
    del K, V, G
    say("  proj_in sampled rows ok")
    gen = torch.Generator(device=DEV).manual_seed(6)
    O = (torch.randn((w.B, w.H, w.N, w.d), generator=gen, device=DEV) * 0.05).to(x.dtype)
    x1 = ha.hybrid_attn_proj_out(O, t["W_out"][0], x)
    torch.cuda.synchronize()
    ref1 = oracle.project_out(to_f64(O[:, :, rows]), to_f64(t["W_out"][0]), xr)
    e = rel_err(to_f64(x1[:, rows]), ref1)
    say(f"  proj_out sampled rows: {e:.2e}")
    assert e < TOL["bf16"]
    del t, Q, O, x1
    torch.cuda.empty_cache()


def test_proj_out_wide_sampled():
    # O of exactly 4 GiB (B = 1, N = 2^20, C = 2048): its byte offsets no longer
    # fit 32 bits, so proj_out loads its token rows through 64-bit lane
    # addresses; rows sampled across the tensor, the last one included
    B, N, H, d = 1, 1 << 20, 16, 128
    C = H * d
    say(f"proj_out with a 4 GiB O: B={B} N={N} C={C}")
    gen = torch.Generator(device=DEV).manual_seed(11)
    O = torch.randn((B, H, N, d), generator=gen, device=DEV, dtype=torch.bfloat16) * 0.05
    assert O.numel() * O.element_size() == 1 << 32
    x = torch.randn((B, N, C), generator=gen, device=DEV, dtype=torch.bfloat16)
    W = (torch.randn((C, C), generator=gen, device=DEV, dtype=torch.float32) / C ** 0.5).to(torch.bfloat16)
    x1 = ha.hybrid_attn_proj_out(O, W, x)
    torch.cuda.synchronize()
    rows = sample_rows(N, n_rand=48, seed=12)
    ref = oracle.project_out(to_f64(O[:, :, rows]), to_f64(W), to_f64(x[:, rows]))
    e = rel_err(to_f64(x1[:, rows]), ref)
    say(f"  sampled rows: {e:.2e}")
    assert e < TOL["bf16"]
    del O, x, W, x1
    torch.cuda.empty_cache()
