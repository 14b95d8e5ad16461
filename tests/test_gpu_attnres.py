"""AttnRes parity: the mixture kernel and the routed block / stack against the
float64 AttnRes oracle (pinned on the CPU) on the same seeded inputs."""
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


def _dt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _rand(shape, seed, dtype, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(_dt(dtype)).to(DEV)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [0, 1, 3])
@pytest.mark.parametrize("B,N,C", [(1, 1, 128), (2, 300, 192), (1, 777, 3072), (1, 97, 5120), (1, 33, 6400)])
def test_mix_parity(dtype, M, B, N, C):
    # bf16 rows of up to 6,144 features take the single-pass kernel (1 to 12
    # 16-byte chunks per lane: C = 128 and 192 leave lanes idle, 5,120 uses 10),
    # 6,400 the two-pass one, as does float32
    say(f"attnres mix {dtype} M={M} B={B} N={N} C={C}")
    x = _rand((B, N, C), 1, dtype)
    S = _rand((M, B, N, C), 2, dtype, scale=2.0) if M else None
    w = _rand((C,), 3, "f32")
    h = ha.hybrid_attn_attnres_mix(S, x, w)
    torch.cuda.synchronize()
    cands = np.concatenate([to_f64(S), to_f64(x)[None]]) if M else to_f64(x)[None]
    ref = oracle.attnres_mix(cands, to_f64(w))
    e = rel_err(to_f64(h), ref)
    say(f"  max rel err {e:.2e}")
    assert e < TOL[dtype], e
    if M == 0:
        assert torch.equal(h, x)        # one candidate: weight exactly 1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mix_most_candidates(dtype):
    M, B, N, C = 63, 1, 50, 256           # the largest number of summaries
    say(f"attnres mix {dtype} M={M} C={C}")
    x = _rand((B, N, C), 5, dtype)
    S = _rand((M, B, N, C), 6, dtype, scale=2.0)
    w = _rand((C,), 7, "f32", scale=4.0)   # peaked weights: the running maximum moves
    h = ha.hybrid_attn_attnres_mix(S, x, w)
    torch.cuda.synchronize()
    ref = oracle.attnres_mix(np.concatenate([to_f64(S), to_f64(x)[None]]), to_f64(w))
    e = rel_err(to_f64(h), ref)
    say(f"  max rel err {e:.2e}")
    assert e < TOL[dtype], e


def _routed_inputs(dtype, d, B, N, H, nblocks, out_scale=3.0):
    base = get("tiny") if dtype == "f32" else get("480p")
    w = dataclasses.replace(base, d=d)
    ins = [block_inputs_host(dataclasses.replace(w, seed=k), B=B, N=N, H=H, d=d, device=DEV, out_scale=out_scale)
           for k in range(nblocks)]
    x = ins[0]["x"]
    W_in = torch.stack([t["W_in"] for t in ins]).contiguous()
    W_out = torch.stack([t["W_out"] for t in ins]).contiguous()
    g = torch.Generator(device="cpu").manual_seed(11)
    w_route = (torch.randn((nblocks, 4, H * d), generator=g) * 2.0).to(DEV)
    return x, W_in, W_out, w_route


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_routed_block_without_summaries_is_block(dtype, d):
    say(f"routed block M=0 vs block {dtype} d={d}")
    x, W_in, W_out, w_route = _routed_inputs(dtype, d, 1, 500, 2, 1)
    a = ha.hybrid_attn_block_routed(x, None, w_route[0], W_in[0], W_out[0], 2)
    b = ha.hybrid_attn_block(x, W_in[0], W_out[0], 2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_routed_stack_parity(dtype, d):
    B, N, H, nb = 1, 300, 2, 3
    C = H * d
    say(f"routed stack {dtype} d={d} N={N} H={H} blocks={nb}")
    # 12 sub-layers: with W_out at the fan-in scale the stream keeps its size
    # (larger output weights grow it layer by layer until a 2^-12 change of the
    # input moves the result by percents)
    x, W_in, W_out, w_route = _routed_inputs(dtype, d, B, N, H, nb, out_scale=1.0)
    summaries = torch.empty((nb, B, N, C), dtype=x.dtype, device=DEV)
    for k in range(nb):
        xin = x if k == 0 else summaries[k - 1]
        ha.hybrid_attn_block_routed(xin, summaries[:k] if k else None, w_route[k].contiguous(), W_in[k], W_out[k], H,
                                    x_out=summaries[k])
    torch.cuda.synchronize()
    store = oracle.round_bf16 if dtype == "bf16" else None
    ref = oracle.stack_routed(to_f64(x), to_f64(w_route), to_f64(W_in), to_f64(W_out), H, store=store)
    got = to_f64(summaries[nb - 1])
    x0 = to_f64(x)
    e, eu = rel_err(got, ref), rel_err(got - x0, ref - x0)
    say(f"  max rel err {e:.2e} (accumulated update {eu:.2e})")
    assert e < TOL[dtype], e
    # the update is ~0.25 |x|; 12 bf16 stores of the stream may each round half
    # an ulp (2^-9 |x|) differently on two correct paths: up to
    # sqrt(12) 2^-8 / 0.25 = 5.4e-2 of the update
    assert eu < (5.4e-2 if dtype == "bf16" else TOL[dtype]), eu


def test_mix_720p5s_sampled():
    w = get("720p5s")
    C = w.H * w.d
    say(f"attnres mix 720p5s N={w.N} C={C} M=3")
    x = block_inputs_device(w, DEV, layers=1)["x"]
    g = torch.Generator(device=DEV).manual_seed(8)
    S = torch.randn((3, w.B, w.N, C), generator=g, device=DEV).to(x.dtype)
    wr = torch.randn((C,), generator=g, device=DEV)
    h = ha.hybrid_attn_attnres_mix(S, x, wr)
    torch.cuda.synchronize()
    rows = sample_rows(w.N, n_rand=2048, seed=2)
    cands = np.concatenate([to_f64(S[:, :, rows]), to_f64(x[:, rows])[None]])
    ref = oracle.attnres_mix(cands, to_f64(wr))
    assert rel_err(to_f64(h[:, rows]), ref) < TOL["bf16"]
    del x, S, h
    torch.cuda.empty_cache()
