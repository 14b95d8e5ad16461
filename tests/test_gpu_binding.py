"""The Python binding checks every tensor the caller supplies -- outputs,
gradients, summaries, workspaces -- against the shape, dtype and device the
kernels assume, and raises before anything is launched."""
import pytest
import torch

import hybrid_linear_softmax_amd as ha

pytestmark = pytest.mark.gpu

B, H, N, d = 1, 2, 96, 64


def _qkvg(dtype=torch.bfloat16, shape=(B, H, N, d)):
    g = torch.Generator(device="cuda").manual_seed(0)
    return [torch.randn(shape, generator=g, device="cuda").to(dtype) for _ in range(4)]


def test_layer_outputs_are_checked():
    Q, K, V, G = _qkvg()
    for fn in (ha.hybrid_attn_softmax, ha.hybrid_attn_linear):
        with pytest.raises(ValueError, match="O:"):
            fn(Q, K, V, G, torch.empty((B, H, N - 1, d), dtype=Q.dtype, device="cuda"))
        with pytest.raises(ValueError, match="O:"):
            fn(Q, K, V, G, torch.empty_like(Q, dtype=torch.float32))
        with pytest.raises(ValueError, match="O:"):
            fn(Q, K, V, G, torch.empty((B, H, d, N), dtype=Q.dtype, device="cuda").transpose(2, 3))
        with pytest.raises(ValueError, match="O:"):
            fn(Q, K, V, G, torch.empty_like(Q, device="cpu"))
    # a correct preallocated output is used as given
    O = torch.empty_like(Q)
    assert ha.hybrid_attn_softmax(Q, K, V, G, O) is O
    assert torch.equal(O, ha.hybrid_attn_softmax(Q, K, V, G))


def test_state_lse_and_gradients_are_checked():
    Q, K, V, G = _qkvg()
    with pytest.raises(ValueError, match="S:"):
        ha.hybrid_attn_kv_state(K, V, S=torch.empty((B, H, d, d - 1), device="cuda"))
    with pytest.raises(ValueError, match="z:"):
        ha.hybrid_attn_kv_state(K, V, z=torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="lse:"):
        ha.hybrid_attn_softmax_lse(Q, K, V, G, lse=torch.empty((B, H, N - 1), device="cuda"))
    O, lse = ha.hybrid_attn_softmax_lse(Q, K, V, G)
    dO = torch.randn_like(Q)
    with pytest.raises(ValueError, match="lse:"):
        ha.hybrid_attn_softmax_backward(Q, K, V, G, O, dO, lse[:, :, :-1])
    bad = [torch.empty_like(Q) for _ in range(3)] + [torch.empty((B, H, N // 2, d), dtype=Q.dtype, device="cuda")]
    with pytest.raises(ValueError, match="dG:"):
        ha.hybrid_attn_softmax_backward(Q, K, V, G, O, dO, lse, grads=bad)
    with pytest.raises(ValueError, match="dG:"):
        ha.hybrid_attn_linear_backward(Q, K, V, G, dO, grads=bad)
    with pytest.raises(ValueError, match="four tensors"):
        ha.hybrid_attn_linear_backward(Q, K, V, G, dO, grads=bad[:3])


def test_workspaces_are_checked():
    Q, K, V, G = _qkvg()
    need = ha.workspace_bytes(B, H, N, d)
    with pytest.raises(ValueError, match="workspace"):
        ha.hybrid_attn_linear(Q, K, V, G, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace"):
        ha.hybrid_attn_linear(Q, K, V, G, workspace=torch.empty((2, need), dtype=torch.uint8, device="cuda")[:, 0])
    # too small: the library's own check
    with pytest.raises(ha.HybridAttnError):
        ha.hybrid_attn_linear(Q, K, V, G, workspace=torch.empty(need - 1, dtype=torch.uint8, device="cuda"))


def test_block_and_attnres_tensors_are_checked():
    C = H * d
    g = torch.Generator(device="cuda").manual_seed(1)
    x = torch.randn((B, N, C), generator=g, device="cuda").to(torch.bfloat16)
    W_in4 = torch.randn((4, 4 * C, C), generator=g, device="cuda").to(torch.bfloat16)
    W_out4 = torch.randn((4, C, C), generator=g, device="cuda").to(torch.bfloat16)
    w = torch.randn((4, C), generator=g, device="cuda")
    with pytest.raises(ValueError, match="x_out:"):
        ha.hybrid_attn_block(x, W_in4, W_out4, H, x_out=torch.empty((B, N - 1, C), dtype=x.dtype, device="cuda"))
    with pytest.raises(ValueError, match="W_in4:"):
        ha.hybrid_attn_block(x, W_in4[:, :-1], W_out4, H)
    with pytest.raises(ValueError, match="summaries:"):
        ha.hybrid_attn_block_routed(x, torch.empty((2, B, N - 1, C), dtype=x.dtype, device="cuda"), w, W_in4, W_out4, H)
    with pytest.raises(ValueError, match="w_route:"):
        ha.hybrid_attn_block_routed(x, None, w[:, :-1], W_in4, W_out4, H)
    with pytest.raises(ValueError, match="h:"):
        ha.hybrid_attn_attnres_mix(None, x, w[0], h=torch.empty((B, N, C + 1), dtype=x.dtype, device="cuda"))
    with pytest.raises(ValueError, match="w:"):
        ha.hybrid_attn_attnres_mix(None, x, w[0].to(torch.bfloat16))
    with pytest.raises(ValueError, match="Q:"):
        ha.hybrid_attn_proj_in(x, W_in4[0], H, Q=torch.empty((B, H, N, d + 1), dtype=x.dtype, device="cuda"))


def test_side_stream_allocations_belong_to_that_stream():
    """An entry point called with stream= allocates its workspace and outputs on
    that stream: a tensor allocated and filled on the current stream right after
    the call cannot take the workspace's memory while the side stream's kernels
    still use it, so the result equals the same call on the current stream."""
    n = 4096
    g = torch.Generator(device="cuda").manual_seed(2)
    Q, K, V, G = (torch.randn((1, 4, n, 128), generator=g, device="cuda").to(torch.bfloat16) for _ in range(4))
    ref_lin = ha.hybrid_attn_linear(Q, K, V, G)
    dO = torch.randn_like(Q)
    ref_bwd = ha.hybrid_attn_linear_backward(Q, K, V, G, dO)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        # a long kernel first keeps the side stream busy while the current
        # stream allocates and writes
        ha.hybrid_attn_softmax(Q, K, V, G, stream=side)
        out = ha.hybrid_attn_linear(Q, K, V, G, stream=side)
        grads = ha.hybrid_attn_linear_backward(Q, K, V, G, dO, stream=side)
        junk = [torch.full((1 << 22,), 7, dtype=torch.uint8, device="cuda") for _ in range(8)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        del junk
        assert torch.equal(out, ref_lin)
        for a, b in zip(grads, ref_bwd):
            assert torch.equal(a, b)
