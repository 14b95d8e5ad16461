"""HIP graph capture of the library's entry points (through torch's graph
capture on its side stream): the library allocates nothing, records no memset
and enqueues everything on the caller's stream, so a captured call replays the
same kernels on the same buffers.  Each graph is replayed several times with
eager work and synchronisations between the replays; every replay must equal
the eager call bitwise, also after new values are copied into the captured
inputs (the graph reads live memory, it does not hold a snapshot)."""
import dataclasses

import pytest
import torch

import hybrid_linear_softmax_amd as ha
from gpu_util import say
from workloads import block_inputs_host, get, layer_inputs_host
from workloads.sparsity import random_pattern

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
B, H, N, D = 1, 2, 1000, 128


def _layer(seed_layer):
    w = dataclasses.replace(get("480p"), d=D)
    return layer_inputs_host(w, seed_layer, B=B, H=H, N=N, device=DEV)


def _replay_and_check(capture, run_eager, outputs, inputs, fresh):
    """capture(): the calls to record; run_eager(): the same calls eagerly;
    outputs: the tensors they write; inputs: the tensors they read; fresh():
    new values for the inputs (same shapes)."""
    run_eager()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(3):
        for o in outputs:
            o.fill_(float("nan"))       # eager work between the replays
        scratch.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w_ in zip(outputs, want):
            assert torch.equal(o, w_), f"replay {rep}"
    # new input values: the graph reads them, and matches the eager call on them
    for t, v in zip(inputs, fresh()):
        t.copy_(v)
    run_eager()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    for o in outputs:
        o.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    for o, w_ in zip(outputs, want):
        assert torch.equal(o, w_), "replay on new inputs"


def test_graph_group():
    say("graph: hybrid_attn_group")
    x = _layer(0)
    stacked = {n: torch.stack([x[n]] * 4).contiguous() for n in "QKVG"}
    O4 = torch.empty_like(stacked["Q"])
    ws = torch.empty(ha.workspace_bytes(B, H, N, D), dtype=torch.uint8, device=DEV)

    def call():
        ha.hybrid_attn_group(stacked["Q"], stacked["K"], stacked["V"], stacked["G"], O4, workspace=ws)

    def fresh():
        y = _layer(1)
        return [torch.stack([y[n]] * 4) for n in "QKVG"]

    _replay_and_check(call, call, [O4], [stacked[n] for n in "QKVG"], fresh)


def test_graph_layers_and_blocksparse():
    say("graph: linear, softmax, block-sparse anchor")
    x = _layer(2)
    O1, O2, O3 = (torch.empty_like(x["Q"]) for _ in range(3))
    ws = torch.empty(ha.workspace_bytes(B, H, N, D), dtype=torch.uint8, device=DEV)
    off, idx = random_pattern(N, keep=0.5, seed=3, empty_every=3, invalid=1, shuffle=True)
    off_d, idx_d = torch.from_numpy(off).to(DEV), torch.from_numpy(idx).to(DEV)

    def call():
        ha.hybrid_attn_linear(x["Q"], x["K"], x["V"], x["G"], O1, workspace=ws)
        ha.hybrid_attn_softmax(x["Q"], x["K"], x["V"], x["G"], O2)
        ha.hybrid_attn_softmax_blocksparse(x["Q"], x["K"], x["V"], x["G"], off_d, idx_d, O=O3)

    def fresh():
        y = _layer(3)
        return [y[n] for n in "QKVG"]

    _replay_and_check(call, call, [O1, O2, O3], [x[n] for n in "QKVG"], fresh)


def test_graph_backward():
    say("graph: forward with lse and both backward passes")
    x = _layer(4)
    g = torch.Generator(device=DEV).manual_seed(5)
    dO = torch.randn(x["Q"].shape, generator=g, device=DEV).to(x["Q"].dtype)
    O, lse = torch.empty_like(x["Q"]), torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    gl = [torch.empty_like(x["Q"]) for _ in range(4)]
    gs = [torch.empty_like(x["Q"]) for _ in range(4)]
    wl = torch.empty(ha.linear_backward_workspace_bytes(B, H, N, D), dtype=torch.uint8, device=DEV)
    wsm = torch.empty(ha.softmax_backward_workspace_bytes(B, H, N, D), dtype=torch.uint8, device=DEV)

    def call():
        ha.hybrid_attn_linear_backward(x["Q"], x["K"], x["V"], x["G"], dO, grads=gl, workspace=wl)
        ha.hybrid_attn_softmax_lse(x["Q"], x["K"], x["V"], x["G"], O, lse)
        ha.hybrid_attn_softmax_backward(x["Q"], x["K"], x["V"], x["G"], O, dO, lse, grads=gs, workspace=wsm)

    def fresh():
        y = _layer(6)
        return [y[n] for n in "QKVG"]

    _replay_and_check(call, call, [O, lse] + gl + gs, [x[n] for n in "QKVG"], fresh)


def test_graph_block_and_routed_block():
    say("graph: attention block and AttnRes-routed block")
    Hb, Nb, d = 2, 300, 64
    w = dataclasses.replace(get("480p"), d=d)
    t = block_inputs_host(w, B=1, N=Nb, H=Hb, d=d, device=DEV)
    C = Hb * d
    x_out1, x_out2 = torch.empty_like(t["x"]), torch.empty_like(t["x"])
    ws1 = torch.empty(ha.block_workspace_bytes(1, Hb, Nb, d, t["x"].dtype), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty(ha.block_routed_workspace_bytes(1, Hb, Nb, d, t["x"].dtype), dtype=torch.uint8, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(7)
    summ = torch.randn((2, 1, Nb, C), generator=gen, device=DEV).to(t["x"].dtype)
    w_route = torch.randn((4, C), generator=gen, device=DEV)

    def call():
        ha.hybrid_attn_block(t["x"], t["W_in"], t["W_out"], Hb, x_out=x_out1, workspace=ws1)
        ha.hybrid_attn_block_routed(t["x"], summ, w_route, t["W_in"], t["W_out"], Hb, x_out=x_out2, workspace=ws2)

    def fresh():
        return [t["x"].roll(7, dims=1) * 0.5, summ.flip(0)]

    _replay_and_check(call, call, [x_out1, x_out2], [t["x"], summ], fresh)
