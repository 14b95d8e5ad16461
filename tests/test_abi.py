"""The C ABI on the host: the library loads, exports what the header declares,
and rejects bad arguments before any HIP call (no GPU is touched here)."""
import ctypes
import subprocess

import pytest

from hybrid_linear_softmax_amd import _lib

HA_BF16, HA_F32 = _lib.HA_BF16, _lib.HA_F32
OK, EINVAL, EUNSUP, EALIGN, EWS = _lib.HA_OK, _lib.HA_EINVAL, _lib.HA_EUNSUPPORTED, _lib.HA_EALIGN, _lib.HA_EWORKSPACE

# Fake, distinct, 256-byte aligned "device" addresses: validation only compares them.
GB = 1 << 30
Q, K, V, G, O, WS, S, Z, OFF, IDX = (GB * (i + 1) for i in range(10))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    declared = _lib.header_functions()
    assert set(declared) == set(_lib.SIGNATURES), declared
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing else leaks out of the library's own code
    assert {n for n in exported if n.startswith("hybrid_attn_")} == set(declared)


def test_strerror_and_schedule(lib):
    for code in (OK, EINVAL, EUNSUP, EALIGN, EWS, _lib.HA_EHIP, 12345):
        assert lib.hybrid_attn_strerror(code)
    kinds = (ctypes.c_int * 4)()
    assert lib.hybrid_attn_group_schedule(kinds) == OK
    assert list(kinds) == [0, 0, 0, 1]
    assert lib.hybrid_attn_group_schedule(None) == EINVAL


def test_workspace_is_pure_and_monotone(lib):
    w = lib.hybrid_attn_workspace_bytes
    assert w(1, 24, 75600, 128, HA_BF16) == w(1, 24, 75600, 128, HA_BF16)
    assert w(1, 24, 75600, 128, HA_BF16) > w(1, 24, 75600, 128, HA_F32) > 0
    assert w(2, 40, 75600, 128, HA_BF16) >= w(1, 40, 75600, 128, HA_BF16)
    assert w(0, 24, 100, 128, HA_BF16) == 0
    assert w(1, 24, 100, 96, HA_BF16) == 0
    assert w(1, 24, -1, 128, HA_BF16) == 0
    assert w(1, 1, 0, 64, HA_F32) > 0       # an empty sequence still has a (zero) state


def _linear(lib, q=Q, k=K, v=V, g=G, o=O, B=1, H=2, N=100, d=64, dt=HA_BF16, ws=WS, nb=None):
    if nb is None:
        nb = lib.hybrid_attn_workspace_bytes(B, H, N, d, dt) if B * H > 0 and d in (64, 128) else 0
    return lib.hybrid_attn_linear(q, k, v, g, o, B, H, N, d, dt, ws, nb, None)


def _softmax(lib, q=Q, k=K, v=V, g=G, o=O, B=1, H=2, N=100, d=64, dt=HA_BF16):
    return lib.hybrid_attn_softmax(q, k, v, g, o, B, H, N, d, dt, None)


def _softmax_bs(lib, q=Q, k=K, v=V, g=G, o=O, B=1, H=2, N=100, d=64, dt=HA_BF16, off=OFF, idx=IDX, n=7):
    return lib.hybrid_attn_softmax_blocksparse(q, k, v, g, o, B, H, N, d, dt, off, idx, n, None)


@pytest.mark.parametrize("call", [_linear, _softmax, _softmax_bs])
def test_argument_errors(lib, call):
    assert call(lib, d=96) == EUNSUP
    assert call(lib, d=0) == EUNSUP
    assert call(lib, dt=7) == EUNSUP
    assert call(lib, B=-1) == EINVAL
    assert call(lib, N=-5) == EINVAL
    assert call(lib, N=(1 << 23) + 1) == EINVAL
    assert call(lib, B=1 << 11, H=1 << 10) == EINVAL
    assert call(lib, q=None) == EINVAL
    assert call(lib, o=None) == EINVAL
    assert call(lib, v=V + 8) == EALIGN
    assert call(lib, o=O + 2) == EALIGN
    assert call(lib, o=Q) == EINVAL                 # output aliases an input
    assert call(lib, o=G + 64 * 16) == EINVAL       # output overlaps the tail of G
    # empty problems: nothing to do, success, even with null pointers
    assert call(lib, N=0, q=None, o=None) == OK
    assert call(lib, B=0) == OK
    assert call(lib, H=0) == OK


def test_workspace_errors(lib):
    need = lib.hybrid_attn_workspace_bytes(1, 2, 100, 64, HA_BF16)
    assert _linear(lib, ws=None) == EWS
    assert _linear(lib, nb=need - 1) == EWS
    assert _linear(lib, ws=WS + 4) == EALIGN
    st = lib.hybrid_attn_kv_state(K, V, S, Z, 1, 2, 100, 64, HA_BF16, WS, need - 1, None)
    assert st == EWS
    assert lib.hybrid_attn_kv_state(K, V, None, Z, 1, 2, 100, 64, HA_BF16, WS, need, None) == EINVAL
    assert lib.hybrid_attn_kv_state(K, V, S, S + 64, 1, 2, 100, 64, HA_BF16, WS, need, None) == EINVAL
    assert lib.hybrid_attn_kv_state(K, V, K, Z, 1, 2, 100, 64, HA_BF16, WS, need, None) == EINVAL
    # a workspace overlapping any tensor of the call is rejected (only rejected
    # calls here: a valid one would launch on the fake addresses)
    tensor = 1 * 2 * 100 * 64 * 2
    for t in (Q, K, V, G, O):
        assert _linear(lib, ws=t + 256) == EINVAL, t
        assert _linear(lib, ws=t - need + 256 if t - need + 256 > 0 else t) == EINVAL, t
    for t in (K, V, S, Z):
        assert lib.hybrid_attn_kv_state(K, V, S, Z, 1, 2, 100, 64, HA_BF16, t + 256, need, None) == EINVAL, t
    # the size check runs before the overlap check
    assert _linear(lib, ws=Q + 256, nb=need - 1) == EWS
    assert tensor < GB


def test_blocksparse_pattern_errors(lib):
    # (only rejected calls here: a valid one would launch on the fake addresses)
    assert _softmax_bs(lib, off=None) == EINVAL
    assert _softmax_bs(lib, idx=None) == EINVAL
    assert _softmax_bs(lib, n=-1) == EINVAL
    assert _softmax_bs(lib, n=1 << 31) == EINVAL
    assert _softmax_bs(lib, n=1 << 30) == EINVAL
    assert _softmax_bs(lib, off=OFF + 2) == EALIGN
    assert _softmax_bs(lib, idx=IDX + 1) == EALIGN
    assert _softmax_bs(lib, off=O + 64) == EINVAL         # the output may not overwrite the pattern
    assert _softmax_bs(lib, idx=O - 8, n=4) == EINVAL
    # the size checks run first: a bad head dimension wins over a bad pattern
    assert _softmax_bs(lib, d=96, off=None) == EUNSUP
    assert lib.hybrid_attn_softmax_blocksparse(Q, K, V, G, O, 1, 2, 0, 64, HA_BF16, None, None, 0, None) == OK


def test_group_errors(lib):
    args = (Q, K, V, G, O, 1, 2, 100, 64, HA_BF16)
    need = lib.hybrid_attn_workspace_bytes(1, 2, 100, 64, HA_BF16)
    assert lib.hybrid_attn_group(*args, WS, need - 1, None) == EWS
    # the group spans 4 layers: an output that overlaps layer 3 of an input is rejected
    layer_bytes = 1 * 2 * 100 * 64 * 2
    bad = (Q, K, V, G, G + 3 * layer_bytes, 1, 2, 100, 64, HA_BF16)
    assert lib.hybrid_attn_group(*bad, WS, need, None) == EINVAL
    evs = (ctypes.c_void_p * 5)(1, 2, None, 4, 5)
    assert lib.hybrid_attn_group_timed(*args, WS, need, None, evs) == EINVAL
    # the timed linear layer: a missing event array or entry, then the layer's own checks
    ev4 = (ctypes.c_void_p * 4)(1, 2, 3, None)
    assert lib.hybrid_attn_linear_timed(*args, WS, need, None, ev4) == EINVAL
    assert lib.hybrid_attn_linear_timed(*args, WS, need, None, None) == EINVAL
    ev4 = (ctypes.c_void_p * 4)(1, 2, 3, 4)
    assert lib.hybrid_attn_linear_timed(*args, WS, need - 1, None, ev4) == EWS
    assert lib.hybrid_attn_linear_timed(Q, K, V, G, O, 1, 2, 100, 80, HA_BF16, WS, need, None, ev4) == EUNSUP
    assert lib.hybrid_attn_group(Q, K, V, G, O, 1, 2, 100, 80, HA_BF16, WS, need, None) == EUNSUP
    # the workspace may not overlap any of the stacked tensors, layer 3 included
    assert lib.hybrid_attn_group(*args, O + 3 * layer_bytes, need, None) == EINVAL
    assert lib.hybrid_attn_group(*args, Q + 256, need, None) == EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_projection_errors(lib):
    # (only rejected calls: a valid one would launch on the fake addresses)
    def pin_(x=Q, w=K, q=O, k=S, v=Z, g=OFF, d=64, dt=HA_BF16, H=2):
        return lib.hybrid_attn_proj_in(x, w, q, k, v, g, 1, H, 100, d, dt, None)

    assert pin_(d=96) == EUNSUP and pin_(dt=7) == EUNSUP
    assert pin_(H=-1) == EINVAL
    assert pin_(x=None) == EINVAL and pin_(g=None) == EINVAL
    assert pin_(w=K + 8) == EALIGN and pin_(v=Z + 4) == EALIGN
    assert pin_(q=Q) == EINVAL                      # an output aliases x
    assert pin_(k=K + 4096) == EINVAL               # an output overlaps W_in
    assert pin_(k=O) == EINVAL                      # two outputs alias
    assert lib.hybrid_attn_proj_in(Q, K, O, S, Z, OFF, 1, 2, 0, 64, HA_BF16, None) == OK

    def pout(o=Q, w=K, x=V, xo=O, d=64):
        return lib.hybrid_attn_proj_out(o, w, x, xo, 1, 2, 100, d, HA_BF16, None)

    assert pout(d=80) == EUNSUP
    assert pout(o=None) == EINVAL and pout(xo=None) == EINVAL
    assert pout(xo=V + 64) == EINVAL                # overlaps x without being x
    assert pout(xo=Q + 16) == EINVAL                # overlaps O
    assert pout(w=K + 2) == EALIGN


def test_block_errors(lib):
    w = lib.hybrid_attn_block_workspace_bytes
    need = w(1, 2, 100, 64, HA_BF16)
    assert need > 5 * 100 * 128 * 2 and w(1, 2, 100, 64, HA_BF16) == need
    assert w(1, 2, 100, 96, HA_BF16) == 0 and w(0, 2, 100, 64, HA_BF16) == 0

    def blk(x=Q, wi=K, wo=V, xo=O, ws=WS, nb=need, d=64):
        return lib.hybrid_attn_block(x, wi, wo, xo, 1, 2, 100, d, HA_BF16, ws, nb, None)

    assert blk(d=32) == EUNSUP
    assert blk(wi=None) == EINVAL
    assert blk(xo=K + 128) == EINVAL                # output overlaps the input weights
    assert blk(ws=None) == EWS and blk(nb=need - 1) == EWS
    assert blk(ws=WS + 4) == EALIGN
    assert blk(ws=Q - 1024) == EINVAL               # workspace overlaps x
    assert blk(ws=O - 4096) == EINVAL               # workspace overlaps x_out
    assert lib.hybrid_attn_block(Q, K, V, O, 1, 2, 0, 64, HA_BF16, None, 0, None) == OK


def test_linear_backward_errors(lib):
    need = lib.hybrid_attn_linear_backward_workspace_bytes(1, 2, 100, 64, HA_BF16)
    assert need > 0 and lib.hybrid_attn_linear_backward_workspace_bytes(1, 2, 100, 96, HA_BF16) == 0
    DQ, DK, DV, DG, DO = (GB * (20 + i) for i in range(5))

    def bwd(q=Q, dq=DQ, dk=DK, do=DO, ws=WS, nb=need, d=64):
        return lib.hybrid_attn_linear_backward(q, K, V, G, do, dq, dk, DV, DG, 1, 2, 100, d, HA_BF16, ws, nb, None)

    assert bwd(d=80) == EUNSUP
    assert bwd(do=None) == EINVAL and bwd(dq=None) == EINVAL
    assert bwd(dq=Q) == EINVAL                     # a gradient aliases an input
    assert bwd(dk=DQ + 64) == EINVAL               # two gradients overlap
    assert bwd(do=DO + 4) == EALIGN
    assert bwd(ws=None) == EWS and bwd(nb=need - 1) == EWS
    assert bwd(ws=DG - 512) == EINVAL              # workspace overlaps a gradient
    assert lib.hybrid_attn_linear_backward(Q, K, V, G, DO, DQ, DK, DV, DG, 1, 2, 0, 64, HA_BF16,
                                           None, 0, None) == OK


def test_softmax_lse_and_backward_errors(lib):
    LSE, DQ, DK, DV, DG, DO = (GB * (30 + i) for i in range(6))
    assert lib.hybrid_attn_softmax_lse(Q, K, V, G, O, None, 1, 2, 100, 64, HA_BF16, None) == EINVAL
    assert lib.hybrid_attn_softmax_lse(Q, K, V, G, O, LSE + 2, 1, 2, 100, 64, HA_BF16, None) == EALIGN
    assert lib.hybrid_attn_softmax_lse(Q, K, V, G, O, O + 64, 1, 2, 100, 64, HA_BF16, None) == EINVAL
    need = lib.hybrid_attn_softmax_backward_workspace_bytes(1, 2, 100, 64, HA_BF16)
    assert need >= 1 * 2 * 100 * (64 * 2 + 4)

    def bwd(o=O, lse=LSE, dq=DQ, ws=WS, nb=need, d=64):
        return lib.hybrid_attn_softmax_backward(Q, K, V, G, o, DO, lse, dq, DK, DV, DG, 1, 2, 100, d, HA_BF16,
                                                ws, nb, None)

    assert bwd(d=96) == EUNSUP
    assert bwd(lse=None) == EINVAL and bwd(o=None) == EINVAL
    assert bwd(dq=LSE) == EINVAL                   # a gradient overlaps lse
    assert bwd(ws=None) == EWS and bwd(nb=need - 1) == EWS
    assert bwd(ws=LSE - 64) == EINVAL              # workspace overlaps lse


def test_attnres_errors(lib):
    X, Hh, W, SUM = GB * 40, GB * 41, GB * 42, GB * 43
    mix = lib.hybrid_attn_attnres_mix
    assert mix(SUM, 2, X, W, Hh, 1, 100, 100, HA_BF16, None) == EUNSUP      # C not a multiple of 8
    assert mix(SUM, 2, X, W, Hh, 1, 100, 128, 9, None) == EUNSUP
    assert mix(SUM, 64, X, W, Hh, 1, 100, 128, HA_BF16, None) == EINVAL     # too many summaries
    assert mix(None, 2, X, W, Hh, 1, 100, 128, HA_BF16, None) == EINVAL
    assert mix(SUM, 2, X, W + 4, Hh, 1, 100, 128, HA_BF16, None) == EALIGN
    assert mix(SUM, 2, X, W, X + 256, 1, 100, 128, HA_BF16, None) == EINVAL  # h overlaps x
    assert mix(SUM, 2, X, W, SUM + 256, 1, 100, 128, HA_BF16, None) == EINVAL
    assert mix(None, 0, X, W, Hh, 1, 0, 128, HA_BF16, None) == OK
    need = lib.hybrid_attn_block_routed_workspace_bytes(1, 2, 100, 64, HA_BF16)
    assert need > lib.hybrid_attn_block_workspace_bytes(1, 2, 100, 64, HA_BF16)
    tb = 100 * 128 * 2

    def blk(x=X, s=SUM, m=2, xo=Hh, ws=WS, nb=need):
        return lib.hybrid_attn_block_routed(x, s, m, W, Q, K, xo, 1, 2, 100, 64, HA_BF16, ws, nb, None)

    assert blk(m=64) == EINVAL and blk(s=None) == EINVAL
    assert blk(xo=SUM + tb) == EINVAL               # output inside the summaries
    assert blk(ws=None) == EWS and blk(nb=need - 1) == EWS
    assert blk(ws=SUM - 512) == EINVAL


def test_binding_rejects_host_tensors():
    import torch
    import hybrid_linear_softmax_amd as ha
    t = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        ha.hybrid_attn_softmax(t, t, t, t)
    with pytest.raises(ValueError, match="device tensor"):
        ha.hybrid_attn_linear(t, t, t, t)
    with pytest.raises(ValueError, match="device tensor"):
        ha.hybrid_attn_proj_in(torch.zeros((1, 8, 128), dtype=torch.bfloat16), torch.zeros((512, 128)), 2)


def test_probe_errors(lib):
    SRC, DST, SINK = GB * 50, GB * 51, GB * 52
    flops = lib.hybrid_attn_probe_mfma_flops
    assert flops(1, 1) == 4 * 4 * 2 * 32 * 32 * 16
    assert flops(2048, 65536) == 2048 * 65536 * flops(1, 1)
    assert flops(0, 1) == 0.0 and flops(1, 0) == 0.0 and flops(1 << 21, 1) == 0.0 and flops(1, (1 << 24) + 1) == 0.0
    mfma = lib.hybrid_attn_probe_mfma
    assert mfma(0, 1, SINK, None) == EINVAL and mfma(1, 0, SINK, None) == EINVAL
    assert mfma((1 << 20) + 1, 1, SINK, None) == EINVAL and mfma(1, 1, None, None) == EINVAL
    data = lib.hybrid_attn_probe_mfma_data
    assert data(0, 1, SINK, None) == EINVAL and data(1, 0, SINK, None) == EINVAL
    assert data(1, (1 << 24) + 1, SINK, None) == EINVAL and data(1, 1, None, None) == EINVAL
    read = lib.hybrid_attn_probe_read
    assert read(None, 1024, SINK, None) == EINVAL and read(SRC, 1024, None, None) == EINVAL
    assert read(SRC + 8, 1024, SINK, None) == EALIGN and read(SRC, 1000, SINK, None) == EALIGN
    assert read(SRC, 0, SINK, None) == OK                      # nothing enqueued
    copy = lib.hybrid_attn_probe_copy
    assert copy(None, DST, 1024, 0, None) == EINVAL and copy(SRC, None, 1024, 0, None) == EINVAL
    assert copy(SRC, SRC + 512, 1024, 0, None) == EINVAL       # ranges overlap
    assert copy(SRC, DST + 8, 1024, 1, None) == EALIGN and copy(SRC, DST, 1000, 0, None) == EALIGN
    assert copy(SRC, DST, 0, 0, None) == OK
    ov = lib.hybrid_attn_probe_overlap
    assert ov(0, 2, 1, 1, None, None) == EINVAL                # no sink
    assert ov(-1, 2, 1, 1, SINK, None) == EINVAL and ov(4, 2, 1, 1, SINK, None) == EINVAL   # unknown modes
    assert ov(0, 0, 1, 1, SINK, None) == EINVAL and ov(0, 3, 1, 1, SINK, None) == EINVAL    # 1 or 2 waves per SIMD
    assert ov(3, 1, 1, 1, SINK, None) == EINVAL                # the split needs two waves per SIMD
    assert ov(0, 1, 0, 1, SINK, None) == EINVAL and ov(0, 1, 1, 0, SINK, None) == EINVAL
    assert ov(0, 1, (1 << 20) + 1, 1, SINK, None) == EINVAL and ov(0, 1, 1, (1 << 24) + 1, SINK, None) == EINVAL


def test_noalloc_group_limits(lib):
    """The scratch-array group rejects problems whose workspace exceeds the
    array before touching the device, and gives the group's own status to
    invalid or empty problems (nothing to launch)."""
    na = lib.hybrid_attn_group_noalloc
    limit = 64 << 20
    big = (1, 4096, 1000, 128)                      # one chunk per head: 4096 partial states
    assert lib.hybrid_attn_workspace_bytes(*big, HA_BF16) > limit
    assert na(Q, K, V, G, O, *big, HA_BF16, None) == EWS
    assert lib.hybrid_attn_workspace_bytes(1, 24, 75600, 128, HA_BF16) <= limit   # the 720p/5s shape fits
    assert lib.hybrid_attn_workspace_bytes(2, 40, 75600, 128, HA_BF16) <= limit   # and the 14B batch
    assert na(Q, K, V, G, O, 1, 2, 100, 96, HA_BF16, None) == EUNSUP
    assert na(Q, K, V, G, O, 1, 2, -1, 64, HA_BF16, None) == EINVAL
    assert na(Q, K, V, G, O, 1, 2, 100, 64, 7, None) == EUNSUP
    assert na(Q, K, V, G, O, 1, 2, 0, 64, HA_BF16, None) == OK      # empty sequence
    assert na(Q, K, V, G, O, 0, 2, 100, 64, HA_BF16, None) == OK    # no heads
