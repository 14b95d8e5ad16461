"""MI355X (gfx950) Hybrid Linear-Softmax Attention: Python binding of
libhybrid_attn.so.

The functions below only marshal torch tensors (device memory) and the current
HIP stream into the C ABI of include/hybrid_attn.h (and the measurement probes
of include/ha_probe.h); every step of the
computation runs in the library's HIP kernels.  Outputs and the workspace are
allocated with torch when the caller does not pass them.
"""
import contextlib
import ctypes
import functools
import inspect

import torch

from . import _lib
from ._lib import HA_BF16, HA_F32  # noqa: F401

__all__ = [
    "HybridAttnError",
    "workspace_bytes",
    "hybrid_attn_kv_state",
    "hybrid_attn_linear",
    "hybrid_attn_softmax",
    "hybrid_attn_softmax_blocksparse",
    "SPARSE_BLOCK_Q",
    "SPARSE_BLOCK_K",
    "hybrid_attn_group",
    "hybrid_attn_group_schedule",
    "hybrid_attn_group_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "hybrid_attn_linear_backward",
    "hybrid_attn_softmax_lse",
    "hybrid_attn_softmax_backward",
    "softmax_backward_workspace_bytes",
    "linear_backward_workspace_bytes",
    "hybrid_attn_attnres_mix",
    "hybrid_attn_block_routed",
    "block_routed_workspace_bytes",
    "hybrid_attn_proj_in",
    "hybrid_attn_proj_out",
    "hybrid_attn_block",
    "block_workspace_bytes",
    "probe_mfma",
    "probe_mfma_data",
    "probe_read",
    "probe_copy",
    "probe_overlap",
    "PROBE_OVERLAP_MODES",
    "LAYER_KINDS",
]

LAYER_KINDS = {0: "linear", 1: "softmax"}
SPARSE_BLOCK_Q, SPARSE_BLOCK_K = 256, 64   # HA_SPARSE_BLOCK_Q / HA_SPARSE_BLOCK_K
NOALLOC_SCRATCH_BYTES = 64 << 20           # HA_NOALLOC_SCRATCH_BYTES
_DTYPES = {torch.bfloat16: HA_BF16, torch.float32: HA_F32}


class HybridAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.load().hybrid_attn_strerror(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def _check(status: int, where: str):
    if status != 0:
        raise HybridAttnError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32") from None


def _on_current_device(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the library launches on the current device "
                         f"cuda:{torch.cuda.current_device()}")


def _tensors(names, tensors, ndim):
    ref = tensors[0]
    for n, t in zip(names, tensors):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
        _on_current_device(n, t)
        if t.dim() != ndim or t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{n}: expected shape {tuple(ref.shape)} / dtype {ref.dtype}, "
                             f"got {tuple(t.shape)} / {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    return ref


def _like(name, t, shape, dtype, device):
    """A caller-supplied tensor: a contiguous `shape` / `dtype` tensor on `device`
    (the kernels write or read exactly that many elements)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device or tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {tuple(shape)} {dtype} tensor on {device}, got "
                         f"{tuple(t.shape)} {t.dtype} on {t.device}{'' if t.is_contiguous() else ', not contiguous'}")
    return t


def _out(name, t, shape, dtype, device):
    """An output: allocated when the caller passes None, else checked by _like."""
    if t is None:
        return torch.empty(tuple(shape), dtype=dtype, device=device)
    return _like(name, t, shape, dtype, device)


def _ws_tensor(workspace, need, device):
    """The workspace: allocated when the caller passes None, else a contiguous
    tensor on `device` (its byte size is checked by the library)."""
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return workspace


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run an entry point with `stream` (when given) as torch's current stream,
    so that every output or workspace it allocates belongs to the stream its
    kernels run on: the caching allocator then reuses a freed workspace only
    for work ordered after those kernels."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind(*args, **kwargs).arguments.get("stream")
        ctx = contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)
        with ctx:
            return fn(*args, **kwargs)
    return wrapper


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_workspace_bytes(B, H, N, d, code))


def _workspace(B, H, N, d, dtype, device, workspace):
    workspace = _ws_tensor(workspace, workspace_bytes(B, H, N, d, dtype), device)
    return workspace, workspace.numel() * workspace.element_size()


@_on_stream
def hybrid_attn_kv_state(K, V, S=None, z=None, workspace=None, stream=None):
    """Float32 state S [B, H, d, d] and normaliser z [B, H, d] of K, V [B, H, N, d]."""
    ref = _tensors(("K", "V"), (K, V), 4)
    B, H, N, d = ref.shape
    S = _out("S", S, (B, H, d, d), torch.float32, ref.device)
    z = _out("z", z, (B, H, d), torch.float32, ref.device)
    ws, nbytes = _workspace(B, H, N, d, ref.dtype, ref.device, workspace)
    _check(_lib.load().hybrid_attn_kv_state(_ptr(K), _ptr(V), _ptr(S), _ptr(z), B, H, N, d,
                                            _dtype_code(ref), _ptr(ws), nbytes, _stream(stream)),
           "hybrid_attn_kv_state")
    return S, z


@_on_stream
def hybrid_attn_linear(Q, K, V, G, O=None, workspace=None, stream=None, events=None):
    """One gated linear-attention layer; Q, K, V, G, O: [B, H, N, d].  `events`:
    an optional list of four torch.cuda.Event(enable_timing=True), recorded
    before pass 1 of the state reduction, after it, after pass 2 and after the
    apply."""
    ref = _tensors(("Q", "K", "V", "G"), (Q, K, V, G), 4)
    B, H, N, d = ref.shape
    O = _out("O", O, ref.shape, ref.dtype, ref.device)
    ws, nbytes = _workspace(B, H, N, d, ref.dtype, ref.device, workspace)
    args = (_ptr(Q), _ptr(K), _ptr(V), _ptr(G), _ptr(O), B, H, N, d, _dtype_code(ref), _ptr(ws), nbytes,
            _stream(stream))
    if events is None:
        _check(_lib.load().hybrid_attn_linear(*args), "hybrid_attn_linear")
    else:
        _check(_lib.load().hybrid_attn_linear_timed(*args, _event_array(events, 4, stream)),
               "hybrid_attn_linear_timed")
    return O


def _event_array(events, n, stream):
    """A C array of the HIP events behind n torch.cuda.Event objects (created,
    when torch has not yet done so, by a first record on the call's stream)."""
    if len(events) != n:
        raise ValueError(f"events: {n} torch.cuda.Event objects expected")
    s = torch.cuda.current_stream() if stream is None else stream
    for e in events:
        if not e.cuda_event:
            e.record(s)
    return (ctypes.c_void_p * n)(*(e.cuda_event for e in events))


@_on_stream
def hybrid_attn_softmax(Q, K, V, G, O=None, stream=None):
    """One gated softmax anchor layer; Q, K, V, G, O: [B, H, N, d]."""
    ref = _tensors(("Q", "K", "V", "G"), (Q, K, V, G), 4)
    B, H, N, d = ref.shape
    O = _out("O", O, ref.shape, ref.dtype, ref.device)
    _check(_lib.load().hybrid_attn_softmax(_ptr(Q), _ptr(K), _ptr(V), _ptr(G), _ptr(O), B, H, N, d,
                                           _dtype_code(ref), _stream(stream)),
           "hybrid_attn_softmax")
    return O


@_on_stream
def hybrid_attn_softmax_blocksparse(Q, K, V, G, block_offsets, block_indices, O=None, stream=None):
    """Block-sparse gated softmax anchor; Q, K, V, G, O: [B, H, N, d].  The
    pattern is CSR over query blocks of SPARSE_BLOCK_Q rows: int32 device
    tensors block_offsets [ceil(N / SPARSE_BLOCK_Q) + 1] and block_indices
    (key blocks of SPARSE_BLOCK_K keys, distinct within a query block)."""
    ref = _tensors(("Q", "K", "V", "G"), (Q, K, V, G), 4)
    B, H, N, d = ref.shape
    nqb = -(-N // SPARSE_BLOCK_Q)
    for n, t in (("block_offsets", block_offsets), ("block_indices", block_indices)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1:
            raise ValueError(f"{n} must be a 1-d int32 tensor")
        if not t.is_contiguous() or t.device != ref.device:
            raise ValueError(f"{n} must be contiguous on {ref.device}")
    if block_offsets.numel() != nqb + 1:
        raise ValueError(f"block_offsets: {nqb + 1} entries expected for N={N}, got {block_offsets.numel()}")
    O = _out("O", O, ref.shape, ref.dtype, ref.device)
    n_idx = block_indices.numel()
    idx_ptr = _ptr(block_indices) if n_idx > 0 else ctypes.c_void_p(None)
    _check(_lib.load().hybrid_attn_softmax_blocksparse(_ptr(Q), _ptr(K), _ptr(V), _ptr(G), _ptr(O), B, H, N,
                                                       d, _dtype_code(ref), _ptr(block_offsets), idx_ptr,
                                                       n_idx, _stream(stream)),
           "hybrid_attn_softmax_blocksparse")
    return O


@_on_stream
def hybrid_attn_group(Q4, K4, V4, G4, O4=None, workspace=None, stream=None, events=None):
    """One 3:1 hybrid group over stacked [4, B, H, N, d] tensors.  `events`: an
    optional list of five torch.cuda.Event(enable_timing=True) recorded before
    layer 0 and after each layer."""
    ref = _tensors(("Q4", "K4", "V4", "G4"), (Q4, K4, V4, G4), 5)
    L, B, H, N, d = ref.shape
    if L != 4:
        raise ValueError(f"a group has 4 layers, got {L}")
    O4 = _out("O4", O4, ref.shape, ref.dtype, ref.device)
    ws, nbytes = _workspace(B, H, N, d, ref.dtype, ref.device, workspace)
    lib = _lib.load()
    args = (_ptr(Q4), _ptr(K4), _ptr(V4), _ptr(G4), _ptr(O4), B, H, N, d, _dtype_code(ref),
            _ptr(ws), nbytes, _stream(stream))
    if events is None:
        _check(lib.hybrid_attn_group(*args), "hybrid_attn_group")
    else:
        _check(lib.hybrid_attn_group_timed(*args, _event_array(events, 5, stream)), "hybrid_attn_group_timed")
    return O4


@_on_stream
def hybrid_attn_group_noalloc(Q4, K4, V4, G4, O4, stream=None):
    """hybrid_attn_group with the library's fixed device scratch array as the
    workspace: nothing is allocated, here or in the library (O4 is the caller's).
    Calls that overlap on one device share that array and must not be issued."""
    ref = _tensors(("Q4", "K4", "V4", "G4"), (Q4, K4, V4, G4), 5)
    L, B, H, N, d = ref.shape
    if L != 4:
        raise ValueError(f"a group has 4 layers, got {L}")
    _like("O4", O4, ref.shape, ref.dtype, ref.device)
    _check(_lib.load().hybrid_attn_group_noalloc(_ptr(Q4), _ptr(K4), _ptr(V4), _ptr(G4), _ptr(O4), B, H, N, d,
                                                 _dtype_code(ref), _stream(stream)),
           "hybrid_attn_group_noalloc")
    return O4


def hybrid_attn_group_schedule():
    """Layer kinds of a group, in order ("linear" or "softmax")."""
    kinds = (ctypes.c_int * 4)()
    _check(_lib.load().hybrid_attn_group_schedule(kinds), "hybrid_attn_group_schedule")
    return [LAYER_KINDS[k] for k in kinds]


def _check_weight(name, t, shape, ref):
    _like(name, t, shape, ref.dtype, ref.device)


def _block_dims(x, heads):
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, N, C] device tensor")
    _on_current_device("x", x)
    _dtype_code(x)
    B, N, C = x.shape
    if heads <= 0 or C % heads:
        raise ValueError(f"heads={heads} must divide C={C}")
    return B, N, C, C // heads


def block_workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_block_workspace_bytes(B, H, N, d, code))


@_on_stream
def hybrid_attn_proj_in(x, W_in, heads, Q=None, K=None, V=None, G=None, stream=None):
    """Q, K, V, G [B, H, N, d] = the four C-wide blocks of x W_in^T split into
    `heads` heads; x: [B, N, C], W_in: [4C, C]."""
    B, N, C, d = _block_dims(x, heads)
    _check_weight("W_in", W_in, (4 * C, C), x)
    outs = [_out(n, t, (B, heads, N, d), x.dtype, x.device) for n, t in zip("QKVG", (Q, K, V, G))]
    _check(_lib.load().hybrid_attn_proj_in(_ptr(x), _ptr(W_in), *(_ptr(t) for t in outs), B, heads, N, d,
                                           _dtype_code(x), _stream(stream)),
           "hybrid_attn_proj_in")
    return tuple(outs)


@_on_stream
def hybrid_attn_proj_out(O, W_out, x, x_out=None, stream=None):
    """x_out = x + concat_heads(O) W_out^T; O: [B, H, N, d], W_out: [C, C],
    x: [B, N, C].  Pass x_out=x to update x in place."""
    _tensors(("O",), (O,), 4)
    B, H, N, d = O.shape
    _block_dims(x, H)
    if tuple(x.shape) != (B, N, H * d) or x.dtype != O.dtype:
        raise ValueError(f"x: expected {(B, N, H * d)} / {O.dtype}, got {tuple(x.shape)} / {x.dtype}")
    _check_weight("W_out", W_out, (H * d, H * d), x)
    x_out = _out("x_out", x_out, x.shape, x.dtype, x.device)
    _check(_lib.load().hybrid_attn_proj_out(_ptr(O), _ptr(W_out), _ptr(x), _ptr(x_out), B, H, N, d,
                                            _dtype_code(x), _stream(stream)),
           "hybrid_attn_proj_out")
    return x_out


@_on_stream
def hybrid_attn_block(x, W_in4, W_out4, heads, x_out=None, workspace=None, stream=None):
    """The attention block: four sub-layers (linear, linear, linear, softmax),
    each x = x + concat_heads(layer(split(x W_in[l]^T))) W_out[l]^T.  x: [B, N, C],
    W_in4: [4, 4C, C], W_out4: [4, C, C].  Pass x_out=x to update in place."""
    B, N, C, d = _block_dims(x, heads)
    _check_weight("W_in4", W_in4, (4, 4 * C, C), x)
    _check_weight("W_out4", W_out4, (4, C, C), x)
    x_out = _out("x_out", x_out, x.shape, x.dtype, x.device)
    workspace = _ws_tensor(workspace, block_workspace_bytes(B, heads, N, d, x.dtype), x.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().hybrid_attn_block(_ptr(x), _ptr(W_in4), _ptr(W_out4), _ptr(x_out), B, heads, N, d,
                                         _dtype_code(x), _ptr(workspace), nbytes, _stream(stream)),
           "hybrid_attn_block")
    return x_out


def _grads(grads, ref):
    """The four gradient outputs dQ, dK, dV, dG, each shaped like `ref`."""
    if grads is None:
        return [torch.empty_like(ref) for _ in range(4)]
    grads = list(grads)
    if len(grads) != 4:
        raise ValueError("grads: four tensors (dQ, dK, dV, dG) expected")
    return [_like(n, t, ref.shape, ref.dtype, ref.device) for n, t in zip(("dQ", "dK", "dV", "dG"), grads)]


def linear_backward_workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_linear_backward_workspace_bytes(B, H, N, d, code))


@_on_stream
def hybrid_attn_linear_backward(Q, K, V, G, dO, grads=None, workspace=None, stream=None):
    """dQ, dK, dV, dG of the gated linear layer for the upstream gradient dO
    (all [B, H, N, d]).  `grads` may hold four preallocated output tensors."""
    ref = _tensors(("Q", "K", "V", "G", "dO"), (Q, K, V, G, dO), 4)
    B, H, N, d = ref.shape
    grads = _grads(grads, ref)
    workspace = _ws_tensor(workspace, linear_backward_workspace_bytes(B, H, N, d, ref.dtype), ref.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().hybrid_attn_linear_backward(*(_ptr(t) for t in (Q, K, V, G, dO)), *(_ptr(t) for t in grads),
                                                   B, H, N, d, _dtype_code(ref), _ptr(workspace), nbytes,
                                                   _stream(stream)),
           "hybrid_attn_linear_backward")
    return tuple(grads)


@_on_stream
def hybrid_attn_softmax_lse(Q, K, V, G, O=None, lse=None, stream=None):
    """The gated softmax anchor plus the per-row log-sum-exp (float32 [B, H, N]),
    the forward pass whose outputs hybrid_attn_softmax_backward consumes."""
    ref = _tensors(("Q", "K", "V", "G"), (Q, K, V, G), 4)
    B, H, N, d = ref.shape
    O = _out("O", O, ref.shape, ref.dtype, ref.device)
    lse = _out("lse", lse, (B, H, N), torch.float32, ref.device)
    _check(_lib.load().hybrid_attn_softmax_lse(_ptr(Q), _ptr(K), _ptr(V), _ptr(G), _ptr(O), _ptr(lse), B, H, N, d,
                                               _dtype_code(ref), _stream(stream)),
           "hybrid_attn_softmax_lse")
    return O, lse


def softmax_backward_workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_softmax_backward_workspace_bytes(B, H, N, d, code))


@_on_stream
def hybrid_attn_softmax_backward(Q, K, V, G, O, dO, lse, grads=None, workspace=None, stream=None):
    """dQ, dK, dV, dG of the gated softmax anchor; O and lse from
    hybrid_attn_softmax_lse."""
    ref = _tensors(("Q", "K", "V", "G", "O", "dO"), (Q, K, V, G, O, dO), 4)
    B, H, N, d = ref.shape
    _like("lse", lse, (B, H, N), torch.float32, ref.device)
    grads = _grads(grads, ref)
    workspace = _ws_tensor(workspace, softmax_backward_workspace_bytes(B, H, N, d, ref.dtype), ref.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().hybrid_attn_softmax_backward(*(_ptr(t) for t in (Q, K, V, G, O, dO, lse)),
                                                    *(_ptr(t) for t in grads), B, H, N, d, _dtype_code(ref),
                                                    _ptr(workspace), nbytes, _stream(stream)),
           "hybrid_attn_softmax_backward")
    return tuple(grads)


@_on_stream
def hybrid_attn_attnres_mix(summaries, x, w, h=None, stream=None):
    """AttnRes mixture h [B, N, C] over the candidates summaries [M, B, N, C]
    (M may be 0; pass None) and x, with routing vector w (float32 [C])."""
    B, N, C = _block_dims(x, 1)[:3]
    M = _summaries(summaries, x)
    _like("w", w, (C,), torch.float32, x.device)
    h = _out("h", h, x.shape, x.dtype, x.device)
    _check(_lib.load().hybrid_attn_attnres_mix(_ptr(summaries) if M else ctypes.c_void_p(None), M, _ptr(x), _ptr(w),
                                               _ptr(h), B, N, C, _dtype_code(x), _stream(stream)),
           "hybrid_attn_attnres_mix")
    return h


def _summaries(summaries, x):
    """Number of completed-block summaries: 0 for None, else M of a contiguous
    [M, B, N, C] tensor shaped and typed like x."""
    if summaries is None:
        return 0
    if not isinstance(summaries, torch.Tensor) or summaries.dim() != 4:
        raise ValueError("summaries must be an [M, B, N, C] tensor or None")
    M = summaries.shape[0]
    _like("summaries", summaries, (M, *x.shape), x.dtype, x.device)
    return M


def block_routed_workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_block_routed_workspace_bytes(B, H, N, d, code))


@_on_stream
def hybrid_attn_block_routed(x, summaries, w_route, W_in4, W_out4, heads, x_out=None, workspace=None, stream=None):
    """hybrid_attn_block with AttnRes routing of `summaries` ([M, B, N, C] or
    None) into the linear sub-layers; w_route float32 [4, C]."""
    B, N, C, d = _block_dims(x, heads)
    _check_weight("W_in4", W_in4, (4, 4 * C, C), x)
    _check_weight("W_out4", W_out4, (4, C, C), x)
    _like("w_route", w_route, (4, C), torch.float32, x.device)
    M = _summaries(summaries, x)
    x_out = _out("x_out", x_out, x.shape, x.dtype, x.device)
    workspace = _ws_tensor(workspace, block_routed_workspace_bytes(B, heads, N, d, x.dtype), x.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().hybrid_attn_block_routed(_ptr(x), _ptr(summaries) if M else ctypes.c_void_p(None), M,
                                                _ptr(w_route), _ptr(W_in4), _ptr(W_out4), _ptr(x_out), B, heads, N, d,
                                                _dtype_code(x), _ptr(workspace), nbytes, _stream(stream)),
           "hybrid_attn_block_routed")
    return x_out


def _stream_buffer(name, t):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    _on_current_device(name, t)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.numel() * t.element_size()


def _sink(sink):
    if sink is None:
        return torch.empty(1, dtype=torch.float32, device=torch.cuda.current_device())
    _like("sink", sink, (1,), torch.float32, torch.device("cuda", torch.cuda.current_device()))
    return sink


@_on_stream
def probe_mfma(blocks: int, iters: int, sink=None, stream=None) -> float:
    """Enqueue the MFMA throughput probe; returns the flop count it performs."""
    sink = _sink(sink)
    _check(_lib.load().hybrid_attn_probe_mfma(blocks, iters, _ptr(sink), _stream(stream)), "hybrid_attn_probe_mfma")
    return float(_lib.load().hybrid_attn_probe_mfma_flops(blocks, iters))


@_on_stream
def probe_mfma_data(blocks: int, iters: int, sink=None, stream=None) -> float:
    """Enqueue the MFMA probe on operands that change every instruction (random
    bf16); returns the flop count it performs."""
    sink = _sink(sink)
    _check(_lib.load().hybrid_attn_probe_mfma_data(blocks, iters, _ptr(sink), _stream(stream)),
           "hybrid_attn_probe_mfma_data")
    return float(_lib.load().hybrid_attn_probe_mfma_flops(blocks, iters))


PROBE_OVERLAP_MODES = {"mfma": 0, "valu": 1, "both": 2, "split": 3}


@_on_stream
def probe_overlap(mode: str, waves_per_simd: int, blocks: int, iters: int, sink=None, stream=None) -> dict:
    """Enqueue the issue-overlap probe (mode "mfma", "valu", "both" or "split");
    returns the work it performs: bf16 MFMA flops and VALU instructions."""
    if mode not in PROBE_OVERLAP_MODES:
        raise ValueError(f"mode must be one of {sorted(PROBE_OVERLAP_MODES)}")
    sink = _sink(sink)
    _check(_lib.load().hybrid_attn_probe_overlap(PROBE_OVERLAP_MODES[mode], waves_per_simd, blocks, iters,
                                                 _ptr(sink), _stream(stream)), "hybrid_attn_probe_overlap")
    waves = blocks * 4 * waves_per_simd
    mfma_waves = {"mfma": waves, "valu": 0, "both": waves, "split": waves // 2}[mode]
    valu_waves = {"mfma": 0, "valu": waves, "both": waves, "split": waves // 2}[mode]
    return {"mfma_flops": float(mfma_waves) * iters * 4 * 2 * 32 * 32 * 16,
            "valu_insts": float(valu_waves) * iters * 25}


@_on_stream
def probe_read(src, sink=None, stream=None) -> int:
    """Enqueue the HBM read probe over all of `src`; returns the bytes read."""
    nbytes = _stream_buffer("src", src)
    sink = _sink(sink)
    _check(_lib.load().hybrid_attn_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "hybrid_attn_probe_read")
    return nbytes


@_on_stream
def probe_copy(src, dst, nontemporal: bool = False, stream=None) -> int:
    """Enqueue the HBM copy probe src -> dst (same byte size); returns the bytes
    moved (read plus written)."""
    nbytes = _stream_buffer("src", src)
    if _stream_buffer("dst", dst) != nbytes:
        raise ValueError("src and dst must have the same byte size")
    _check(_lib.load().hybrid_attn_probe_copy(_ptr(src), _ptr(dst), nbytes, int(bool(nontemporal)), _stream(stream)),
           "hybrid_attn_probe_copy")
    return 2 * nbytes
