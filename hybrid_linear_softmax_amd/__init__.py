"""MI355X (gfx950) Hybrid Linear-Softmax Attention: Python binding of
libhybrid_attn.so.

The functions below only marshal torch tensors (device memory) and the current
HIP stream into the C ABI of include/hybrid_attn.h; every step of the
computation runs in the library's HIP kernels.  Outputs and the workspace are
allocated with torch when the caller does not pass them.
"""
import ctypes

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
    "LAYER_KINDS",
]

LAYER_KINDS = {0: "linear", 1: "softmax"}
SPARSE_BLOCK_Q, SPARSE_BLOCK_K = 256, 64   # HA_SPARSE_BLOCK_Q / HA_SPARSE_BLOCK_K
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


def _tensors(names, tensors, ndim):
    ref = tensors[0]
    for n, t in zip(names, tensors):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"{n} must be a device tensor")
        if t.dim() != ndim or t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{n}: expected shape {tuple(ref.shape)} / dtype {ref.dtype}, "
                             f"got {tuple(t.shape)} / {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    return ref


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_workspace_bytes(B, H, N, d, code))


def _workspace(B, H, N, d, dtype, device, workspace):
    need = workspace_bytes(B, H, N, d, dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def hybrid_attn_kv_state(K, V, S=None, z=None, workspace=None, stream=None):
    """Float32 state S [B, H, d, d] and normaliser z [B, H, d] of K, V [B, H, N, d]."""
    ref = _tensors(("K", "V"), (K, V), 4)
    B, H, N, d = ref.shape
    if S is None:
        S = torch.empty((B, H, d, d), dtype=torch.float32, device=ref.device)
    if z is None:
        z = torch.empty((B, H, d), dtype=torch.float32, device=ref.device)
    ws, nbytes = _workspace(B, H, N, d, ref.dtype, ref.device, workspace)
    _check(_lib.load().hybrid_attn_kv_state(_ptr(K), _ptr(V), _ptr(S), _ptr(z), B, H, N, d,
                                            _dtype_code(ref), _ptr(ws), nbytes, _stream(stream)),
           "hybrid_attn_kv_state")
    return S, z


def hybrid_attn_linear(Q, K, V, G, O=None, workspace=None, stream=None):
    """One gated linear-attention layer; Q, K, V, G, O: [B, H, N, d]."""
    ref = _tensors(("Q", "K", "V", "G"), (Q, K, V, G), 4)
    B, H, N, d = ref.shape
    O = torch.empty_like(ref) if O is None else O
    ws, nbytes = _workspace(B, H, N, d, ref.dtype, ref.device, workspace)
    _check(_lib.load().hybrid_attn_linear(_ptr(Q), _ptr(K), _ptr(V), _ptr(G), _ptr(O), B, H, N, d,
                                          _dtype_code(ref), _ptr(ws), nbytes, _stream(stream)),
           "hybrid_attn_linear")
    return O


def hybrid_attn_softmax(Q, K, V, G, O=None, stream=None):
    """One gated softmax anchor layer; Q, K, V, G, O: [B, H, N, d]."""
    ref = _tensors(("Q", "K", "V", "G"), (Q, K, V, G), 4)
    B, H, N, d = ref.shape
    O = torch.empty_like(ref) if O is None else O
    _check(_lib.load().hybrid_attn_softmax(_ptr(Q), _ptr(K), _ptr(V), _ptr(G), _ptr(O), B, H, N, d,
                                           _dtype_code(ref), _stream(stream)),
           "hybrid_attn_softmax")
    return O


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
    O = torch.empty_like(ref) if O is None else O
    n_idx = block_indices.numel()
    idx_ptr = _ptr(block_indices) if n_idx > 0 else ctypes.c_void_p(None)
    _check(_lib.load().hybrid_attn_softmax_blocksparse(_ptr(Q), _ptr(K), _ptr(V), _ptr(G), _ptr(O), B, H, N,
                                                       d, _dtype_code(ref), _ptr(block_offsets), idx_ptr,
                                                       n_idx, _stream(stream)),
           "hybrid_attn_softmax_blocksparse")
    return O


def hybrid_attn_group(Q4, K4, V4, G4, O4=None, workspace=None, stream=None, events=None):
    """One 3:1 hybrid group over stacked [4, B, H, N, d] tensors.  `events`: an
    optional list of five torch.cuda.Event(enable_timing=True) recorded before
    layer 0 and after each layer."""
    ref = _tensors(("Q4", "K4", "V4", "G4"), (Q4, K4, V4, G4), 5)
    L, B, H, N, d = ref.shape
    if L != 4:
        raise ValueError(f"a group has 4 layers, got {L}")
    O4 = torch.empty_like(ref) if O4 is None else O4
    ws, nbytes = _workspace(B, H, N, d, ref.dtype, ref.device, workspace)
    lib = _lib.load()
    args = (_ptr(Q4), _ptr(K4), _ptr(V4), _ptr(G4), _ptr(O4), B, H, N, d, _dtype_code(ref),
            _ptr(ws), nbytes, _stream(stream))
    if events is None:
        _check(lib.hybrid_attn_group(*args), "hybrid_attn_group")
    else:
        if len(events) != 5:
            raise ValueError("events: five torch.cuda.Event objects expected")
        s = torch.cuda.current_stream() if stream is None else stream
        for e in events:          # torch creates the underlying event on first record
            if not e.cuda_event:
                e.record(s)
        arr = (ctypes.c_void_p * 5)(*(e.cuda_event for e in events))
        _check(lib.hybrid_attn_group_timed(*args, arr), "hybrid_attn_group_timed")
    return O4


def hybrid_attn_group_schedule():
    """Layer kinds of a group, in order ("linear" or "softmax")."""
    kinds = (ctypes.c_int * 4)()
    _check(_lib.load().hybrid_attn_group_schedule(kinds), "hybrid_attn_group_schedule")
    return [LAYER_KINDS[k] for k in kinds]


def _check_weight(name, t, shape, ref):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != ref.dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {tuple(shape)} / {ref.dtype}, got {tuple(t.shape)} / {t.dtype}")


def _block_dims(x, heads):
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, N, C] device tensor")
    B, N, C = x.shape
    if heads <= 0 or C % heads:
        raise ValueError(f"heads={heads} must divide C={C}")
    return B, N, C, C // heads


def block_workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_block_workspace_bytes(B, H, N, d, code))


def hybrid_attn_proj_in(x, W_in, heads, Q=None, K=None, V=None, G=None, stream=None):
    """Q, K, V, G [B, H, N, d] = the four C-wide blocks of x W_in^T split into
    `heads` heads; x: [B, N, C], W_in: [4C, C]."""
    B, N, C, d = _block_dims(x, heads)
    _check_weight("W_in", W_in, (4 * C, C), x)
    outs = [torch.empty((B, heads, N, d), dtype=x.dtype, device=x.device) if t is None else t
            for t in (Q, K, V, G)]
    _tensors(("Q", "K", "V", "G"), outs, 4)
    _check(_lib.load().hybrid_attn_proj_in(_ptr(x), _ptr(W_in), *(_ptr(t) for t in outs), B, heads, N, d,
                                           _dtype_code(x), _stream(stream)),
           "hybrid_attn_proj_in")
    return tuple(outs)


def hybrid_attn_proj_out(O, W_out, x, x_out=None, stream=None):
    """x_out = x + concat_heads(O) W_out^T; O: [B, H, N, d], W_out: [C, C],
    x: [B, N, C].  Pass x_out=x to update x in place."""
    _tensors(("O",), (O,), 4)
    B, H, N, d = O.shape
    _block_dims(x, H)
    if tuple(x.shape) != (B, N, H * d) or x.dtype != O.dtype:
        raise ValueError(f"x: expected {(B, N, H * d)} / {O.dtype}, got {tuple(x.shape)} / {x.dtype}")
    _check_weight("W_out", W_out, (H * d, H * d), x)
    x_out = torch.empty_like(x) if x_out is None else x_out
    _check(_lib.load().hybrid_attn_proj_out(_ptr(O), _ptr(W_out), _ptr(x), _ptr(x_out), B, H, N, d,
                                            _dtype_code(x), _stream(stream)),
           "hybrid_attn_proj_out")
    return x_out


def hybrid_attn_block(x, W_in4, W_out4, heads, x_out=None, workspace=None, stream=None):
    """The attention block: four sub-layers (linear, linear, linear, softmax),
    each x = x + concat_heads(layer(split(x W_in[l]^T))) W_out[l]^T.  x: [B, N, C],
    W_in4: [4, 4C, C], W_out4: [4, C, C].  Pass x_out=x to update in place."""
    B, N, C, d = _block_dims(x, heads)
    _check_weight("W_in4", W_in4, (4, 4 * C, C), x)
    _check_weight("W_out4", W_out4, (4, C, C), x)
    x_out = torch.empty_like(x) if x_out is None else x_out
    need = block_workspace_bytes(B, heads, N, d, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().hybrid_attn_block(_ptr(x), _ptr(W_in4), _ptr(W_out4), _ptr(x_out), B, heads, N, d,
                                         _dtype_code(x), _ptr(workspace), nbytes, _stream(stream)),
           "hybrid_attn_block")
    return x_out


def linear_backward_workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_linear_backward_workspace_bytes(B, H, N, d, code))


def hybrid_attn_linear_backward(Q, K, V, G, dO, grads=None, workspace=None, stream=None):
    """dQ, dK, dV, dG of the gated linear layer for the upstream gradient dO
    (all [B, H, N, d]).  `grads` may hold four preallocated output tensors."""
    ref = _tensors(("Q", "K", "V", "G", "dO"), (Q, K, V, G, dO), 4)
    B, H, N, d = ref.shape
    grads = [torch.empty_like(ref) for _ in range(4)] if grads is None else list(grads)
    _tensors(("dQ", "dK", "dV", "dG"), grads, 4)
    need = linear_backward_workspace_bytes(B, H, N, d, ref.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=ref.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().hybrid_attn_linear_backward(*(_ptr(t) for t in (Q, K, V, G, dO)), *(_ptr(t) for t in grads),
                                                   B, H, N, d, _dtype_code(ref), _ptr(workspace), nbytes,
                                                   _stream(stream)),
           "hybrid_attn_linear_backward")
    return tuple(grads)


def hybrid_attn_softmax_lse(Q, K, V, G, O=None, lse=None, stream=None):
    """The gated softmax anchor plus the per-row log-sum-exp (float32 [B, H, N]),
    the forward pass whose outputs hybrid_attn_softmax_backward consumes."""
    ref = _tensors(("Q", "K", "V", "G"), (Q, K, V, G), 4)
    B, H, N, d = ref.shape
    O = torch.empty_like(ref) if O is None else O
    lse = torch.empty((B, H, N), dtype=torch.float32, device=ref.device) if lse is None else lse
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    _check(_lib.load().hybrid_attn_softmax_lse(_ptr(Q), _ptr(K), _ptr(V), _ptr(G), _ptr(O), _ptr(lse), B, H, N, d,
                                               _dtype_code(ref), _stream(stream)),
           "hybrid_attn_softmax_lse")
    return O, lse


def softmax_backward_workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_softmax_backward_workspace_bytes(B, H, N, d, code))


def hybrid_attn_softmax_backward(Q, K, V, G, O, dO, lse, grads=None, workspace=None, stream=None):
    """dQ, dK, dV, dG of the gated softmax anchor; O and lse from
    hybrid_attn_softmax_lse."""
    ref = _tensors(("Q", "K", "V", "G", "O", "dO"), (Q, K, V, G, O, dO), 4)
    B, H, N, d = ref.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    grads = [torch.empty_like(ref) for _ in range(4)] if grads is None else list(grads)
    _tensors(("dQ", "dK", "dV", "dG"), grads, 4)
    need = softmax_backward_workspace_bytes(B, H, N, d, ref.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=ref.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().hybrid_attn_softmax_backward(*(_ptr(t) for t in (Q, K, V, G, O, dO, lse)),
                                                    *(_ptr(t) for t in grads), B, H, N, d, _dtype_code(ref),
                                                    _ptr(workspace), nbytes, _stream(stream)),
           "hybrid_attn_softmax_backward")
    return tuple(grads)


def hybrid_attn_attnres_mix(summaries, x, w, h=None, stream=None):
    """AttnRes mixture h [B, N, C] over the candidates summaries [M, B, N, C]
    (M may be 0; pass None) and x, with routing vector w (float32 [C])."""
    B, N, C = _block_dims(x, 1)[:3]
    M = 0 if summaries is None else summaries.shape[0]
    if M:
        if tuple(summaries.shape[1:]) != (B, N, C) or summaries.dtype != x.dtype or not summaries.is_contiguous():
            raise ValueError("summaries must be a contiguous [M, B, N, C] tensor of x's dtype")
    if w.dtype != torch.float32 or tuple(w.shape) != (C,) or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 [C] tensor")
    h = torch.empty_like(x) if h is None else h
    _check(_lib.load().hybrid_attn_attnres_mix(_ptr(summaries) if M else ctypes.c_void_p(None), M, _ptr(x), _ptr(w),
                                               _ptr(h), B, N, C, _dtype_code(x), _stream(stream)),
           "hybrid_attn_attnres_mix")
    return h


def block_routed_workspace_bytes(B: int, H: int, N: int, d: int, dtype=torch.bfloat16) -> int:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().hybrid_attn_block_routed_workspace_bytes(B, H, N, d, code))


def hybrid_attn_block_routed(x, summaries, w_route, W_in4, W_out4, heads, x_out=None, workspace=None, stream=None):
    """hybrid_attn_block with AttnRes routing of `summaries` ([M, B, N, C] or
    None) into the linear sub-layers; w_route float32 [4, C]."""
    B, N, C, d = _block_dims(x, heads)
    _check_weight("W_in4", W_in4, (4, 4 * C, C), x)
    _check_weight("W_out4", W_out4, (4, C, C), x)
    if w_route.dtype != torch.float32 or tuple(w_route.shape) != (4, C) or not w_route.is_contiguous():
        raise ValueError("w_route must be a contiguous float32 [4, C] tensor")
    M = 0 if summaries is None else summaries.shape[0]
    x_out = torch.empty_like(x) if x_out is None else x_out
    need = block_routed_workspace_bytes(B, heads, N, d, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().hybrid_attn_block_routed(_ptr(x), _ptr(summaries) if M else ctypes.c_void_p(None), M,
                                                _ptr(w_route), _ptr(W_in4), _ptr(W_out4), _ptr(x_out), B, heads, N, d,
                                                _dtype_code(x), _ptr(workspace), nbytes, _stream(stream)),
           "hybrid_attn_block_routed")
    return x_out
