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
