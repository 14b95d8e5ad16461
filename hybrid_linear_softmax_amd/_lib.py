"""ctypes declaration of libhybrid_attn.so (the C ABI in include/hybrid_attn.h and
the measurement probes in include/ha_probe.h).

Loading is lazy so that the package can be imported to build the library; any
call into the library raises if it has not been built.  There is no fallback
implementation.
"""
import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# HA_LIBRARY names another build of the same library (the host-sanitized test
# build); by default the in-tree library is loaded.
LIB_PATH = os.environ.get("HA_LIBRARY") or os.path.join(PKG, "libhybrid_attn.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HEADER = os.path.join(INCLUDE, "hybrid_attn.h")

HA_BF16, HA_F32 = 0, 1
HA_OK, HA_EINVAL, HA_EUNSUPPORTED, HA_EALIGN, HA_EWORKSPACE, HA_EHIP = 0, -1, -2, -3, -4, -5

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

SIGNATURES = {
    "hybrid_attn_strerror": (ctypes.c_char_p, [_i]),
    "hybrid_attn_workspace_bytes": (_sz, [_i, _i, _i64, _i, _i]),
    "hybrid_attn_kv_state": (_i, [_p, _p, _p, _p, _i, _i, _i64, _i, _i, _p, _sz, _p]),
    "hybrid_attn_linear": (_i, [_p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p, _sz, _p]),
    "hybrid_attn_linear_timed": (_i, [_p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p, _sz, _p,
                                      ctypes.POINTER(_p)]),
    "hybrid_attn_softmax": (_i, [_p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p]),
    "hybrid_attn_softmax_blocksparse": (_i, [_p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p, _p, _i64, _p]),
    "hybrid_attn_group": (_i, [_p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p, _sz, _p]),
    "hybrid_attn_group_timed": (_i, [_p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p, _sz, _p,
                                     ctypes.POINTER(_p)]),
    "hybrid_attn_group_schedule": (_i, [ctypes.POINTER(_i)]),
    "hybrid_attn_group_noalloc": (_i, [_p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p]),
    "hybrid_attn_linear_backward_workspace_bytes": (_sz, [_i, _i, _i64, _i, _i]),
    "hybrid_attn_linear_backward": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p, _sz, _p]),
    "hybrid_attn_softmax_lse": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p]),
    "hybrid_attn_softmax_backward_workspace_bytes": (_sz, [_i, _i, _i64, _i, _i]),
    "hybrid_attn_softmax_backward": (_i, [_p] * 11 + [_i, _i, _i64, _i, _i, _p, _sz, _p]),
    "hybrid_attn_attnres_mix": (_i, [_p, _i, _p, _p, _p, _i, _i64, _i, _i, _p]),
    "hybrid_attn_block_routed_workspace_bytes": (_sz, [_i, _i, _i64, _i, _i]),
    "hybrid_attn_block_routed": (_i, [_p, _p, _i, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p, _sz, _p]),
    "hybrid_attn_proj_in": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _p]),
    "hybrid_attn_proj_out": (_i, [_p, _p, _p, _p, _i, _i, _i64, _i, _i, _p]),
    "hybrid_attn_block_workspace_bytes": (_sz, [_i, _i, _i64, _i, _i]),
    "hybrid_attn_block": (_i, [_p, _p, _p, _p, _i, _i, _i64, _i, _i, _p, _sz, _p]),
    "hybrid_attn_probe_mfma_flops": (ctypes.c_double, [_i, _i]),
    "hybrid_attn_probe_mfma": (_i, [_i, _i, _p, _p]),
    "hybrid_attn_probe_mfma_data": (_i, [_i, _i, _p, _p]),
    "hybrid_attn_probe_read": (_i, [_p, _sz, _p, _p]),
    "hybrid_attn_probe_copy": (_i, [_p, _p, _sz, _i, _p]),
    "hybrid_attn_probe_overlap": (_i, [_i, _i, _i, _i, _p, _p]),
}

_lib = None


def load() -> ctypes.CDLL:
    """The loaded library, with argument and result types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                "(hipcc for gfx950).  The HIP library is the only implementation.")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions(paths=None) -> list:
    """Names of the functions the headers under include/ declare (HA_API ...)."""
    if paths is None:
        paths = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))
    names = []
    for path in paths:
        with open(path) as f:
            names += re.findall(r"HA_API\s+[\w\s\*]+?\b(hybrid_attn_\w+)\s*\(", f.read())
    return names
