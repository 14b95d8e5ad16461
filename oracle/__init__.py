"""Plain, slow CPU oracle (float64 numpy) for the Hybrid Linear-Softmax
Attention group and the attention block around it.  Test infrastructure only: the test suite, the smoke check and
the bench's CPU-baseline leg use it; the library path never does."""
from .hybrid_ref import (  # noqa: F401
    EPS,
    SCHEDULE,
    SPARSE_BLOCK_Q,
    SPARSE_BLOCK_K,
    allowed_keys,
    softmax_attention_blocksparse,
    phi,
    sigmoid,
    kv_state,
    linear_attention,
    linear_attention_bruteforce,
    softmax_attention,
    layer,
    group,
)
from .block_ref import (  # noqa: F401
    RMS_EPS, attnres_mix, block, block_routed, merge_heads, project_in, project_out, round_bf16,
    split_heads, stack_routed,
)
from .backward_ref import (  # noqa: F401
    layer_backward,
    linear_attention_backward,
    softmax_attention_backward,
    softmax_attention_backward_keys,
    softmax_attention_backward_rows,
    softmax_lse,
)
