"""The no-allocation group (hybrid_attn_group_noalloc, workspace in the
library's fixed device array) against hybrid_attn_group with a caller
workspace: two calls in a row, the second smaller, and both dtypes; the
kernels are the same, so the outputs are bitwise equal."""
import pytest
import torch

import hybrid_linear_softmax_amd as ha
from gpu_util import TOL, rel_err, say
from workloads import to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _group_inputs(B, H, N, d, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    scale = 1.0 if dtype == torch.float32 else d ** -0.5
    x = [torch.randn((4, B, H, N, d), generator=g, device="cuda") * scale for _ in range(3)]
    x.append(torch.randn((4, B, H, N, d), generator=g, device="cuda"))
    return [t.to(dtype) for t in x]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_group_equals_group_twice(dtype):
    for (B, H, N, d, seed) in ((1, 8, 20000, 128, 1), (1, 2, 3001, 64, 2)):
        say(f"noalloc group {dtype} B={B} H={H} N={N} d={d}")
        Q4, K4, V4, G4 = _group_inputs(B, H, N, d, dtype, seed)
        ref = ha.hybrid_attn_group(Q4, K4, V4, G4)
        O4 = torch.full_like(ref, float("nan"))
        out = ha.hybrid_attn_group_noalloc(Q4, K4, V4, G4, O4)
        torch.cuda.synchronize()
        assert out is O4
        assert torch.equal(O4, ref), f"max rel diff {rel_err(to_f64(O4), to_f64(ref)):.3e}"
        # the same call again reuses the array's contents from the call before
        O4b = torch.empty_like(ref)
        ha.hybrid_attn_group_noalloc(Q4, K4, V4, G4, O4b)
        torch.cuda.synchronize()
        assert torch.equal(O4b, ref)
        assert rel_err(to_f64(O4), to_f64(ref)) < TOL["bf16" if dtype == torch.bfloat16 else "f32"]


def test_noalloc_group_rejects_problems_beyond_the_array():
    Q4, K4, V4, G4 = _group_inputs(1, 1, 64, 64, torch.bfloat16, 3)
    need = ha.workspace_bytes(1, 4096, 1000, 128)
    assert need > ha.NOALLOC_SCRATCH_BYTES
    big = torch.empty((4, 1, 4096, 1000, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ha.HybridAttnError, match="workspace"):
        ha.hybrid_attn_group_noalloc(big, big, big, big, big)
