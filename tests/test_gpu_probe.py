"""The achievable-peak probes (include/ha_probe.h) through the C ABI: the copy
probe reproduces its source bitwise (ordinary and non-temporal accesses, sizes
that leave a tail after the four-deep loop), the read, MFMA (constant and
random operands) and issue-overlap probes complete, and the binding returns
the work each call performs."""
import pytest
import torch

import hybrid_linear_softmax_amd as ha
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 64 << 20])
@pytest.mark.parametrize("nontemporal", [False, True])
def test_copy_probe_is_a_copy(nbytes, nontemporal):
    say(f"copy probe: {nbytes} bytes, nontemporal={nontemporal}")
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    assert ha.probe_copy(src, dst, nontemporal=nontemporal) == 2 * nbytes
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_read_and_mfma_probes_complete():
    say("read and MFMA probes")
    src = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    assert ha.probe_read(src, sink) == 1 << 20
    assert ha.probe_read(src[:48], sink) == 48
    flops = ha.probe_mfma(8, 16, sink)
    assert flops == 8 * 4 * 4 * 16 * 2 * 32 * 32 * 16
    assert ha.probe_mfma_data(8, 16, sink) == flops
    assert ha.probe_mfma_data(8, 17, sink) == 8 * 4 * 4 * 17 * 2 * 32 * 32 * 16   # an odd round count
    torch.cuda.synchronize()
    assert sink.item() == 0.0          # the sinks are written only in cases that cannot occur here


@pytest.mark.parametrize("wps", [1, 2])
@pytest.mark.parametrize("mode", ["mfma", "valu", "both", "split"])
def test_overlap_probe_completes(mode, wps):
    if mode == "split" and wps == 1:
        pytest.skip("the split runs two waves per SIMD")
    say(f"overlap probe: {mode}, {wps} wave(s) per SIMD")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    work = ha.probe_overlap(mode, wps, cus, 64, sink)
    waves = cus * 4 * wps
    per = {"mfma": (waves, 0), "valu": (0, waves), "both": (waves, waves), "split": (waves // 2, waves // 2)}[mode]
    assert work == {"mfma_flops": per[0] * 64 * 4 * 2 * 32 * 32 * 16, "valu_insts": per[1] * 64 * 25}
    torch.cuda.synchronize()
    assert sink.item() == 0.0


def test_probe_binding_checks():
    a = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="same byte size"):
        ha.probe_copy(a, torch.empty(32, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ha.HybridAttnError):
        ha.probe_copy(a[:40], torch.empty(40, dtype=torch.uint8, device="cuda"))   # not a multiple of 16
    with pytest.raises(ha.HybridAttnError):
        ha.probe_mfma(0, 1)
    with pytest.raises(ValueError, match="mode"):
        ha.probe_overlap("fma", 1, 1, 1)
    with pytest.raises(ha.HybridAttnError):
        ha.probe_overlap("split", 1, 1, 1)
