"""The C-ABI tests again, against a host-side AddressSanitizer +
UndefinedBehaviorSanitizer build of the library (argument validation and the
launchers' host code; device code is unsanitized).  CPU only: every call in
test_abi.py returns before any kernel is launched."""
import os
import subprocess
import sys

import pytest

from hybrid_linear_softmax_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")),
                    reason="the process already preloads a library; the sanitizer runtime is not layered over it")
def test_abi_under_address_and_undefined_behaviour_sanitizers():
    lib = _build.build_host_sanitized(os.path.join(ROOT, "_build", "asan"))
    env = dict(os.environ,
               LD_PRELOAD=_build.asan_runtime(),
               # the interpreter and the HIP runtime keep allocations to exit;
               # errors abort with a report on stderr
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HA_LIBRARY=lib)
    # -s: a sanitizer report is written straight to stderr before the abort
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    assert " passed" in r.stdout
