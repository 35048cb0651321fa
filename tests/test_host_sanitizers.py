"""The C ABI's validation layer under host AddressSanitizer and UndefinedBehaviorSanitizer.

A host-sanitized copy of the library (device code built as usual, every -fsanitize=
applied to the host side only) is built into a temporary directory, and the host-side
ABI tests (tests/test_abi.py: argument validation, aliasing, workspace queries, exported
symbols, the binding's own checks) run against it in a child process with the
sanitizer runtime preloaded; any report aborts that process.  No GPU is needed: every
call there fails validation or only queries sizes, so nothing is launched.
"""
import os
import shutil
import subprocess
import sys

import pytest

from retnet_retention_fwd_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the library")
def test_validation_layer_under_host_sanitizers(tmp_path):
    rt = B.sanitizer_runtime()
    if not rt:
        pytest.skip("no shared AddressSanitizer runtime next to the ROCm clang")
    lib = B.build(verbose=False, sanitize=True, out_dir=str(tmp_path))
    code = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import retnet_retention_fwd_amd._lib as L\n"
        f"L.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        "rc = pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py'])\n"
        "assert L.lib()._name == L.LIB_PATH\n"
        "sys.exit(int(rc))\n"
    )
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "passed" in r.stdout
