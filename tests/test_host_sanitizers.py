"""CPU: the library's host-side C++ under AddressSanitizer and
UndefinedBehaviorSanitizer.  tests/sanitize/build_and_run.py compiles libhad
with both sanitizers on the host side (the device code is compiled as usual
and never runs) and links abi_validation.cpp, which calls every entry point
with arguments its checks must reject (null and misaligned pointers, bad
sizes, out-of-range enum values, small workspaces, shapes past the limits)
and checks the status and error text.  Any sanitizer report fails the run.
"""

import os
import shutil
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("ld.lld") is None
                    and not os.path.exists("/opt/rocm/llvm/bin/ld.lld"), reason="needs the ROCm toolchain")
def test_abi_validation_under_address_and_undefined_behavior_sanitizers(tmp_path):
    import build_and_run

    r = build_and_run.run(build_and_run.build(str(tmp_path)))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks held" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
