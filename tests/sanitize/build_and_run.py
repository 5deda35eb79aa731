"""Builds libhad with AddressSanitizer and UndefinedBehaviorSanitizer on its
host-side C++ (argument checks, status codes, dispatch; the device code is
compiled as usual and never runs), links it with abi_validation.cpp and runs
that on the CPU: every call it makes must fail its checks before any GPU
work.  Used by tests/test_host_sanitizers.py.

    python tests/sanitize/build_and_run.py [build dir]
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "sparse_attention_had_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["had_api.hip", "had_pack.hip", "had_attention.hip", "had_decode.hip", "had_backward.hip",
           "had_soft.hip"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)

    def host_obj(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        # each sanitizer flag applies to the host side only
        _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
              "-fPIC", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fsanitize=undefined", f"-I{INCLUDE}", f"-I{CSRC}",
              "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(host_obj, SOURCES))
    drv = os.path.join(out_dir, "abi_validation.o")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          f"-I{INCLUDE}", "-c", os.path.join(HERE, "abi_validation.cpp"), "-o", drv])
    exe = os.path.join(out_dir, "abi_validation")
    _run([CLANGXX, "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    return exe


def run(exe: str) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    env.pop("LD_PRELOAD", None)
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


if __name__ == "__main__":
    d = sys.argv[1] if len(sys.argv) > 1 else tempfile.mkdtemp(prefix="had_san_")
    r = run(build(d))
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    sys.exit(r.returncode)
