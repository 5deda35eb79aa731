"""Build libhad.so (gfx950) in-tree with hipcc, plus two measurement builds
of the same sources: libhad_popcount.so, whose attention kernel takes its
logit tiles from XOR + popcount on the vector ALU instead of the int8 matrix
cores, and libhad_fusedq.so, whose had_forward packs only K in a launch of its
own and forms Q's sign words inside the attention launch.  Load either with
HAD_LIBRARY=.../libhad_<name>.so.

Usage: python -m sparse_attention_had_amd.build   (or __graft_entry__.build())
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhad.so")
LIB_POPCOUNT = os.path.join(PKG, "libhad_popcount.so")
LIB_FUSEDQ = os.path.join(PKG, "libhad_fusedq.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["had_api.hip", "had_pack.hip", "had_attention.hip", "had_decode.hip", "had_backward.hip",
           "had_soft.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core operands and accumulators in arch VGPRs (no AGPR copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _compile(job) -> str:
    src, tag, defs = job
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950, link libhad.so and libhad_popcount.so;
    returns the path of libhad.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = [(src, "", []) for src in SOURCES]
    jobs.append(("had_attention.hip", "_popcount", ["-DHAD_LOGITS_POPCOUNT=1"]))
    jobs.append(("had_attention.hip", "_fusedq", ["-DHAD_FUSED_QPACK=1"]))
    jobs.append(("had_api.hip", "_fusedq", ["-DHAD_FUSED_QPACK=1"]))
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(_compile, jobs))
    main_objs = objs[:len(SOURCES)]
    _link(main_objs, LIB)
    variant = dict(zip([(j[0], j[1]) for j in jobs], objs))
    pop_objs = [variant.get((src, "_popcount"), o) for src, o in zip(SOURCES, main_objs)]
    _link(pop_objs, LIB_POPCOUNT)
    fq_objs = [variant.get((src, "_fusedq"), o) for src, o in zip(SOURCES, main_objs)]
    _link(fq_objs, LIB_FUSEDQ)
    if verbose:
        print(f"built {LIB}, {LIB_POPCOUNT} and {LIB_FUSEDQ}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
