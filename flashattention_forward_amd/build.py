"""Build libfa.so (gfx950 kernels + C-ABI front end) in-tree with hipcc.

Usage: ``python flashattention_forward_amd/build.py`` (or ``build()`` of this file
loaded by path: importing the package itself loads the library, which a build
must not need). Every call recompiles; objects go to ``_build/`` next to this
file.

Two libraries come out of the same sources:
  libfa.so           the library;
  libfa_ldsdebug.so  the LDS-race debug build (-DFA_LDS_DEBUG=1): every LDS
                     hand-off waits for all outstanding memory operations and
                     the shared-stage loops add a barrier per step. Same
                     arithmetic, so the tests require bit-identical results.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
LIB_LDSDEBUG = os.path.join(PKG, "libfa_ldsdebug.so")
VARIANTS = {"fast": (LIB, []), "ldsdebug": (LIB_LDSDEBUG, ["-DFA_LDS_DEBUG=1"])}

SOURCES = ["prefill.hip", "prefill_f16.hip", "prefill_d64.hip", "prefill_pp.hip", "decode.hip",
           "decode_mla.hip", "combine.hip", "noalloc.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# No fast-math: -inf scores and exp2(-inf) = 0 must stay IEEE. Packed fp32 VALU
# forms are switched off for all device code. MFMA accumulators stay in
# ordinary VGPRs (-amdgpu-mfma-vgpr-form): left to its heuristics the compiler
# put the paged GQA decode's accumulators in AGPRs and copied all of them to
# VGPRs and back on every tile (about 70 extra instructions per tile); the
# other kernels already get the VGPR form.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(job) -> str:
    variant, src = job
    out_dir = os.path.join(BUILD, variant)
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + VARIANTS[variant][1] + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} ({variant}):\n{r.stderr}")
    return obj


def _link(variant: str, objs) -> str:
    lib = VARIANTS[variant][0]
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + list(objs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({variant}):\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, variants=("fast", "ldsdebug")) -> str:
    """Compile and link the requested variants; returns the path of libfa.so."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    for v in variants:
        os.makedirs(os.path.join(BUILD, v), exist_ok=True)
    jobs = [(v, s) for v in variants for s in SOURCES]
    # The head-size-128 prefill sources are the long poles: start them first.
    jobs.sort(key=lambda j: not j[1].startswith("prefill"))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, jobs))
    for v in variants:
        lib = _link(v, [o for (vj, _), o in zip(jobs, objs) if vj == v])
        if verbose:
            print(f"built {lib}")
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
