"""Build the C-ABI library libkvdecode.so in-tree with hipcc for gfx950.

    python -m kv_cached_decode_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvdecode.so")
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = ["kvd_copy.hip", "kvd_attn.hip", "kvd_attn_mfma.hip", "kvd_verify.hip", "kvd_beam.hip",
           "kvd_probe.hip", "kvd_static.hip", "kvd_prefill.hip",
           "kvd_api.cpp"]
ARCH = "gfx950"
# Per-file code generation options. The matrix-core kernels keep their
# accumulators in ordinary VGPRs (the VGPR form of v_mfma) instead of AGPRs:
# their softmax reads and rescales them every step, and in AGPRs each of
# those accesses costs a v_accvgpr copy (measured: 64 copies per 32-key step
# in the prefill tile, 127 in the 5-row decode tile).
# The streaming and the matrix-core decode kernels take their first 11
# arguments as plain scalars (the values their first key loads need); the
# hardware preloads them into SGPRs at wave start, about 0.25 us before a
# load of them would return.
FILE_FLAGS = {"kvd_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "kvd_attn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
                                    "-mllvm", "-amdgpu-kernarg-preload-count=11"],
              "kvd_attn.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=11"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkvdecode.so")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU forms stay off: hipcc -O3 would otherwise form them
        # from plain float code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # no implicit fma contraction: every fused multiply-add is explicit,
        # so the same expression rounds the same way at every call site
        "-ffp-contract=off",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}: {cmd[-1]}")
    if verbose and res.stderr.strip():
        # the host pass does not know the packed-fp32 feature and says so
        msgs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if msgs:
            sys.stderr.write("\n".join(msgs) + "\n")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source (one hipcc per file, in parallel) and link
    libkvdecode.so; returns its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc, flags = hipcc(), compile_flags()
    objs, cmds = [], []
    for s in SOURCES:
        o = os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o")
        objs.append(o)
        cmds.append([cc, *flags, *FILE_FLAGS.get(s, []), "-c", "-o", o, os.path.join(CSRC, s)])
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
