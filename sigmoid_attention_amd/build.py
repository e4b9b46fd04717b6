"""Build libsigattn.so in-tree with hipcc for gfx950.

    python -m sigmoid_attention_amd.build        # or __graft_entry__.build()

Compiles every source on each call (a few tens of seconds), in parallel, and
links ``sigmoid_attention_amd/libsigattn.so``.  All HIP code is compiled with
packed-FP32 instructions disabled (``-Xclang -target-feature -Xclang
-packed-fp32-ops``); hipcc's host pass warns that it does not know that
feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsigattn.so")
ARCH = "gfx950"

# (source, extra flags): the kernels are compiled once per element type.
HIP_SOURCES = [("kernels.hip", []), ("kernels.hip", ["-DSIGATTN_FP16"]), ("probe.hip", [])]
CXX_SOURCES = ["api.cpp", "plan.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsigattn")


def rocm_include() -> str:
    root = os.environ.get("ROCM_PATH") or os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    return os.path.join(root, "include")


COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
# The AMDGPU register-pressure trackers in the machine scheduler: the head-dim
# 128 backward kernels, at the register limit, spill 8 bytes instead of 24
# and run 2 % faster (same-session A/B on MI355X); the others are unchanged.
DEVICE = [f"--offload-arch={ARCH}", "-mllvm", "--amdgpu-use-amdgpu-trackers",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="sigattn_build_")
    try:
        jobs = []
        objs = []
        for i, (src, flags) in enumerate(HIP_SOURCES):
            obj = os.path.join(tmp, f"{src}.{i}.o")
            jobs.append([cc, *COMMON, *DEVICE, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        for src in CXX_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            jobs.append([cc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{rocm_include()}",
                         "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            list(ex.map(lambda c: _run(c, verbose), jobs))
        out_tmp = LIB + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp], verbose)
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
