"""Build librkv.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every call compiles from source.  The result lands next to this file; the
Python binding loads it from there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librkv.so")
SOURCES = ["rkv_api.cpp", "reps.hip", "select.hip", "attn.hip", "stage.hip",
           "static_scratch.hip", "stage_copy.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librkv.so)")


def compile_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object, link librkv.so, return its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="rkv_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [cc] + compile_flags() + lang + ["-c", os.path.join(CSRC, src),
                                                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT,
                                                text=True)))
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        while procs:
            _wait(procs.pop(0))
        tmp_lib = os.path.join(tmp, "librkv.so")
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                           text=True)
        if r.returncode != 0:
            raise RuntimeError("linking librkv.so failed:\n" + r.stdout)
        staged = LIB + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.replace(staged, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    noisy = [ln for ln in out.splitlines()
             if "packed-fp32-ops" not in ln and ln.strip()]
    if noisy:
        print(f"[{src}]\n" + "\n".join(noisy), flush=True)


if __name__ == "__main__":
    print(build(verbose=True))
