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
# the same sources built with RKV_DEBUG: kernels report out-of-range values
DEBUG_LIB = os.path.join(HERE, "librkv_debug.so")
# the same sources built with RKV_WAVE_STAMPS: per-wave timestamps of the
# folded-selection attention launch (rkv_debug_wave_stamps)
STAMPS_LIB = os.path.join(HERE, "librkv_stamps.so")
SOURCES = ["rkv_api.cpp", "reps.hip", "select.hip", "attn.hip", "stage.hip",
           "static_scratch.hip", "stage_copy.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librkv.so)")


def compile_flags(debug: bool = False, stamps: bool = False) -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            *(["-DRKV_DEBUG=1"] if debug else []),
            *(["-DRKV_WAVE_STAMPS=1"] if stamps else []),
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, jobs: int = 4, debug: bool = False,
          stamps: bool = False) -> str:
    """Compile every source to an object, link librkv.so (librkv_debug.so
    with `debug`: RKV_DEBUG bounds reports; librkv_stamps.so with `stamps`:
    per-wave timestamps), return its path."""
    cc = hipcc()
    out_lib = DEBUG_LIB if debug else (STAMPS_LIB if stamps else LIB)
    with tempfile.TemporaryDirectory(prefix="rkv_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [cc] + compile_flags(debug, stamps) + lang + [
                "-c", os.path.join(CSRC, src), "-o", obj]
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
        staged = out_lib + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.replace(staged, out_lib)
    return out_lib


# The host C++ layer (argument checks, workspace sizing, the copy-engine
# staging) built with AddressSanitizer for the CPU ABI tests: the .cpp
# sources by g++ with the sanitizer, the kernel files by hipcc as usual.
ASAN_LIB = os.path.join(HERE, "librkv_asan.so")
HOST_SOURCES = [s for s in SOURCES if s.endswith(".cpp")]


def asan_runtime() -> str:
    """The g++ AddressSanitizer runtime a process must preload to load
    librkv_asan.so."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], check=True,
                          stdout=subprocess.PIPE, text=True).stdout.strip()


def build_asan(verbose: bool = False) -> str:
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    with tempfile.TemporaryDirectory(prefix="rkv_asan_") as tmp:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            if src in HOST_SOURCES:
                cmd = ["g++", "-fsanitize=address", "-fno-omit-frame-pointer", "-g",
                       "-O1", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                       "-I", os.path.join(rocm, "include"), "-I", INCLUDE, "-I", CSRC,
                       "-c", os.path.join(CSRC, src), "-o", obj]
            else:
                cmd = [hipcc()] + compile_flags() + ["-x", "hip", "-c",
                                                     os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
        for item in procs:
            _wait(item)
        tmp_lib = os.path.join(tmp, "librkv_asan.so")
        cmd = (["g++", "-shared", "-fsanitize=address", "-o", tmp_lib] + objs +
               ["-L", os.path.join(rocm, "lib"), "-lamdhip64",
                "-Wl,-rpath," + os.path.join(rocm, "lib")])
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("linking librkv_asan.so failed:\n" + r.stdout)
        shutil.copyfile(tmp_lib, ASAN_LIB + ".tmp")
        os.replace(ASAN_LIB + ".tmp", ASAN_LIB)
    return ASAN_LIB


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
