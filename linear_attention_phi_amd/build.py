"""Build liblaphi.so (the C-ABI HIP library) in-tree for gfx950.

    python -m linear_attention_phi_amd.build

Every HIP source is compiled with hipcc for gfx950 only, with packed-fp32
instructions disabled on the device (-Xclang -target-feature -Xclang
-packed-fp32-ops): the kernels use plain fp32 arithmetic and MFMA only.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblaphi.so")
ARCH = "gfx950"

SOURCES = ["la_api.cpp", "la_control.hip", "la_noalloc.hip", "la_kernels.hip", "la_fused.hip", "la_forward_bf16.hip", "la_forward_f32.hip", "la_window.hip", "la_window_fused.hip", "la_backward.hip"]


def _flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out: str = LIB) -> list[str]:
    """One hipcc line that compiles and links every source (for reference)."""
    return [_hipcc(), *_flags(), "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


# hipcc's host pass does not know the packed-fp32 device feature and says so
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel, under _build/), then
    link liblaphi.so; the library is replaced only once the link succeeds."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        jobs.append(([_hipcc(), *_flags(), "-c", os.path.join(CSRC, src), "-o", obj], obj))
    if verbose:
        for cmd, _ in jobs:
            print(" ".join(cmd), flush=True)
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        errs = list(ex.map(lambda j: _run(j[0]), jobs))
    link = [_hipcc(), f"--offload-arch={ARCH}", "-shared", *[o for _, o in jobs], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    errs.append(_run(link))
    if verbose:
        for e in errs:
            if e.strip():
                print(e, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


# Host sanitizers for the CPU tests: AddressSanitizer and UndefinedBehavior-
# Sanitizer on the host code only (each flag behind -Xarch_host; the device
# code is compiled as usual), against the shared ASan runtime, so that a
# Python process that preloads that runtime can load the library.
SAN_DIR = os.path.join(HERE, "_build", "san")
SAN_LIB = os.path.join(SAN_DIR, "liblaphi_san.so")
_SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libasan"]


def _sources_mtime() -> float:
    files = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "la.h")]
    return max(os.path.getmtime(f) for f in files)


def build_sanitized(verbose: bool = False) -> str:
    """Build the library with host sanitizers into _build/san (reused while it
    is newer than every source); returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    if os.path.exists(SAN_LIB) and os.path.getmtime(SAN_LIB) > _sources_mtime():
        return SAN_LIB
    os.makedirs(SAN_DIR, exist_ok=True)
    flags = [f for f in _flags() if f != "-O3"] + ["-O1", "-g", *_SAN_FLAGS]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        jobs.append(([_hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        errs = list(ex.map(lambda j: _run(j[0]), jobs))
    link = [_hipcc(), f"--offload-arch={ARCH}", "-shared", *_SAN_FLAGS, *[o for _, o in jobs], "-o",
            SAN_LIB + ".tmp"]
    errs.append(_run(link))
    if verbose:
        for e in errs:
            if e.strip():
                print(e, file=sys.stderr)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


def asan_runtime() -> str | None:
    """The shared ASan runtime of the compiler that builds the library."""
    import glob

    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(_hipcc()))),
                                         "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


if __name__ == "__main__":
    print(build(verbose=True))
