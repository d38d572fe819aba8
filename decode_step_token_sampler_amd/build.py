"""Build the HIP library of the decode-step sampler for gfx950, in-tree.

``build()`` always recompiles (it is the "does it build" check); loaders call
``ensure_built()``, which compiles only when the library is missing or older
than its sources.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdsts_sampler.so")
# the same library with the row kernel's phase stamps compiled in (for
# performance work only; the stamps' stores perturb the timings a little)
LIB_STAMPS = os.path.join(PKG, "libdsts_sampler_stamps.so")
SOURCES = [os.path.join(CSRC, "sampler_kernel.hip"), os.path.join(CSRC, "sampler_runtime.cpp")]
HEADERS = [os.path.join(CSRC, "sampler_internal.h"), os.path.join(INCLUDE, "sampler.h")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -ffp-contract=off: each fp32 step of the penalties and the temperature
# division is rounded on its own.  The packed-fp32 feature is disabled for
# the device code (its host-pass warning is harmless).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE]


def build(verbose: bool = False, stamps: bool = False) -> str:
    lib = LIB_STAMPS if stamps else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *(["-DDSTS_PHASE_STAMPS"] if stamps else []), *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, lib)
    return lib


def ensure_built() -> str:
    newest = max(os.path.getmtime(p) for p in SOURCES + HEADERS)
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < newest:
        build()
    return LIB


if __name__ == "__main__":
    import sys
    print(build(verbose=True, stamps="--stamps" in sys.argv[1:]))
