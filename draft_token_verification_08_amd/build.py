"""Build libspecverify.so in-tree with hipcc for gfx950.

    python -m draft_token_verification_08_amd.build

Compiles the HIP kernels and the host ABI layer into one shared object next to
this file.  Flags: -O3, no floating-point contraction (the draw pass recomputes
the same weights twice and relies on bitwise-equal results), and packed-FP32
instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libspecverify.so")
ARCH = os.environ.get("SV_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return out


def build(out: str = LIB, verbose: bool = False, defines=(), objdir: str | None = None) -> str:
    """Compile and link; `defines` are extra -D tuning flags (e.g. SV_ARGMAX_UNROLL=16)."""
    objdir = objdir or os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    k_obj = os.path.join(objdir, "sv_kernels.o")
    l_obj = os.path.join(objdir, "sv_lmhead.o")
    a_obj = os.path.join(objdir, "sv_api.o")
    n_obj = os.path.join(objdir, "sv_noalloc.o")
    logs = []
    dflags = [f"-D{d}" for d in defines]
    logs.append(_run([HIPCC, f"--offload-arch={ARCH}", *COMMON, *dflags, "-x", "hip", "-c",
                      os.path.join(CSRC, "sv_kernels.hip"), "-o", k_obj]))
    logs.append(_run([HIPCC, f"--offload-arch={ARCH}", *COMMON, *dflags, "-x", "hip", "-c",
                      os.path.join(CSRC, "sv_lmhead.hip"), "-o", l_obj]))
    logs.append(_run([HIPCC, *COMMON, *dflags, "-c", os.path.join(CSRC, "sv_api.cpp"), "-o", a_obj]))
    logs.append(_run([HIPCC, f"--offload-arch={ARCH}", *COMMON, *dflags, "-x", "hip", "-c",
                      os.path.join(CSRC, "sv_noalloc.hip"), "-o", n_obj]))
    tmp = out + ".tmp"
    logs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", k_obj, l_obj, a_obj, n_obj, "-o", tmp]))
    os.replace(tmp, out)
    if verbose:
        print("\n".join(l for l in logs if l))
    return out


if __name__ == "__main__":
    print(build(verbose=True))
