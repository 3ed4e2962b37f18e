"""Build libfa.so (gfx950) in-tree with hipcc.

Usage: python -m exact_tiled_attention_08_amd.build   (or call build()).
Objects go to _build/ at the repository root; the library lands next to this
file so it travels with the source tree.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fwd_bf16.hip", "fwd_fp8.hip", "decode_bf16.hip", "fwd_f32.hip", "bwd_bf16.hip", "ceilings.hip",
           "api.cpp"]
ARCH = "gfx950"

# Packed-FP32 instruction forms are kept out of every kernel.  LDS addresses
# in these kernels are never negative, so constant parts of DS addresses may
# always be folded into the instructions' offset field.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Xclang", "-target-feature", "-Xclang", "+unsafe-ds-offset-folding"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-command-line-argument"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; install ROCm or set HIPCC")


def _compile(src, hipcc, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    noise = ("packed-fp32-ops", "warning: feature flag", "1 warning generated", "warnings generated")
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if not any(n in ln for n in noise)]
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return obj


def build(verbose=False):
    """Compile every source for gfx950 and link libfa.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libfa.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
