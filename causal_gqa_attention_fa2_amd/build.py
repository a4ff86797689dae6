"""Build libattn.so (the C-ABI attention library) and libattn_probe.so (the
benchmark's peak-measurement kernels) in-tree for gfx950.

Usage: ``python -m causal_gqa_attention_fa2_amd.build`` or ``build()``.
Each source compiles to an object under ``_build/`` (in parallel), then
hipcc links the shared library next to this file. Compiles every time it is
called.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libattn.so")
# Measurement kernels (measured MFMA and HBM peaks), loaded by the benchmark only.
PROBE_SOURCE = "probe_peaks.hip"
PROBE_LIB_PATH = os.path.join(PKG, "libattn_probe.so")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_cache.hip",
           "attn_norm.hip", "attn_sample.hip", "attn_rope.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Per-source extra flags. The forward kernel never produces or consumes NaN on
# valid input (masked scores are a large negative finite value), so its max
# reductions need no IEEE NaN quieting: one v_max per value instead of two.
EXTRA_FLAGS = {"attn_fwd.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}
ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed fp32 VALU forms are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fp32 atomic adds map to the hardware instruction.
    "-munsafe-fp-atomics",
    "-Wall",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose=False):
    """Compile every HIP/C++ source and link libattn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    probe_obj = _compile(PROBE_SOURCE, verbose)
    tmp = PROBE_LIB_PATH + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", probe_obj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc link failed (probe):\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
