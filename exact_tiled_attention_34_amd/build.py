"""Build libfa2.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m exact_tiled_attention_34_amd.build`` (or ``build()``).
The library is written next to this file; objects go to ``_build/``.
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
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libfa2.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["fa2_api.hip", "fa2_fwd.hip", "fa2_bwd.hip", "fa2_bwd_dq256.hip"]
# Kernels that run one wavefront per SIMD may use all 512 registers of a lane,
# and for those the compiler otherwise writes every MFMA result to the
# accumulator registers: the S and dP products (and the forward's scores at
# head dim 256) were then copied to vector registers on every step for the
# softmax.  With MFMA results in vector registers they are read in place
# (dK/dV on MI355X: B4 H32 N4096 d64 causal -11 %, B2 H32 N8192 d80 causal
# -6.5 %; head dim 256 forward -8 %).  Kernels with two or more wavefronts per
# SIMD compile to the same code either way.  The head-dim-256 dQ kernel, whose
# accumulators are only ever MFMA operands, measured 21 % slower with it and
# keeps the default (its own unit).
SOURCE_FLAGS = {
    "fa2_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fa2_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 VALU forms stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libfa2.so)")
    return exe


def _compile(src, extra):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; that note is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=False, extra_flags=()):
    """Compile every HIP source for gfx950 and link libfa2.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    for _, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
