"""Builds the HIP library ``liblmce.so`` in the package directory (gfx950 only).

    python -m lm_head_chunked_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Every HIP source is built with
packed-FP32 instruction selection switched off.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblmce.so"
SOURCES = ["lmce_api.hip", "lmce_fwd.hip", "lmce_bwd.hip", "lmce_gemm.hip", "lmce_chunked.hip", "lmce_mlp.hip"]
ARCH = "gfx950"


def hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-result",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def lib_path():
    return os.path.join(PKG, LIB_NAME)


def build(verbose: bool = False) -> str:
    """Compiles every source and links liblmce.so; returns its path."""
    out = lib_path()
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(), "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, flush=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
