"""Build librq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m rotation_w4a4_quantization_amd.build`` or ``build()``.
The library is written next to this file so that it travels with the source
tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "librq.so")
# every HIP source of the library (csrc/*.hip), in a fixed order
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    # packed fp32 VALU forms stay out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Extra flags per source.  The attention kernel keeps its MFMA accumulators
# in VGPRs (its loop also scales them with VALU instructions; in AGPRs the
# compiler copies them back and forth every iteration).
FILE_FLAGS = {"decode_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link librq.so."""
    objdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)
    noise = "is not a recognized feature for this target"
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f != "-shared"], *FILE_FLAGS.get(src, []),
               "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.PIPE, text=True)))
    objs = []
    for src, obj, pr in procs:
        _, err = pr.communicate()
        err = "\n".join(l for l in err.splitlines() if noise not in l)
        if pr.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src} ({pr.returncode}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
