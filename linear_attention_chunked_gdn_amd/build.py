"""Build the gfx950 HIP library (libgdn_mi355x.so) in-tree with hipcc.

    python -m linear_attention_chunked_gdn_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgdn_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["gdn_api.cpp", "gdn_prefill.hip", "gdn_prefill_pipe.hip", "gdn_decode.hip",
           "kda_map.hip", "kda_chain.hip", "gdn_prefill_pipe_prologue.hip", "gdn_map.hip",
           "gdn_seg.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build_library(out_path: str = LIB_PATH, extra_flags=(), verbose: bool = False) -> str:
    """Compile all sources into one shared library.  Always recompiles."""
    flags = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out_path + ".tmp"
    cmd = [hipcc(), *flags, *extra_flags, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build_library(verbose=True))
