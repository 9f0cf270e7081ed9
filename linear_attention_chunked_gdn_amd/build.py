"""Build the gfx950 HIP library (libgdn_mi355x.so) in-tree with hipcc.

    python -m linear_attention_chunked_gdn_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``), one object per source
(compiled in parallel), then linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgdn_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["gdn_api.cpp", "gdn_prefill.hip", "gdn_prefill_pipe.hip", "gdn_decode.hip",
           "kda_map.hip", "kda_chain.hip", "gdn_map.hip", "gdn_seg.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


# Per-source flags.  The chain kernel keeps its MFMA accumulators (the state and v) in
# ordinary VGPRs, where its VALU work on them (conversions, the decay) needs no copies to
# and from the accumulation registers; its prefetched operands take the latter instead.
SOURCE_FLAGS = {"kda_chain.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
# the host pass does not know the packed-fp32 feature and says so; that is harmless
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build_library(out_path: str = LIB_PATH, extra_flags=(), verbose: bool = False) -> str:
    """Compile every source (in parallel) and link one shared library.  Always recompiles."""
    flags = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
    objdir = tempfile.mkdtemp(prefix="gdn_build_")
    try:
        objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
        cmds = [[hipcc(), *flags, *SOURCE_FLAGS.get(s, []), *extra_flags, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out_path + ".tmp"
        _run([hipcc(), *flags, *extra_flags, "-shared", "-o", tmp, *objs], verbose)
        os.replace(tmp, out_path)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return out_path


if __name__ == "__main__":
    print(build_library(verbose=True))
