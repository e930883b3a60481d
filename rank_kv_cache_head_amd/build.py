"""Build liblrattn.so (gfx950) in-tree with hipcc.

    python -m rank_kv_cache_head_amd.build [--verbose]

Compiles every source under csrc/ for gfx950 and links them into
rank_kv_cache_head_amd/liblrattn.so.  Always recompiles.  Packed-fp32 VALU
instructions are disabled in device code (-packed-fp32-ops); hipcc's host pass
prints a harmless "not a recognized feature" warning for that flag.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblrattn.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile and link; returns the path of the built library."""
    cc = hipcc()
    out = os.path.join(PKG, LIB_NAME)
    with tempfile.TemporaryDirectory(prefix="lrattn_build_") as tmp:
        objs = []
        cmds = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([cc, *COMMON, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
        with ThreadPoolExecutor(max(1, len(cmds))) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp_out = os.path.join(tmp, LIB_NAME)
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_out, *objs], verbose)
        shutil.move(tmp_out, out + ".tmp")
        os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
