"""Build libmoe.so in-tree with hipcc for gfx950 (CDNA4).

    python -m sparse_moe_routed_amd.build      # or __graft_entry__.build()

Every HIP source under csrc/ is compiled to an object in parallel, then the
objects are linked into sparse_moe_routed_amd/libmoe.so.  The build always
recompiles (it is the "does it build" check).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-ffp-contract=off",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True, out: str = OUT, defines=()) -> str:
    objdir = OBJDIR if out == OUT else os.path.join(ROOT, "_build", "obj_" + os.path.basename(out))
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    extra = [f"-D{d}" for d in defines]
    with ThreadPoolExecutor(max(1, min(8, len(srcs)))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, objdir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    build()
