"""Build libar.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "lib", "libar.so")
SOURCES = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_add_f32 etc.)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc per file, in parallel) and link
    ar_rmsnorm_amd/lib/libar.so.  Always recompiles."""
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    objdir = os.path.join(os.path.dirname(LIB), "obj")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SOURCES]
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        errs = list(pool.map(lambda so: _run([HIPCC, *compile_flags, "-c", so[0], "-o", so[1]]),
                             zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    errs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]))
    if verbose:
        for e in errs:
            if e.strip():
                print(e)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
