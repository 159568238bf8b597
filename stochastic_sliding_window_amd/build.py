"""Build libssw.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

    python stochastic_sliding_window_amd/build.py

(run as a script: importing the package loads libssw.so, which this script produces)

Produces stochastic_sliding_window_amd/libssw.so.  Every HIP translation unit is compiled with
packed-fp32 instruction selection turned off (plain fp32 VALU code only).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libssw.so")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
SOURCES = ["ssw_api.cpp", "band_attn.hip", "band_attn_bwd.hip", "band_decode.hip", "gate_proj.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libssw.so)")


def build(verbose: bool = False, out_path: str = LIB_PATH, defines=()) -> str:
    """Compile every source and link libssw.so; returns its path.  Always rebuilds.

    ``defines``: extra -D macros (tile-shape knobs of band_attn.hip, for tuning builds written
    to ``out_path``)."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="ssw_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [cc, *HIP_FLAGS, *[f"-D{d}" for d in defines], f"-I{INCLUDE}", *lang, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            _run(cmd, verbose)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libssw.so")
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        shutil.copyfile(tmp_lib, out_path + ".tmp")
        os.replace(out_path + ".tmp", out_path)
    return out_path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag and says so; that is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("-o", default=LIB_PATH)
    ap.add_argument("-D", action="append", default=[])
    a = ap.parse_args()
    print(build(verbose=a.v, out_path=a.o, defines=a.D))
