"""Build libselscan.so in-tree with hipcc for gfx950.

Usage: ``python -m selective_state_space_48_amd.build`` (or call ``build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libselscan.so")
SOURCES = ["api.hip", "fwd.hip", "step.hip", "conv.hip", "bwd.hip", "ssd.hip"]
# Counter-calibration copies (measurement only), a library of their own.
CALIB_LIB = os.path.join(PKG, "libselscan_calib.so")
CALIB_SOURCES = ["calib.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Keep the compiler from forming packed fp32 instructions (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    noise = ("packed-fp32-ops", "not a recognized feature for this target", "--hip-link")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if ln.strip() and not any(n in ln for n in noise)]
    return res.returncode, msgs


def _compile_link(sources, lib, objdir, verbose):
    inc = ["-I", os.path.join(ROOT, "include")]
    jobs = []
    for src in sources:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append([HIPCC, *FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        results = list(ex.map(_run, jobs))
    for cmd, (rc, msgs) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
    tmp = lib + f".tmp{os.getpid()}"
    objs = [j[-1] for j in jobs]
    rc, msgs = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link libselscan.so and the
    counter-calibration library; returns the path of libselscan.so."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=2) as ex:
        futs = [ex.submit(_compile_link, SOURCES, LIB, objdir, verbose),
                ex.submit(_compile_link, CALIB_SOURCES, CALIB_LIB, objdir, verbose)]
        for f in futs:
            f.result()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
