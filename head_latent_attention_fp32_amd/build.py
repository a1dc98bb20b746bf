"""Build libmla.so (the HIP kernels and their C ABI) for gfx950 with hipcc, in the package folder.

    python -m head_latent_attention_fp32_amd.build [--verbose]

Every call recompiles. Objects are built in parallel, then linked into one shared library.
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
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla.so")
SOURCES = ["mla_api.cpp", "query_path.hip", "decode.hip", "prefill.hip", "kv_side.hip", "out_proj.hip"]
# The benchmark's in-process rate probes (stream read, MFMA loop): a library of their own, outside
# libmla's ABI.
PEAKS_LIB = os.path.join(PKG, "libmla_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# The attention kernels take row maxima of scores that are finite or -inf (masked), never NaN:
# without NaN semantics each fmaxf is one v_max instead of two operand-quieting v_max plus the max.
PER_FILE = {"decode.hip": ["-fno-honor-nans"], "prefill.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmla")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = {LIB: [], PEAKS_LIB: []}
    jobs = []
    for lib, sources in ((LIB, SOURCES), (PEAKS_LIB, PEAKS_SOURCES)):
        for s in sources:
            o = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
            objs[lib].append(o)
            lang = ["-x", "hip"] if s.endswith(".cpp") else []
            jobs.append([cc] + COMMON + PER_FILE.get(s, []) + lang + ["-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    for lib, o in objs.items():
        tmp = lib + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + o, verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
