"""Builds the HIP libraries in-tree with hipcc for gfx950.

    python -m long_context_memory_chunk_amd.build

produces long_context_memory_chunk_amd/libmsa.so (the MSA C ABI declared in
include/msa.h) and msa_synth/libmsasynth.so (the synthetic-input fill
kernel).  Every source is compiled each time this runs.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmsa.so")
SYNTH_SRC = os.path.join(ROOT, "msa_synth", "fill.hip")
SYNTH_LIB = os.path.join(ROOT, "msa_synth", "libmsasynth.so")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the MSA library needs ROCm's hipcc")
    return exe


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(verbose=False, jobs=8):
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = []
    cmds = []
    for f in srcs:
        obj = os.path.join(BUILD, f[:-4] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
                     os.path.join(CSRC, f), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, *FLAGS, "-shared", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    _run([hipcc, *FLAGS, "-shared", SYNTH_SRC, "-o", tmp])
    os.replace(tmp, SYNTH_LIB)
    return LIB, SYNTH_LIB


if __name__ == "__main__":
    for p in build(verbose="-v" in sys.argv):
        print("built", p)
