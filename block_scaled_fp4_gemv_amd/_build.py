"""In-tree build of the native libraries.

* ``synth/libsynth.so``  - seeded input generator (gcc, OpenMP).
* ``libmoe_fp4.so``      - the C-ABI library: host code plus HIP kernels for
                           gfx950 (hipcc; one shared object).

Every call recompiles.  HIP sources are built with packed-fp32 instruction
selection disabled (``-packed-fp32-ops``).
"""

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
MOE_LIB = os.path.join(PKG, "libmoe_fp4.so")
SYNTH_LIB = os.path.join(PKG, "synth", "libsynth.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_synth():
    src = os.path.join(PKG, "synth", "synth.c")
    tmp = SYNTH_LIB + ".tmp"
    _run(["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
          src, "-o", tmp, "-lm"])
    os.replace(tmp, SYNTH_LIB)


def host_sources():
    """Plain host C++ (no HIP), built by the host compiler with OpenMP."""
    return sorted(glob.glob(os.path.join(CSRC, "*_host.cpp")))


def hip_sources():
    host = set(host_sources())
    return sorted(s for s in glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp"))
                  if s not in host)


def build_moe(jobs=8):
    srcs = hip_sources()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-result"]
    objs, procs = [], []
    for s in srcs:
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(o)
        cmd = [HIPCC, "-c", "-x", "hip", s, "-o", o] + flags
        print("+", " ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
        if len(procs) >= jobs:
            if procs.pop(0).wait() != 0:
                raise RuntimeError("hipcc failed")
    for p in procs:
        if p.wait() != 0:
            raise RuntimeError("hipcc failed")
    for s in host_sources():
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(o)
        _run(["g++", "-c", s, "-o", o, "-O3", "-mavx2", "-mfma", "-fopenmp", "-fPIC", "-std=c++17", "-I", INCLUDE,
              "-Wall"])
    tmp = MOE_LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + ["-lgomp"])
    os.replace(tmp, MOE_LIB)


def build_all():
    build_synth()
    if hip_sources():
        build_moe()


if __name__ == "__main__":
    build_all()
    sys.exit(0)
