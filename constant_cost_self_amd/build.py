"""Build libsata.so (HIP, gfx950) in-tree with hipcc.

    python -m constant_cost_self_amd.build

Compiles every source under csrc/ for --offload-arch=gfx950 into
constant_cost_self_amd/_lib/libsata.so, and the benchmark's ceiling probes
(probe/ceilings.hip) into constant_cost_self_amd/_lib/libsata_ceilings.so.  Packed fp32 VALU instructions are
disabled for all device code.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libsata.so")
PROBE_SRC = os.path.join(HERE, "probe", "ceilings.hip")
PROBE_LIB = os.path.join(LIBDIR, "libsata_ceilings.so")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-result",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = ["hipcc", "-c", "-x", "hip", src, "-o", obj] + FLAGS
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs)
            procs = []
    _wait(procs)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    # the benchmark's ceiling probes: a library of their own, not linked into libsata
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-shared", "-x", "hip", PROBE_SRC, "-o", tmp] + FLAGS
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_LIB)
    return LIB


def _wait(procs):
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((src, text))
        elif text.strip():
            sys.stderr.write(text)
    if failed:
        for src, text in failed:
            sys.stderr.write("==== %s\n%s\n" % (src, text))
        raise RuntimeError("hipcc failed for: " + ", ".join(s for s, _ in failed))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
