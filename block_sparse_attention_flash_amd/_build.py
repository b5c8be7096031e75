"""Build libblasst.so in-tree with hipcc for gfx950.

Each source compiles to its own object (in parallel), then one shared library is
linked next to this file.  Every HIP compile carries
``-Xclang -target-feature -Xclang -packed-fp32-ops`` (packed-FP32 instructions
off).  hipcc's host pass warns that it does not know that feature; the warning
is harmless and filtered from the log.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libblasst.so")
SOURCES = ["api.cpp", "decode.hip", "prefill.hip", "mla.hip"]
ARCH = os.environ.get("BLASST_OFFLOAD_ARCH", "gfx950")

HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    log = "\n".join(line for line in p.stdout.splitlines() if "packed-fp32-ops" not in line)
    if p.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), log))
    return log


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmds.append([HIPCC] + COMMON + DEVICE + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(cmds)) as ex:
        logs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp%d" % os.getpid()
    logs.append(_run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs))
    os.replace(tmp, LIB)
    if verbose:
        for log in logs:
            if log.strip():
                print(log, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
